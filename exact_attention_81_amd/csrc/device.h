// Vector types and wave-level helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace exattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

}  // namespace exattn

namespace exattn {

constexpr int kNumXcd = 8;  // MI355X: 256 CUs in 8 accelerator complex dies

// Maps the hardware workgroup index to (b*H + h, query tile).
//
// The dispatcher deals consecutive workgroups to the 8 XCDs round-robin. The
// remap hands each XCD a contiguous range of heads, so the K/V tiles of a head
// are re-read from that XCD's own L2 by all of its query tiles. For causal
// problems the query tiles with the most visible keys are issued first
// (longest job first), which evens out the tail of the grid.
__device__ inline void map_block(int bid, int n_qtiles, int BH, bool causal, int& bh, int& qt) {
  if (BH % kNumXcd == 0) {
    const int xcd = bid % kNumXcd;
    const int local = bid / kNumXcd;
    const int heads_per = BH / kNumXcd;
    if (causal) {
      qt = n_qtiles - 1 - local / heads_per;
      bh = xcd * heads_per + local % heads_per;
    } else {
      bh = xcd * heads_per + local / n_qtiles;
      qt = local % n_qtiles;
    }
  } else if (causal) {
    qt = n_qtiles - 1 - bid / BH;
    bh = bid % BH;
  } else {
    bh = bid / n_qtiles;
    qt = bid % n_qtiles;
  }
}

// max(x, x of lane ^ 32) in every lane of a wave64.
//
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second, so with both operands equal to x the partner's
// value lands in r[1] for lanes 0-31 and in r[0] for lanes 32-63; the max over
// x, r[0] and r[1] is the same in every lane either way.
__device__ inline float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// x + x of lane ^ 32 in every lane of a wave64. After v_permlane32_swap with both
// operands equal to x, one of r[0], r[1] holds the lane's own x and the other its
// partner's (which one depends on the lane half), so their sum is the pair's sum,
// bitwise the same in both halves since float addition commutes. Unlike a shuffle it
// needs no lane-index register.
__device__ inline float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace exattn
