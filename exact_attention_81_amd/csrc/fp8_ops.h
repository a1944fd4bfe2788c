// e4m3 helpers shared by the gfx950 fp8 attention kernels.
#pragma once

#include "device.h"

namespace exattn {

// e4m3 x e4m3 -> f32, 32x32 output, K = 64. Operand lane l: row/column l % 32,
// bytes k = 32 (l / 32) + 0..31.
__device__ inline f32x16_t mfma_f8(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ inline i32x8_t join8(u32x4_t lo, u32x4_t hi) {
  return (i32x8_t){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Four e4m3 codes (RNE) in one dword, a in the lowest byte. Inputs are finite
// and at most 256 in magnitude. The first convert writes the low half and keeps the
// high half of its "old" operand, which the second overwrites: passing a's own bits
// there (a dies here) lets the destination take a's register, where a constant 0
// costs a v_mov per dword (16 per tile and wave in the fp8 attention, 2.5 % of its
// time).
__device__ inline unsigned pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (unsigned)w;
}

}  // namespace exattn
