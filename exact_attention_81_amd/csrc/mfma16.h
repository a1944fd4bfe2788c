// 16-bit (bf16 / fp16) MFMA operands, transposing LDS reads and the LDS swizzles
// shared by the gfx950 attention kernels that stream K/V tiles through LDS.
#pragma once

#include "device.h"
#include "tile_io.h"

namespace exattn {

template <bool F16> struct Elem;
template <> struct Elem<false> {
  static __device__ inline unsigned pack2(float a, float b) {
    bf16x2_t r = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);  // v_cvt_pk_bf16_f32, RNE
    return __builtin_bit_cast(unsigned, r);
  }
  static __device__ inline f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Elem<true> {
  static __device__ inline unsigned pack2(float a, float b) {
    f16x2_t r = __builtin_convertvector((f32x2_t){a, b}, f16x2_t);  // RNE
    return __builtin_bit_cast(unsigned, r);
  }
  static __device__ inline f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};

// Transposing read: within each group of 16 lanes, lane i receives element i%4
// of the 8 bytes read by lanes 4t + i/4, t = 0..3 (a 4 x 16 block of 16-bit
// values, returned column-wise).
__device__ inline u32x2_t lds_read_tr16(const lds_u8* p) {
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p);
  return __builtin_bit_cast(u32x2_t, v);
}

// Swizzled chunk position inside an LDS row of 16 chunks (256 B) or 8 chunks
// (128 B). `w16` selects the row width.
//   K rows, 16 chunks: chunk c of row r at c ^ (r & 15).
//   K rows,  8 chunks: chunk c of row r at c ^ ((r >> 1) & 7).
//   V rows, 16 chunks: chunk c of row r at c ^ (4 * (r & 3)).
//   V rows,  8 chunks: chunk c of row r at c ^ (4 * ((r >> 1) & 1)).
__device__ constexpr int k_swz(int c, int r, bool w16) { return w16 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7)); }
__device__ constexpr int v_swz(int c, int r, bool w16) { return w16 ? (c ^ (4 * (r & 3))) : (c ^ (4 * ((r >> 1) & 1))); }

}  // namespace exattn
