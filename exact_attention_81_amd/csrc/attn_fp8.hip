// fp8 (OCP e4m3) path for gfx950: per-block quantisation with an optional
// random-sign Hadamard rotation (the attention kernel is in attn_fwd_fp8.hip).
//
// "FlashAttention 3 and 4: When the Bottleneck Moves", section 2.2: the
// tensor cores run FP8 at about twice the 16-bit rate; each block of values
// gets its own scale; Q and K are multiplied by one fixed random rotation
// before quantising, which leaves Q K^T unchanged because R R^T = I.
#include <math.h>

#include "device.h"

namespace exattn {
namespace {

constexpr int QBLOCK = 128;  // tokens per scale block
constexpr int QD = 128;      // head dim of the fp8 path
constexpr int QTHREADS = 256;

// One workgroup per (b*H + h, 128-token block); two threads per token row,
// each producing 64 of the row's 128 outputs.
//
// Rotation: y = x diag(signs) H_128 by the fast Walsh-Hadamard transform in
// float64. Every butterfly adds or subtracts partial sums of +-bfloat16
// values, which float64 holds exactly, so y does not depend on the order of
// the stages. The first stage (index bit 6) pairs the two halves of the row;
// each thread reads the whole row and keeps its half of that stage's output,
// then runs the stages for bits 0-5 on its own 64 values. Without rotation a
// thread reads only its half. The column signs are applied as sign-bit flips
// of the bf16 inputs (negation is exact).
// Scale: amax = max |y| over the block, ratio = 448 / amax in float64,
// code = e4m3(float32(y * ratio)) with round-to-nearest-even; the stored
// descale is float32(amax / div), div = 448 * sqrt(128) (rotated) or 448.
// Three waves per SIMD (168 VGPRs, no spills; four would spill the 64 float64 values)
// keep three workgroups' loads in flight per compute unit.
__global__ __launch_bounds__(QTHREADS) __attribute__((amdgpu_waves_per_eu(3, 3))) void quantize_kernel(const uint16_t* __restrict__ x,
                                                           uint8_t* __restrict__ x8,
                                                           float* __restrict__ descale, int N,
                                                           int nb, const float* __restrict__ signs,
                                                           int transpose, double div) {
  __shared__ double red[QTHREADS / 64];
  __shared__ __attribute__((aligned(16))) uint8_t tile[QBLOCK][QD + 16];

  const int blk = blockIdx.x % nb;
  const int bh = blockIdx.x / nb;
  const int tid = threadIdx.x;
  const int row = tid >> 1;
  const int h = tid & 1;
  const int token = blk * QBLOCK + row;
  const bool valid = token < N;

  // Column signs of the rotation as a 128-bit mask in scalar registers (bit c set:
  // column c is negated), built by two ballots per wave; zero without rotation.
  const bool rot = signs != nullptr;
  unsigned long long neg_lo = 0ull, neg_hi = 0ull;
  if (rot) {
    const int lane = tid & 63;
    neg_lo = __ballot(signs[lane] < 0.f);
    neg_hi = __ballot(signs[lane + 64] < 0.f);
  }
  // XOR pattern that negates the bf16 pair of columns (col, col + 1) of one 32-bit word.
  auto pair_flip = [](unsigned long long mask, int col) {
    const unsigned f = (unsigned)(mask >> col) & 3u;
    return ((f & 1u) << 15) | ((f >> 1) << 31);
  };
  auto lo_f = [](unsigned w) { return __uint_as_float(w << 16); };
  auto hi_f = [](unsigned w) { return __uint_as_float(w & 0xffff0000u); };

  double y[64];
  {
    const uint16_t* src = x + ((size_t)bh * N + token) * QD;
    if (rot) {
      // Chunk c holds columns 8c..8c+7 (a) and the partner columns + 64 (b); the first
      // stage gives a + b (h = 0) or a - b (h = 1), the latter as a + (-b): negating b
      // is one more sign-bit flip, folded into b's pattern.
      const unsigned h_flip = h ? 0x80008000u : 0u;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x4_t lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
        if (valid) {
          lo = *(const u32x4_t*)(src + c * 8);
          hi = *(const u32x4_t*)(src + 64 + c * 8);
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int col = c * 8 + 2 * w;
          const unsigned wl = lo[w] ^ pair_flip(neg_lo, col);
          const unsigned wh = hi[w] ^ pair_flip(neg_hi, col) ^ h_flip;
          y[col] = (double)lo_f(wl) + (double)lo_f(wh);
          y[col + 1] = (double)hi_f(wl) + (double)hi_f(wh);
        }
      }
#pragma unroll
      for (int len = 1; len < 64; len <<= 1)
#pragma unroll
        for (int i = 0; i < 64; ++i)
          if ((i & len) == 0) {
            const double a = y[i], b = y[i + len];
            y[i] = a + b;
            y[i + len] = a - b;
          }
    } else {
      // No rotation: thread h takes columns 64h .. 64h + 63 of its row.
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (valid) v = *(const u32x4_t*)(src + 64 * h + c * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          y[c * 8 + 2 * w] = (double)lo_f(v[w]);
          y[c * 8 + 2 * w + 1] = (double)hi_f(v[w]);
        }
      }
    }
  }

  // Block amax: lane, wave, workgroup.
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmax(amax, fabs(y[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmax(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  const double ratio = amax > 0.0 ? 448.0 / amax : 0.0;

  unsigned packed[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = fminf(fmaxf((float)(y[4 * i + t] * ratio), -448.f), 448.f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
    packed[i] = (unsigned)w;
  }

  if (!transpose) {
    if (valid) {
      uint8_t* dst = x8 + ((size_t)bh * N + token) * QD + 64 * h;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(u32x4_t*)(dst + 16 * i) =
            (u32x4_t){packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]};
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(u32x4_t*)(&tile[row][64 * h + 16 * i]) =
          (u32x4_t){packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]};
    __syncthreads();
    // Thread -> (dim c, 64-token half). Output row c of [d, N] is contiguous in tokens.
    const int c = tid >> 1;
    const int t0 = blk * QBLOCK + 64 * h;
    uint8_t* dst = x8 + ((size_t)bh * QD + c) * N + t0;
#pragma unroll
    for (int q16 = 0; q16 < 4; ++q16) {
      if (t0 + 16 * q16 < N) {  // N is a multiple of 16
        unsigned w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int r = 64 * h + 16 * q16 + 4 * k;
          w[k] = (unsigned)tile[r][c] | ((unsigned)tile[r + 1][c] << 8) |
                 ((unsigned)tile[r + 2][c] << 16) | ((unsigned)tile[r + 3][c] << 24);
        }
        *(u32x4_t*)(dst + 16 * q16) = (u32x4_t){w[0], w[1], w[2], w[3]};
      }
    }
  }
  if (tid == 0) descale[(size_t)bh * nb + blk] = (float)(amax / div);
}

}  // namespace

hipError_t launch_quantize_fp8(const void* x, uint8_t* x8, float* descale, int B, int H, int N,
                               const float* signs, bool transpose_out, hipStream_t stream) {
  const int nb = (N + QBLOCK - 1) / QBLOCK;
  const double div = signs ? 448.0 * sqrt((double)QD) : 448.0;
  hipLaunchKernelGGL(quantize_kernel, dim3(nb * B * H), dim3(QTHREADS), 0, stream,
                     (const uint16_t*)x, x8, descale, N, nb, signs, transpose_out ? 1 : 0, div);
  return hipGetLastError();
}

}  // namespace exattn
