// Fused exact-attention forward for gfx950 (MI355X), bf16 / fp16 inputs.
//
// O = softmax(scale * Q K^T [+ causal mask]) V and LSE, one workgroup per
// (query tile, head, batch). The query tile stays in registers while K/V tiles
// stream from HBM through a double-buffered LDS ring; an online softmax keeps
// a running row maximum and row sum, so the N_q x N_kv scores never leave the
// chip ("Attention at Scale - From FlashAttention to FlashAttention-4",
// section "The Evolution": tiling and the online softmax). Loads of tile j+1
// are issued before the products of tile j, the gfx950 form of overlapping
// data movement with compute ("FlashAttention 3 and 4: When the Bottleneck
// Moves", section 2.1). The row maximum used by the exponentials is refreshed
// only when it grows by more than TAU doublings (same page, section 3.2).
//
// Work split. 4 waves x 64 query rows = BLOCK_M 256 rows per workgroup; key
// tiles of BLOCK_N 64. Each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_{bf16,f16}: the 32x32 accumulator gives every lane one
// query column and 16 keys, so the softmax row reductions are in-lane plus one
// exchange with lane ^ 32. The same registers, rounded to 16 bits, are the
// B operand of O^T += V^T P^T: the key order inside an MFMA K-step is the
// accumulator's row order, and V is written to LDS transposed with the
// matching key permutation, so P never moves between lanes.
#include "device.h"

namespace exattn {
namespace {

constexpr int BLOCK_M = 256;
constexpr int BLOCK_N = 64;
constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int ROWS_PER_WAVE = BLOCK_M / NWAVES;  // 64 = two 32-query MFMA columns
constexpr int KPAD = 8;                          // 16-byte row pad: conflict-free b128 reads
constexpr int VPAD = 8;

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

// Position of key `kk` (0..BLOCK_N-1) inside a row of the transposed V tile.
// Within each group of 16 keys, bits 2 and 3 of the key index are swapped, so
// that lanes 0-31 of an MFMA K-step find their 8 keys {0-3, 8-11} and lanes
// 32-63 theirs {4-7, 12-15} as one contiguous 16-byte read. This is exactly
// the key order of the S^T accumulator rows held by the two lane halves.
__device__ constexpr int vt_pos(int kk) {
  return (kk & ~15) | (((kk >> 2) & 1) << 3) | (((kk >> 3) & 1) << 2) | (kk & 3);
}

template <int DQK, int DV, bool CAUSAL, int TAU, bool F16>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(1, 1)))
void attn_fwd_kernel(const FwdParams p) {
  static_assert(DQK % 16 == 0 && DV % 32 == 0, "head dims");
  typedef Elem<F16> E;
  constexpr int KS = DQK / 16;            // MFMA K-steps of S^T
  constexpr int DB = DV / 32;             // 32-row blocks of O^T
  constexpr int KROW = DQK + KPAD;        // LDS row length of K (elements)
  constexpr int VROW = BLOCK_N + VPAD;    // LDS row length of V^T
  constexpr int K_CHUNKS = BLOCK_N * DQK / 8;         // 16-byte chunks per K tile
  constexpr int K_LOADS = (K_CHUNKS + NTHREADS - 1) / NTHREADS;
  constexpr int V_UNITS = (BLOCK_N / 4) * (DV / 8);   // 4 keys x 8 columns per unit
  constexpr int V_LOADS = (V_UNITS + NTHREADS - 1) / NTHREADS;

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BLOCK_N * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][DV * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  const int BH = p.B * p.H;
  int bh, qt;
  map_block(blockIdx.x, p.n_qtiles, BH, CAUSAL, bh, qt);
  const int q0 = qt * BLOCK_M;
  const int offset = p.Nkv - p.Nq;  // causal: key j visible to query i iff j <= i + offset

  const uint16_t* __restrict__ qg = (const uint16_t*)p.q + (size_t)bh * p.Nq * DQK;
  const uint16_t* __restrict__ kg = (const uint16_t*)p.k + (size_t)bh * p.Nkv * DQK;
  const uint16_t* __restrict__ vg = (const uint16_t*)p.v + (size_t)bh * p.Nkv * DV;

  // Keys this workgroup needs: all of them, or up to the last query's limit.
  int kv_end = p.Nkv;
  if (CAUSAL) kv_end = min(p.Nkv, max(0, q0 + BLOCK_M + offset));
  const int ntiles = (kv_end + BLOCK_N - 1) / BLOCK_N;

  // ---- Q^T fragments (B operand): lane = query column, 8 consecutive dims.
  const int wq0 = q0 + wave * ROWS_PER_WAVE;  // first query row of this wave
  u32x4_t qf[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = wq0 + qb * 32 + l32;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (row < p.Nq) x = *(const u32x4_t*)(qg + (size_t)row * DQK + s * 16 + half * 8);
      qf[qb][s] = x;
    }
  }

  // ---- Tile staging through registers.
  u32x4_t kreg[K_LOADS];
  u32x4_t vreg[V_LOADS][4];
  auto load_tile = [&](int j) {
    const int key0 = j * BLOCK_N;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int c = i * NTHREADS + tid;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (c < K_CHUNKS) {
        const int r = c / (DQK / 8), col = c % (DQK / 8);
        if (key0 + r < p.Nkv) x = *(const u32x4_t*)(kg + (size_t)(key0 + r) * DQK + col * 8);
      }
      kreg[i] = x;
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int u = i * NTHREADS + tid;
      const int kq = u % (BLOCK_N / 4), oct = u / (BLOCK_N / 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4_t x = {0u, 0u, 0u, 0u};
        const int key = key0 + kq * 4 + t;
        if (u < V_UNITS && key < p.Nkv) x = *(const u32x4_t*)(vg + (size_t)key * DV + oct * 8);
        vreg[i][t] = x;
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int c = i * NTHREADS + tid;
      if (c < K_CHUNKS) {
        const int r = c / (DQK / 8), col = c % (DQK / 8);
        *(u32x4_t*)(&k_lds[buf][r * KROW + col * 8]) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int u = i * NTHREADS + tid;
      if (u < V_UNITS) {
        const int kq = u % (BLOCK_N / 4), oct = u / (BLOCK_N / 4);
        const int pos = vt_pos(kq * 4);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const unsigned a0 = vreg[i][0][w], a1 = vreg[i][1][w];
          const unsigned a2 = vreg[i][2][w], a3 = vreg[i][3][w];
          // column 2w: low halves of the four keys; column 2w+1: high halves
          u32x2_t lo = {__builtin_amdgcn_perm(a1, a0, 0x05040100u),
                        __builtin_amdgcn_perm(a3, a2, 0x05040100u)};
          u32x2_t hi = {__builtin_amdgcn_perm(a1, a0, 0x07060302u),
                        __builtin_amdgcn_perm(a3, a2, 0x07060302u)};
          *(u32x2_t*)(&v_lds[buf][(oct * 8 + 2 * w) * VROW + pos]) = lo;
          *(u32x2_t*)(&v_lds[buf][(oct * 8 + 2 * w + 1) * VROW + pos]) = hi;
        }
      }
    }
  };

  // ---- Accumulators and softmax state (per lane: 2 query columns).
  f32x16_t oacc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][qb][r] = 0.f;
  float m_ref[2] = {-INFINITY, -INFINITY};  // running max, log2 units
  float l_part[2] = {0.f, 0.f};             // this lane's partial row sums
  const float c = p.scale_log2;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const bool has_next = j + 1 < ntiles;
    if (has_next) load_tile(j + 1);  // in flight during the products below

    const int key0 = j * BLOCK_N;
    // Skip the products when every key of the tile is in this wave's future.
    const bool wave_active = !CAUSAL || key0 <= wq0 + ROWS_PER_WAVE - 1 + offset;
    if (wave_active) {
      // S^T = K Q^T: 2 key blocks x 2 query blocks of 32x32.
      f32x16_t sacc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][qb][r] = 0.f;
      const uint16_t* kt = &k_lds[buf][0];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4_t kf = *(const u32x4_t*)(kt + (kb * 32 + l32) * KROW + s * 16 + half * 8);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) sacc[kb][qb] = E::mfma(kf, qf[qb][s], sacc[kb][qb]);
        }
      }

      // Mask the tail tile and the tiles that cross this wave's diagonal.
      const bool need_mask = (key0 + BLOCK_N > p.Nkv) ||
                             (CAUSAL && key0 + BLOCK_N - 1 > wq0 + offset);
      unsigned vis[2][2] = {{0xffffu, 0xffffu}, {0xffffu, 0xffffu}};  // bit r: key visible
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const int query = wq0 + qb * 32 + l32;
            const int limit = CAUSAL ? min(p.Nkv - 1, query + offset) : p.Nkv - 1;
            unsigned bits = 0;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
              const bool ok = key <= limit;
              bits |= (ok ? 1u : 0u) << r;
              if (!ok) sacc[kb][qb][r] = -INFINITY;
            }
            vis[kb][qb] = bits;
          }
      }

      // Online softmax: tile row max, conditional rescale, exponentials.
      float m_new[2];
      bool grow = false;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = sacc[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
        mx = max_halves(mx);
        const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
        m_new[qb] = fmaxf(m_ref[qb], mt);
        grow |= m_new[qb] > m_ref[qb] + (float)TAU;
      }
      if (__any(grow)) {  // wave-uniform branch; only rows past the threshold re-base
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const bool mine = m_new[qb] > m_ref[qb] + (float)TAU;
          const float alpha = mine ? __builtin_amdgcn_exp2f(m_ref[qb] - m_new[qb]) : 1.f;
          m_ref[qb] = mine ? m_new[qb] : m_ref[qb];
          l_part[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
        }
      }
      u32x4_t pf[2][4];  // P^T B operands: [query block][16-key step]
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float nm = (m_ref[qb] == -INFINITY) ? 0.f : -m_ref[qb];
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float pv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][qb][r], c, nm));
            if (need_mask) e = ((vis[kb][qb] >> r) & 1u) ? e : 0.f;
            pv[r] = e;
            psum += e;
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4_t w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = E::pack2(pv[h * 8 + 2 * i], pv[h * 8 + 2 * i + 1]);
            pf[qb][kb * 2 + h] = w;
          }
        }
        l_part[qb] += psum;
      }

      // O^T += V^T P^T.
      const uint16_t* vt = &v_lds[buf][0];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4_t vf = *(const u32x4_t*)(vt + (db * 32 + l32) * VROW + ks * 16 + half * 8);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = E::mfma(vf, pf[qb][ks], oacc[db][qb]);
        }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- Epilogue: O = acc / l, LSE = ln2 * (m + log2 l).
  uint16_t* __restrict__ og = (uint16_t*)p.o + (size_t)bh * p.Nq * DV;
  float* __restrict__ lg = p.lse + (size_t)bh * p.Nq;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = sum_halves(l_part[qb]);
    const int row = wq0 + qb * 32 + l32;
    const bool any = l > 0.f;
    const float inv = any ? __builtin_amdgcn_rcpf(l) : 0.f;
    if (row < p.Nq) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2_t w = {E::pack2(oacc[db][qb][g * 4 + 0] * inv, oacc[db][qb][g * 4 + 1] * inv),
                       E::pack2(oacc[db][qb][g * 4 + 2] * inv, oacc[db][qb][g * 4 + 3] * inv)};
          *(u32x2_t*)(og + (size_t)row * DV + db * 32 + g * 8 + half * 4) = w;
        }
      if (half == 0)
        lg[row] = any ? 0.69314718055994531f * (m_ref[qb] + __builtin_amdgcn_logf(l)) : -INFINITY;
    }
  }
}

template <int DQK, int DV, bool CAUSAL, int TAU, bool F16>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int grid = p.n_qtiles * p.B * p.H;
  hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, CAUSAL, TAU, F16>), dim3(grid), dim3(NTHREADS), 0,
                     stream, p);
  return hipGetLastError();
}

template <int DQK, int DV, bool F16>
hipError_t dispatch_mask(const FwdParams& p, bool causal, int tau, hipStream_t s) {
  if (causal) return tau == 0 ? launch<DQK, DV, true, 0, F16>(p, s) : launch<DQK, DV, true, 8, F16>(p, s);
  return tau == 0 ? launch<DQK, DV, false, 0, F16>(p, s) : launch<DQK, DV, false, 8, F16>(p, s);
}

}  // namespace

hipError_t launch_fwd16(const FwdParams& p0, int d_qk, int d_v, bool causal, bool fp16, int tau,
                        hipStream_t stream) {
  FwdParams p = p0;
  p.n_qtiles = (p.Nq + BLOCK_M - 1) / BLOCK_M;
  if (d_qk == 64 && d_v == 64)
    return fp16 ? dispatch_mask<64, 64, true>(p, causal, tau, stream)
                : dispatch_mask<64, 64, false>(p, causal, tau, stream);
  if (d_qk == 128 && d_v == 128)
    return fp16 ? dispatch_mask<128, 128, true>(p, causal, tau, stream)
                : dispatch_mask<128, 128, false>(p, causal, tau, stream);
  if (d_qk == 192 && d_v == 128)
    return fp16 ? dispatch_mask<192, 128, true>(p, causal, tau, stream)
                : dispatch_mask<192, 128, false>(p, causal, tau, stream);
  return hipErrorInvalidValue;
}

}  // namespace exattn
