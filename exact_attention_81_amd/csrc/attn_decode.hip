// Split-KV attention forward for decode-shaped problems on gfx950 (MI355X), bf16 /
// fp16 inputs with grouped KV heads, and the merge of the per-split results.
//
// Decode attends a few query rows per head to a long key sequence, and with
// grouped-query attention (H_kv < H key/value heads) one workgroup per KV head
// leaves most compute units idle. The key sequence is therefore cut into
// splits that run as separate workgroups, and their partial results are
// combined by the associative merge of (O, LSE) pairs in a second, light pass
// ("Attention at Scale - From FlashAttention to FlashAttention-4", section
// "Beyond Training: Attention Kernels for Serving", subsections "FlashInfer"
// and "Sequence-Aware Split Heuristic").
//
// Work split. One workgroup per (batch, KV head, split); a split is a range of
// keys. The query rows that share the KV head (g = H / H_kv heads times N_q
// queries, at most 128) are the MFMA column blocks, 32 rows each (NRB blocks).
// Four waves: wave w takes row block w % NRB and every NKP-th 32-key tile of
// the range, starting at tile w / NRB (NKP = 4 / NRB). Each wave streams its
// own tiles through a private two-stage LDS ring with direct-to-LDS loads and
// waits only for its own loads, so the loop has no workgroup barrier. The
// problem is bound by reading K and V once from HBM; the products are the
// same S^T = K Q^T and O^T += V^T P^T on 32x32x16 MFMAs as in the prefill
// kernel, and the softmax is the same online softmax with the row maximum
// refreshed only past 8 doublings. At the end the waves of a row block merge
// their (m, l, O) states through LDS and write O and LSE (one split) or the
// fp32 partial (O_s = O normalised by its own sum, LSE_s) of the split.
#include <mutex>

#include "device.h"
#include "mfma16.h"
#include "tile_io.h"

namespace exattn {
namespace {

constexpr int DEC_WAVES = 4;
constexpr int DEC_THREADS = 64 * DEC_WAVES;
constexpr int DEC_N = 32;  // keys per tile
constexpr int DEC_TAU = 8;  // rescale threshold, doublings

template <int D, bool CAUSAL, bool F16, int NRB>
__global__ __launch_bounds__(DEC_THREADS) void attn_decode_kernel(const DecodeParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(NRB == 1 || NRB == 2 || NRB == 4, "row blocks");
  typedef Elem<F16> E;
  constexpr int KS = D / 16;            // MFMA K-steps of S^T
  constexpr int DB = D / 32;            // 32-row blocks of O^T
  constexpr int ROW = D * 2;            // bytes per K or V row
  constexpr bool W16 = D == 128;        // 16 chunks of 16 bytes per row (else 8)
  constexpr int TILE = DEC_N * ROW;     // bytes of one K (or V) tile
  constexpr int NLD = TILE / 1024;      // wave-wide 1 KB direct loads per K (or V) tile
  constexpr int STAGE = 2 * TILE;       // K tile, then V tile
  constexpr int NKP = DEC_WAVES / NRB;  // waves sharing one row block
  __shared__ __attribute__((aligned(1024))) uint8_t smem[DEC_WAVES * 2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int rb = wave % NRB;
  const int kp = wave / NRB;

  const int g = p.H / p.Hkv;
  const int rows = g * p.Nq;
  const int split = blockIdx.x % p.splits;
  const int bk = blockIdx.x / p.splits;  // b * H_kv + KV head
  const int b = bk / p.Hkv;
  const int hk = bk % p.Hkv;
  const int kv0 = split * p.chunk;
  const int kv1 = min(p.Nkv, kv0 + p.chunk);

  // ---- This lane's query row: i = 32 rb + l32 -> head hk*g + i / N_q, query i % N_q.
  // Rows past the group (i >= g*N_q) repeat its first row; they are never stored.
  const int i = rb * 32 + l32;
  const bool real = i < rows;
  const int h = hk * g + (real ? i / p.Nq : 0);
  const int t = real ? i % p.Nq : 0;
  const size_t qrow = ((size_t)b * p.H + h) * p.Nq + t;  // row of [B*H*N_q]
  // Keys visible to the row: j <= limit (causal: j <= t + N_kv - N_q, bottom-right).
  const int limit = CAUSAL ? min(p.Nkv - 1, t + p.Nkv - p.Nq) : p.Nkv - 1;
  int lim_min = limit, lim_max = limit;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lim_min = min(lim_min, __shfl_xor(lim_min, o));
    lim_max = max(lim_max, __shfl_xor(lim_max, o));
  }
  lim_min = __builtin_amdgcn_readfirstlane(lim_min);
  lim_max = __builtin_amdgcn_readfirstlane(lim_max);

  u32x4_t qf[KS];  // Q^T fragments (B operand): query column l32, 8 dims per K-step
  {
    const uint8_t* src = (const uint8_t*)p.q + qrow * ROW + half * 16;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *(const u32x4_t*)(src + s * 32);
  }

  // ---- The wave's tiles: 32-key tiles kp, kp + NKP, ... of [kv0, kv_end).
  const int kv_end = CAUSAL ? min(kv1, lim_max + 1) : kv1;
  const int ntiles = kv_end > kv0 ? (kv_end - kv0 + DEC_N - 1) / DEC_N : 0;
  const int my_n = ntiles > kp ? (ntiles - kp + NKP - 1) / NKP : 0;

  const uint8_t* kg = (const uint8_t*)p.k + (size_t)bk * p.Nkv * ROW;
  const uint8_t* vg = (const uint8_t*)p.v + (size_t)bk * p.Nkv * ROW;
  lds_u8* const ring = (lds_u8*)smem + wave * 2 * STAGE;

  // Direct-to-LDS loads: instruction ii fills bytes [1024 ii, 1024 ii + 1024) of the
  // tile; lane l writes the 16 bytes at 1024 ii + 16 l, so it loads the global chunk
  // that belongs at that swizzled position. Rows past N_kv read as zeros (the buffer
  // resource ends at N_kv); the wave's tiles past its last one are "loaded" through an
  // empty resource, which keeps the count of loads in flight the same every tile.
  int k_off[NLD], v_off[NLD];
#pragma unroll
  for (int ii = 0; ii < NLD; ++ii) {
    constexpr int rows_per = 1024 / ROW, cpr = ROW / 16;
    const int r = ii * rows_per + lane / cpr;
    k_off[ii] = r * ROW + k_swz(lane % cpr, r, W16) * 16;
    v_off[ii] = r * ROW + v_swz(lane % cpr, r, W16) * 16;
  }
  auto key0_of = [&](int u) { return u < my_n ? kv0 + (kp + u * NKP) * DEC_N : p.Nkv; };
  auto issue = [&](int u, int stage) {
    const int key0 = key0_of(u);
    const i32x4_t krs = make_rsrc(kg + (size_t)key0 * ROW, (unsigned)(p.Nkv - key0) * ROW);
    const i32x4_t vrs = make_rsrc(vg + (size_t)key0 * ROW, (unsigned)(p.Nkv - key0) * ROW);
    lds_u8* st = ring + stage * STAGE;
#pragma unroll
    for (int ii = 0; ii < NLD; ++ii) buffer_load_lds16(krs, st + ii * 1024, k_off[ii]);
#pragma unroll
    for (int ii = 0; ii < NLD; ++ii) buffer_load_lds16(vrs, st + TILE + ii * 1024, v_off[ii]);
  };

  // LDS read offsets inside a stage. K operand of S^T: row l32, chunk 2 s + half.
  int koff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) koff[s] = l32 * ROW + k_swz(2 * s + half, l32, W16) * 16;
  // V^T operand of O^T, for a 16-key step and 32-dim block db: lane j of its 16-lane
  // group reads row 4 half + j/4 (+8), columns 32 db + 16 g16 + 4 (j%4), which puts the
  // keys in the order of the S^T accumulator rows (the B operand P^T).
  int voff[DB];
  {
    const int j = lane & 15, g16 = (lane >> 4) & 1;
    const int rl = 4 * half + (j >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      voff[db] = TILE + rl * ROW + v_swz(4 * db + 2 * g16 + ((j & 3) >> 1), rl, W16) * 16 + 8 * (j & 1);
  }

  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_ref = -INFINITY;  // running reference max, log2 units
  float l_part = 0.f;       // this lane's half of the row sum
  const float c = p.scale_log2;

  issue(0, 0);
  issue(1, 1);
  // A negative scale is applied as -Q (sign bits only, exact) with |scale| in c. The
  // empty asm keeps the wait for the Q loads after the first tile loads are issued.
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    asm volatile("" : "+v"(qf[s]));
    qf[s] ^= p.q_neg;
  }
  for (int u = 0; u < my_n; ++u) {
    const int stage = u & 1;
    const lds_u8* st = ring + stage * STAGE;
    // Tile u has landed once at most the next tile's loads are outstanding.
    __builtin_amdgcn_s_waitcnt(((2 * NLD) & 15) | (7 << 4) | (15 << 8) | (((2 * NLD) >> 4) << 14));
    asm volatile("" ::: "memory");

    // S^T = K Q^T for the tile's 32 keys.
    f32x16_t sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
    u32x4_t kf = lds_read128(st + koff[0]);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4_t cur = kf;
      if (s + 1 < KS) kf = lds_read128(st + koff[s + 1]);
      sacc = E::mfma(cur, qf[s], sacc);
    }

    // Online softmax. Register r holds key key0 + 8 (r/4) + 4 half + r%4.
    const int key0 = key0_of(u);
    const bool mask = key0 + DEC_N - 1 > lim_min;  // some key of the tile is hidden from some row
    const int room = limit - key0 - 4 * half;
    auto visible = [&](int r) { return (r >> 2) * 8 + (r & 3) <= room; };
    if (mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!visible(r)) sacc[r] = -INFINITY;
    }
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = max_halves(mx);
    const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
    const bool grow = mt > m_ref + (float)DEC_TAU;
    if (__any(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - mt) : 1.f;
      m_ref = grow ? mt : m_ref;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float nm = (m_ref == -INFINITY) ? 0.f : -m_ref;
    float pv[16];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float e = __builtin_amdgcn_exp2f(fmaf(sacc[r], c, nm));
      if (mask) e = visible(r) ? e : 0.f;
      pv[r] = e;
      psum += e;
    }
    l_part += psum;
    u32x4_t pf[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 4; ++e) pf[hh][e] = E::pack2(pv[hh * 8 + 2 * e], pv[hh * 8 + 2 * e + 1]);

    // O^T += V^T P^T: two 16-key steps per 32-dim block.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const lds_u8* a = st + voff[db] + ks * 16 * ROW;
        const u32x2_t lo = lds_read_tr16(a);
        const u32x2_t hi = lds_read_tr16(a + 8 * ROW);
        oacc[db] = E::mfma((u32x4_t){lo[0], lo[1], hi[0], hi[1]}, pf[ks], oacc[db]);
      }

    // Every read of this stage has returned before it is refilled.
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
    asm volatile("" ::: "memory");
    issue(u + 2, stage);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // no LDS fill may be in flight past this point

  // ---- Merge the states of the waves that share a row block (same rule as the split
  // merge, in log2 units): M = max m_k, l = sum l_k 2^(m_k - M), O = sum O_k 2^(m_k - M).
  float l = sum_halves(l_part);
  if constexpr (NKP > 1) {
    constexpr int SLOT = (DB * 16 + 2) * 64;  // floats per wave: O^T registers, m, l
    float* const box = (float*)smem;
    __syncthreads();  // every ring is drained and no longer read
    if (kp > 0) {
      float* mine = box + wave * SLOT;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(db * 16 + r) * 64 + lane] = oacc[db][r];
      mine[DB * 16 * 64 + lane] = m_ref;
      mine[(DB * 16 + 1) * 64 + lane] = l;
    }
    __syncthreads();
    if (kp == 0) {
      for (int k2 = 1; k2 < NKP; ++k2) {
        const float* other = box + (rb + k2 * NRB) * SLOT;
        const float m2 = other[DB * 16 * 64 + lane];
        const float l2 = other[(DB * 16 + 1) * 64 + lane];
        const float mm = fmaxf(m_ref, m2);
        const float a1 = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - mm);
        const float a2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - mm);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            oacc[db][r] = oacc[db][r] * a1 + other[(db * 16 + r) * 64 + lane] * a2;
        l = l * a1 + l2 * a2;
        m_ref = mm;
      }
    }
  }
  if (kp != 0 || !real) return;

  // ---- Output: O = acc / l and LSE = ln2 (m + log2 l); no visible key: O = 0, LSE = -inf.
  const bool any = l > 0.f;
  const float inv = any ? __builtin_amdgcn_rcpf(l) : 0.f;
  const float lse = any ? 0.69314718055994531f * (m_ref + __builtin_amdgcn_logf(l)) : -INFINITY;
  if (p.splits == 1) {
    uint8_t* og = (uint8_t*)p.o + qrow * ROW;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const u32x2_t w = {E::pack2(oacc[db][gq * 4 + 0] * inv, oacc[db][gq * 4 + 1] * inv),
                           E::pack2(oacc[db][gq * 4 + 2] * inv, oacc[db][gq * 4 + 3] * inv)};
        *(u32x2_t*)(og + (db * 32 + gq * 8 + half * 4) * 2) = w;
      }
    if (half == 0) p.lse[qrow] = lse;
  } else {
    const size_t prow = (size_t)split * ((size_t)p.B * p.H * p.Nq) + qrow;
    float* og = p.o_part + prow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4_t w = {oacc[db][gq * 4 + 0] * inv, oacc[db][gq * 4 + 1] * inv,
                           oacc[db][gq * 4 + 2] * inv, oacc[db][gq * 4 + 3] * inv};
        *(f32x4_t*)(og + db * 32 + gq * 8 + half * 4) = w;
      }
    if (half == 0) p.lse_part[prow] = lse;
  }
}

// Merge of the split partials, one row per group of D/4 lanes (4 dims per lane):
// M = max_s LSE_s, w_s = exp(LSE_s - M), O = sum w_s O_s / sum w_s, LSE = M + ln sum w_s.
template <int D, bool F16>
__global__ __launch_bounds__(256) void merge_splits_kernel(const float* __restrict__ o_part,
                                                           const float* __restrict__ lse_part,
                                                           void* o, float* lse, int R, int S) {
  typedef Elem<F16> E;
  constexpr int LPR = D / 4;  // lanes per row
  const int row = blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int cq = threadIdx.x % LPR;
  if (row >= R) return;
  float m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmaxf(m, lse_part[(size_t)s * R + row]);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float out_lse = -INFINITY;
  if (m != -INFINITY) {
    float total = 0.f;
    for (int s = 0; s < S; ++s) {
      const float ls = lse_part[(size_t)s * R + row];
      const float w = ls == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((ls - m) * 1.4426950408889634f);
      total += w;
      const f32x4_t x = *(const f32x4_t*)(o_part + ((size_t)s * R + row) * D + 4 * cq);
      acc += w * x;
    }
    const float inv = __builtin_amdgcn_rcpf(total);
    acc *= inv;
    out_lse = m + 0.69314718055994531f * __builtin_amdgcn_logf(total);
  }
  const u32x2_t w2 = {E::pack2(acc[0], acc[1]), E::pack2(acc[2], acc[3])};
  *(u32x2_t*)((uint8_t*)o + ((size_t)row * D + 4 * cq) * 2) = w2;
  if (cq == 0) lse[row] = out_lse;
}

template <int D, bool CAUSAL, bool F16>
hipError_t launch_rb(const DecodeParams& p, int nrb, hipStream_t s) {
  const dim3 grid(p.B * p.Hkv * p.splits);
  if (nrb == 1) hipLaunchKernelGGL((attn_decode_kernel<D, CAUSAL, F16, 1>), grid, dim3(DEC_THREADS), 0, s, p);
  else if (nrb == 2) hipLaunchKernelGGL((attn_decode_kernel<D, CAUSAL, F16, 2>), grid, dim3(DEC_THREADS), 0, s, p);
  else hipLaunchKernelGGL((attn_decode_kernel<D, CAUSAL, F16, 4>), grid, dim3(DEC_THREADS), 0, s, p);
  return hipGetLastError();
}

template <int D, bool F16>
hipError_t launch_d(const DecodeParams& p, bool causal, hipStream_t s) {
  const int rows = p.H / p.Hkv * p.Nq;
  const int nrb = rows <= 32 ? 1 : rows <= 64 ? 2 : 4;
  hipError_t e = causal ? launch_rb<D, true, F16>(p, nrb, s) : launch_rb<D, false, F16>(p, nrb, s);
  if (e != hipSuccess || p.splits == 1) return e;
  const int R = p.B * p.H * p.Nq;
  constexpr int RPB = 256 / (D / 4);
  hipLaunchKernelGGL((merge_splits_kernel<D, F16>), dim3((R + RPB - 1) / RPB), dim3(256), 0, s,
                     p.o_part, p.lse_part, p.o, p.lse, R, p.splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode16(const DecodeParams& p, int d, bool causal, bool fp16, hipStream_t stream) {
  if (d == 64) return fp16 ? launch_d<64, true>(p, causal, stream) : launch_d<64, false>(p, causal, stream);
  if (d == 128) return fp16 ? launch_d<128, true>(p, causal, stream) : launch_d<128, false>(p, causal, stream);
  return hipErrorInvalidValue;
}

// ---- Static scratch for callers that cannot allocate (attn_fwd_decode_noalloc).
// The split partials of a call live in this file-scope device array instead of a
// caller-supplied workspace. Every GPU the library runs on holds its own copy until
// the process ends. In host code `scratch` only names the symbol: its device address
// on the current GPU comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kDecodeScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

size_t decode_scratch_bytes() { return kDecodeScratchBytes; }

hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `dev` current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

int decode_resident_workgroups(int d) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  // LDS per workgroup: 4 waves x 2 stages x (K + V) tiles of 32 rows = 32 KB (d 64) or
  // 128 KB (d 128) of the 160 KB of a compute unit.
  return cus * (d == 64 ? 2 : 1);
}

}  // namespace exattn
