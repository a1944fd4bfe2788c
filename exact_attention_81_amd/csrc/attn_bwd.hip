// Attention backward on gfx950 (MI355X), bf16 / fp16: dQ, dK, dV from Q, K, V, O, dO
// and the forward's LSE.
//
// The gradient of one (b, h) is five matrix products and two elementwise steps
// ("FlashAttention-4: Algorithm and Kernel Pipelining Co-Design for Asymmetric
// Hardware Scaling", Figure 2; "FlashAttention 3 and 4: When the Bottleneck
// Moves", section 3.2, the backward-pass paragraph): with the scores recomputed
// from Q, K and the saved LSE, P = exp(scale Q K^T - LSE),
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   dQ = scale dS K,
//     dK = scale dS^T Q,   D_i = sum_c dO_ic O_ic.
// Two kernels, no atomics, so every result is deterministic:
//   * attn_bwd_dq_kernel: one workgroup per 128 query rows streams the K/V tiles
//     (S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T) and also writes D;
//   * attn_bwd_dkdv_kernel: one workgroup per 128 keys streams 32-query tiles of
//     Q, dO, LSE and D (S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS).
// Products are 32x32x16 MFMAs with the operand layouts of the forward kernel: a
// 16-byte piece of a row per lane for row operands, transposing LDS reads for
// the transposed ones, and P / dS fed from the accumulator registers in the
// row order the transposing reads reproduce. Tiles go straight from global memory
// into LDS (buffer_load ... lds), double-buffered, one workgroup barrier per tile.
// Within a tile, LDS operands are read two products ahead of their MFMA, and the
// elementwise steps run between the products that do not need them (P beside the
// dP products, dS beside the dV products). Tiles whose scores are all visible take
// a body without any mask test; the masked body only runs on ragged and (causal)
// diagonal tiles, in a loop of its own.
#include "device.h"
#include "mfma16.h"
#include "tile_io.h"

namespace exattn {
namespace {

constexpr int BW_WAVES = 4;
constexpr int BW_THREADS = 64 * BW_WAVES;

// Chunk position of 16-byte chunk c of row r in tiles that are read both ways: by rows
// (16 lanes read one chunk of 16 consecutive rows) and transposed (32 lanes read 8 bytes
// in each of 4 chunks of 4 consecutive rows). The XOR mask takes the 16 rows to 16
// distinct chunk positions and the 4 x 4 (row, chunk) pairs of a transposed read to 16
// distinct positions, so neither read meets a bank conflict:
//   16-chunk rows: mask = 4 (r mod 4) + (r / 4 mod 4);
//    8-chunk rows (two rows per 256 bytes): mask = 4 (r/2 mod 2) + (r / 4 mod 4).
__device__ constexpr int b_swz(int c, int r, bool w16) {
  return w16 ? (c ^ (((r & 3) << 2) | ((r >> 2) & 3))) : (c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)));
}

// Row-major tile of R rows x D 16-bit values in LDS, 16-byte chunks swizzled by b_swz.
// Reads: a row piece (A or B operand of a product over D), or, through the transposing
// read, a block of the transposed tile (A operand of a product over the tile's rows,
// rows in the order of the MFMA accumulator rows).
template <int D>
struct SwzTile {
  static constexpr int ROW = D * 2;
  static constexpr bool W16 = D == 128;
  // Byte offset of chunk c (16 bytes) of row r.
  static __device__ int at(int r, int c) { return r * ROW + b_swz(c, r, W16) * 16; }
};

// Direct-to-LDS load of rows [row0, row0 + R) of a [N, D] 16-bit matrix at `base`
// (rows past N read as zeros) into an LDS tile; the waves of the workgroup share the
// 1 KB instructions: instruction i fills LDS bytes [1024 i, 1024 i + 1024), lane l
// writes the 16 bytes at 1024 i + 16 l, so it loads the chunk that belongs there.
template <int D, int R, int NW = BW_WAVES>
__device__ inline void load_tile(lds_u8* dst, const uint8_t* base, int row0, int N, int wave, int lane) {
  constexpr int ROW = D * 2, NI = R * ROW / 1024, ROWS_PER = 1024 / ROW, CPR = ROW / 16;
  static_assert(NI % NW == 0, "every wave issues the same number of loads");
  const int r0 = min(row0, N);
  const i32x4_t rs = make_rsrc(base + (size_t)r0 * ROW, (unsigned)(N - r0) * ROW);
#pragma unroll
  for (int t = 0; t < NI / NW; ++t) {
    const int i = wave + t * NW;
    const int r = i * ROWS_PER + lane / CPR;
    buffer_load_lds16(rs, dst + i * 1024, r * ROW + b_swz(lane % CPR, r, D == 128) * 16);
  }
}

// 256 floats of a float vector [N] from i0 on into LDS (past N: zeros); one wave.
__device__ inline void load_vec32(lds_u8* dst, const float* base, int i0, int N, int lane) {
  const int a = min(i0, N);
  const i32x4_t rs = make_rsrc(base + a, (unsigned)(N - a) * 4u);
  buffer_load_lds16(rs, dst, lane * 16);
}

// A operand of a product over 16 tile rows (K-step `ks` of a 32-row block at row
// `rb0`) taken from the transposed tile: lane j of each 16-lane group reads row
// 4 half + j/4 (+ 8), columns 32 db + 16 g16 + 4 (j % 4): MFMA row 32 db + l32, and the
// 16 tile rows in the order of the accumulator rows of a D-layout operand.
template <int D>
struct TrOffsets {
  int lo[D / 32], hi[D / 32];
  __device__ TrOffsets(int lane) {
    const int half = lane >> 5, j = lane & 15, g16 = (lane >> 4) & 1;
    const int rl = 4 * half + (j >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int c = 4 * db + 2 * g16 + ((j & 3) >> 1);
      lo[db] = SwzTile<D>::at(rl, c) + 8 * (j & 1);
      hi[db] = SwzTile<D>::at(rl + 8, c) + 8 * (j & 1);
    }
  }
};

// Rows 16 ks .. 16 ks + 15 of a tile differ from rows 0..15 by a multiple of 16, which
// leaves the b_swz pattern unchanged (it depends on r mod 16 only).
template <int D>
__device__ inline u32x4_t tr_operand(const lds_u8* tile, const TrOffsets<D>& off, int db, int row0) {
  const lds_u8* a = tile + row0 * SwzTile<D>::ROW;
  const u32x2_t lo = lds_read_tr16(a + off.lo[db]);
  const u32x2_t hi = lds_read_tr16(a + off.hi[db]);
  return (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
}

// Row operand: lane reads row row0 + l32, chunk 2 s + half (dims 16 s + 8 half .. + 8).
template <int D>
__device__ inline u32x4_t row_operand(const lds_u8* tile, int row0, int l32, int half, int s) {
  return lds_read128(tile + SwzTile<D>::at(row0 + l32, 2 * s + half));
}

// bf16/fp16 pairs of a D-layout accumulator (16 rows of one column per lane), as the
// B operands of the two 16-row K-steps of a product over those rows.
template <bool F16>
__device__ inline void pack_rows(const f32x16_t& x, u32x4_t out[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) out[h][i] = Elem<F16>::pack2(x[h * 8 + 2 * i], x[h * 8 + 2 * i + 1]);
}

__device__ inline float unpack_lo(unsigned w, bool f16) {
  return f16 ? (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffff))
             : __uint_as_float(w << 16);
}
__device__ inline float unpack_hi(unsigned w, bool f16) {
  return f16 ? (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16))
             : __uint_as_float(w & 0xffff0000u);
}

__device__ inline void wait_all_and_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------------
// dQ and D. Wave w owns queries q0 + 32 w + l32 (one MFMA column per lane).
template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(BW_THREADS) void attn_bwd_dq_kernel(const BwdParams p) {
  typedef Elem<F16> E;
  typedef SwzTile<D> T;
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int BN = 64;                       // keys per tile
  constexpr int TILE = BN * T::ROW;            // bytes of a K or V tile
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * 2 * TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  // One workgroup per (b*H + h, 128-query tile); the tiles of a head on one XCD (they
  // share its K/V through that XCD's L2), heavy causal tiles first.
  int bh, qt;
  map_block(blockIdx.x, (p.Nq + 32 * BW_WAVES - 1) / (32 * BW_WAVES), p.B * p.H, CAUSAL, bh, qt);
  const int q0 = qt * (32 * BW_WAVES);
  const int my_q = q0 + 32 * wave + l32;
  const int offset = p.Nkv - p.Nq;
  const size_t qbase = (size_t)bh * p.Nq, kbase = (size_t)bh * p.Nkv;
  const uint8_t* kg = (const uint8_t*)p.k + kbase * T::ROW;
  const uint8_t* vg = (const uint8_t*)p.v + kbase * T::ROW;

  // Q^T and dO^T fragments (B operands: query column l32, dims 16 s + 8 half .. + 8), O
  // for D = dO . O; rows past N_q read row N_q - 1 (never stored).
  const size_t row = qbase + min(my_q, p.Nq - 1);
  u32x4_t qf[KS], dof[KS];
  float dsum = 0.f;
  {
    const uint8_t* qs = (const uint8_t*)p.q + row * T::ROW + half * 16;
    const uint8_t* ds = (const uint8_t*)p.dout + row * T::ROW + half * 16;
    const uint8_t* os = (const uint8_t*)p.o + row * T::ROW + half * 16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = *(const u32x4_t*)(qs + s * 32);
      dof[s] = *(const u32x4_t*)(ds + s * 32);
      const u32x4_t ov = *(const u32x4_t*)(os + s * 32);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dsum += unpack_lo(dof[s][e], F16) * unpack_lo(ov[e], F16) +
                unpack_hi(dof[s][e], F16) * unpack_hi(ov[e], F16);
    }
  }
  const float dval = sum_halves(dsum);
  if (half == 0 && my_q < p.Nq) p.delta[qbase + my_q] = dval;
  // log2-domain LSE; a row with no visible key (LSE = -inf) gets P = 0 via +inf.
  const float lse_raw = p.lse[row];
  const float lse2 = lse_raw == -INFINITY ? INFINITY : lse_raw * 1.4426950408889634f;
  const float c = p.scale_log2;

  int kv_end = p.Nkv;
  if (CAUSAL) kv_end = min(p.Nkv, max(0, q0 + 32 * BW_WAVES + offset));
  const int ntiles = (kv_end + BN - 1) / BN;
  const int wave_last_key = q0 + 32 * wave + 31 + offset;

  f32x16_t dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;
  TrOffsets<D> tro(lane);
  const int limit = CAUSAL ? min(p.Nkv - 1, my_q + offset) : p.Nkv - 1;
  const float nl = -lse2;

  // One 32-key block: S^T = K Q^T, then dP^T = V dO^T with P^T = exp2(c S^T - LSE
  // log2 e) computed beside those products, then dQ^T += K^T dS^T with dS^T = P^T (dP^T
  // - D) computed beside the first of them. A operands are read two products ahead.
  // Register r is key key0 + 8 (r/4) + 4 half + r%4.
  auto key_block = [&](const lds_u8* kt, const lds_u8* vt, int kb, int key0, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int PER = 16 / KS;  // weights computed beside each dP product
    f32x16_t s_acc, dp_acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) s_acc[r] = dp_acc[r] = 0.f;
    // operand stream of the S then dP products (step < KS: K rows, else V rows)
    auto opa = [&](int step) { return row_operand<D>(step < KS ? kt : vt, 32 * kb, l32, half, step % KS); };
    u32x4_t a[2] = {opa(0), opa(1)};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4_t cur = a[s % 2];
      a[s % 2] = opa(s + 2);
      s_acc = E::mfma(cur, qf[s], s_acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int room = limit - key0 - 4 * half;
    constexpr int QSTEPS = 2 * DB;  // dQ products: step = ks * DB + db
    auto tra = [&](int step) { return tr_operand<D>(kt, tro, step % DB, 32 * kb + 16 * (step / DB)); };
    u32x4_t t[2];
    float pr[16];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int step = KS + s;
      const u32x4_t cur = a[step % 2];
      if (step + 2 < 2 * KS)
        a[step % 2] = opa(step + 2);
      else
        t[step + 2 - 2 * KS] = tra(step + 2 - 2 * KS);  // the first dQ operands
      dp_acc = E::mfma(cur, dof[s], dp_acc);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int r = s * PER + i;
        const float x = __builtin_amdgcn_exp2f(fmaf(s_acc[r], c, nl));
        pr[r] = (!MASK || (r >> 2) * 8 + (r & 3) <= room) ? x : 0.f;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    auto ds2 = [&](int w) {  // dS^T registers 2 w, 2 w + 1, packed
      return E::pack2(pr[2 * w] * (dp_acc[2 * w] - dval), pr[2 * w + 1] * (dp_acc[2 * w + 1] - dval));
    };
    u32x4_t dsf[2];
#pragma unroll
    for (int w = 0; w < 4; ++w) dsf[0][w] = ds2(w);
#pragma unroll
    for (int step = 0; step < QSTEPS; ++step) {
      const u32x4_t cur = t[step % 2];
      if (step + 2 < QSTEPS) t[step % 2] = tra(step + 2);
      dqacc[step % DB] = E::mfma(cur, dsf[step / DB], dqacc[step % DB]);
      if (step < DB) {
#pragma unroll
        for (int w = step * 4 / DB; w < (step + 1) * 4 / DB; ++w) dsf[1][w] = ds2(4 + w);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  constexpr std::false_type PLAIN{};
  constexpr std::true_type MASKED{};

  lds_u8* const kl = (lds_u8*)smem;
  lds_u8* const vl = (lds_u8*)smem + 2 * TILE;
  if (ntiles > 0) {
    load_tile<D, BN>(kl, kg, 0, p.Nkv, wave, lane);
    load_tile<D, BN>(vl, vg, 0, p.Nkv, wave, lane);
  }
  // Tiles before j_split have no key that some query of the workgroup misses; the rest
  // (the ragged tail, causal: the diagonal) take the masked body. The two ranges run as
  // two loops (one body each keeps the register allocation of each body on its own).
  const int wg_plain_key = CAUSAL ? min(p.Nkv - 1, q0 + offset) : p.Nkv - 1;
  const int j_split = min(ntiles, max(0, (wg_plain_key + 1) / BN));
  auto tile_loop = [&](int from, int to, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    for (int j = from; j < to; ++j) {
      const int st = j & 1;
      wait_all_and_barrier();  // tile j is in LDS; every wave is done with tile j - 1
      if (j + 1 < ntiles) {
        load_tile<D, BN>(kl + (st ^ 1) * TILE, kg, (j + 1) * BN, p.Nkv, wave, lane);
        load_tile<D, BN>(vl + (st ^ 1) * TILE, vg, (j + 1) * BN, p.Nkv, wave, lane);
      }
      if (CAUSAL && j * BN > wave_last_key) continue;  // no key of the tile is visible
      const lds_u8* kt = kl + st * TILE;
      const lds_u8* vt = vl + st * TILE;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key0 = j * BN + 32 * kb;
        // masked range: skip blocks past N_kv or past the wave's last visible key
        if (!MASK || (key0 < p.Nkv && (!CAUSAL || key0 <= wave_last_key))) key_block(kt, vt, kb, key0, mask_tag);
      }
    }
  };
  tile_loop(0, j_split, PLAIN);
  tile_loop(j_split, ntiles, MASKED);
  // dQ leaves through LDS as whole rows (stage_rows / store_rows); the barrier orders the
  // staging writes after every wave's last tile read.
  __builtin_amdgcn_s_waitcnt(0x0070);
  static_assert(BW_WAVES * 32 * staged_row_bytes<D>() <= 2 * 2 * TILE, "dQ staging fits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  lds_u8* const own = (lds_u8*)smem + wave * 32 * staged_row_bytes<D>();
  stage_rows<D, E>(own, dqacc, p.scale, lane);
  store_rows<D>((uint8_t*)p.dq + qbase * T::ROW, T::ROW, own, q0 + 32 * wave, p.Nq, lane);
}

// ---------------------------------------------------------------------------------
// dK and dV. 8 waves: wave w owns keys k0 + 32 (w % 4) + l32 (one MFMA column per lane)
// and the half w / 4 of each 64-query tile; the two waves of a key block add their
// partial sums at the end. Two waves per SIMD, so one's products overlap the other's
// exponentials.
constexpr int KV_WAVES = 8;
template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(64 * KV_WAVES) void attn_bwd_dkdv_kernel(const BwdParams p) {
  typedef Elem<F16> E;
  typedef SwzTile<D> T;
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int BK = 128;                      // keys per workgroup
  constexpr int BQ = 64;                       // queries per streamed tile
  constexpr int KTILE = BK * T::ROW;
  constexpr int QTILE = BQ * T::ROW;
  constexpr int STAGE = 2 * QTILE + 2 * 1024;  // Q, dO, LSE, D
  constexpr int SUM_BYTES = 4 * 2 * DB * 16 * 64 * 4;  // partial dK^T, dV^T of 4 waves
  constexpr int LDS = 2 * KTILE + 2 * STAGE > SUM_BYTES ? 2 * KTILE + 2 * STAGE : SUM_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int kw = wave & 3, qh = wave >> 2;
  // One workgroup per (b*H + h, 128-key tile); the tiles of a head on one XCD (they
  // share its Q, dO through that XCD's L2), causal: the tiles with most queries first.
  const int nkt = (p.Nkv + BK - 1) / BK;
  int bh, kt;
  map_block(blockIdx.x, nkt, p.B * p.H, CAUSAL, bh, kt);
  if (CAUSAL) kt = nkt - 1 - kt;
  const int k0 = kt * BK;
  const int wk0 = k0 + 32 * kw;  // this wave's first key
  const int my_k = wk0 + l32;
  const int offset = p.Nkv - p.Nq;
  const size_t qbase = (size_t)bh * p.Nq, kbase = (size_t)bh * p.Nkv;
  const uint8_t* qg = (const uint8_t*)p.q + qbase * T::ROW;
  const uint8_t* dg = (const uint8_t*)p.dout + qbase * T::ROW;

  lds_u8* const kl = (lds_u8*)smem;
  lds_u8* const vl = kl + KTILE;
  lds_u8* const ring = vl + KTILE;

  // Queries that see some key of the workgroup: i >= k0 - offset (causal).
  int qt0 = 0;
  if (CAUSAL) qt0 = max(0, k0 - offset) / BQ;
  const int qt1 = (p.Nq + BQ - 1) / BQ;
  auto issue = [&](int qt, int st) {
    lds_u8* s = ring + st * STAGE;
    load_tile<D, BQ, KV_WAVES>(s, qg, qt * BQ, p.Nq, wave, lane);
    load_tile<D, BQ, KV_WAVES>(s + QTILE, dg, qt * BQ, p.Nq, wave, lane);
    if (wave == 0) {
      load_vec32(s + 2 * QTILE, p.lse + qbase, qt * BQ, p.Nq, lane);
      load_vec32(s + 2 * QTILE + 1024, p.delta + qbase, qt * BQ, p.Nq, lane);
    }
  };
  load_tile<D, BK, KV_WAVES>(kl, (const uint8_t*)p.k + kbase * T::ROW, k0, p.Nkv, wave, lane);
  load_tile<D, BK, KV_WAVES>(vl, (const uint8_t*)p.v + kbase * T::ROW, k0, p.Nkv, wave, lane);
  if (qt0 < qt1) issue(qt0, 0);

  f32x16_t dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkacc[db][r] = dvacc[db][r] = 0.f;
  TrOffsets<D> tro(lane);
  const float c = p.scale_log2;

  // One tile of the wave's 32 queries: S = Q K^T, then dP = dO V^T with P = exp2(c S -
  // LSE log2 e) computed beside those products, then dV^T += dO^T P with dS = P (dP - D)
  // computed beside them, then dK^T += Q^T dS. Operands are read two products ahead.
  // Register r is query qa + 8 (r/4) + 4 half + r%4.
  //
  // Without a mask, keys past N_kv (zero rows of K and V) only reach their own columns of
  // dK and dV, which are never stored, and queries past N_q (zero rows of Q and dO, LSE
  // and D read as 0) add exact zeros. A query with LSE = -inf sees no key, which only
  // happens under the causal mask, so such rows only occur in masked tiles.
  auto q_tile = [&](const lds_u8* qtile, int qa, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int PER = 16 / KS;  // weights computed beside each dP product
    const lds_u8* dtile = qtile + QTILE;
    typedef const __attribute__((address_space(3))) f32x4_t lds_f32x4;
    lds_f32x4* lse_t = (lds_f32x4*)(qtile + 2 * QTILE + 128 * qh + 16 * half);
    lds_f32x4* del_t = (lds_f32x4*)(qtile + 2 * QTILE + 1024 + 128 * qh + 16 * half);
    f32x16_t s_acc, dp_acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) s_acc[r] = dp_acc[r] = 0.f;
    // operand stream of the S then dP products (step < KS: Q and K rows, else dO and V)
    auto opa = [&](int step) { return row_operand<D>(step < KS ? qtile : dtile, 32 * qh, l32, half, step % KS); };
    auto opb = [&](int step) { return row_operand<D>(step < KS ? kl : vl, 32 * kw, l32, half, step % KS); };
    u32x4_t a[2] = {opa(0), opa(1)}, b[2] = {opb(0), opb(1)};
    f32x4_t lz[4], dz[4];
#pragma unroll
    for (int sk = 0; sk < KS; ++sk) {
      const u32x4_t ca = a[sk % 2], cb = b[sk % 2];
      a[sk % 2] = opa(sk + 2);
      b[sk % 2] = opb(sk + 2);
      s_acc = E::mfma(ca, cb, s_acc);
      if (sk == 0) {
#pragma unroll
        for (int g = 0; g < 4; ++g) lz[g] = lse_t[2 * g];  // queries 8 g + 4 half .. + 3
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // causal: query qa + 8 (r/4) + 4 half + r%4 sees this lane's key iff
    // 8 (r/4) + r%4 >= my_k - offset - qa - 4 half
    const int tq = my_k - offset - qa - 4 * half;
    constexpr int STEPS = 2 * DB;  // transposed-operand products: step = ks * DB + db
    auto tra = [&](const lds_u8* tile, int step) {
      return tr_operand<D>(tile, tro, step % DB, 32 * qh + 16 * (step / DB));
    };
    u32x4_t t[2];
    float pr[16];
#pragma unroll
    for (int sk = 0; sk < KS; ++sk) {
      const int step = KS + sk;
      const u32x4_t ca = a[step % 2], cb = b[step % 2];
      if (step + 2 < 2 * KS) {
        a[step % 2] = opa(step + 2);
        b[step % 2] = opb(step + 2);
      } else {
        t[step + 2 - 2 * KS] = tra(dtile, step + 2 - 2 * KS);  // the first dV operands
      }
      dp_acc = E::mfma(ca, cb, dp_acc);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int r = sk * PER + i;
        const float x = __builtin_amdgcn_exp2f(fmaf(s_acc[r], c, lz[r >> 2][r & 3] * -1.4426950408889634f));
        pr[r] = (!MASK || (r >> 2) * 8 + (r & 3) >= tq) ? x : 0.f;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) dz[g] = del_t[2 * g];
    u32x4_t pf[2], dsf[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int w = 0; w < 4; ++w) pf[h][w] = E::pack2(pr[8 * h + 2 * w], pr[8 * h + 2 * w + 1]);
    auto ds2 = [&](int w) {  // dS registers 2 w, 2 w + 1, packed
      const int r = 2 * w;
      return E::pack2(pr[r] * (dp_acc[r] - dz[r >> 2][r & 3]), pr[r + 1] * (dp_acc[r + 1] - dz[r >> 2][(r & 3) + 1]));
    };
#pragma unroll
    for (int step = 0; step < STEPS; ++step) {
      const u32x4_t cur = t[step % 2];
      t[step % 2] = step + 2 < STEPS ? tra(dtile, step + 2) : tra(qtile, step + 2 - STEPS);
      dvacc[step % DB] = E::mfma(cur, pf[step / DB], dvacc[step % DB]);
#pragma unroll
      for (int w = step * 8 / STEPS; w < (step + 1) * 8 / STEPS; ++w) dsf[w / 4][w % 4] = ds2(w);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int step = 0; step < STEPS; ++step) {
      const u32x4_t cur = t[step % 2];
      if (step + 2 < STEPS) t[step % 2] = tra(qtile, step + 2);
      dkacc[step % DB] = E::mfma(cur, dsf[step / DB], dkacc[step % DB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  constexpr std::false_type PLAIN{};
  constexpr std::true_type MASKED{};

  // Causal: the query tiles before qt_split hold some query that misses some key of the
  // workgroup; from qt_split on every query sees all 128 keys. The two ranges run as two
  // loops (one body each keeps the register allocation of each body on its own).
  int qt_split = qt0;
  if (CAUSAL) {
    const int x = k0 + BK - 1 - offset;  // first query that sees the workgroup's last key
    qt_split = x <= 0 ? qt0 : min(qt1, max(qt0, (x + BQ - 1) / BQ));
  }
  auto tile_loop = [&](int from, int to, auto mask_tag) __attribute__((always_inline)) {
    for (int qt = from; qt < to; ++qt) {
      const int st = (qt - qt0) & 1;
      wait_all_and_barrier();  // tile qt is in LDS; every wave is done with tile qt - 1
      if (qt + 1 < qt1) issue(qt + 1, st ^ 1);
      const int qa = qt * BQ + 32 * qh;  // this wave's 32 queries
      // Causal: none of this wave's queries sees any of its keys (i sees j iff j <= i + offset).
      if (CAUSAL && qa + 31 + offset < wk0) continue;
      q_tile(ring + st * STAGE, qa, mask_tag);
    }
  };
  if (CAUSAL) tile_loop(qt0, qt_split, MASKED);
  tile_loop(qt_split, qt1, PLAIN);
  // The two waves of a key block add their partial sums through LDS.
  wait_all_and_barrier();  // every wave is done with the tiles
  float* const sums = (float*)smem + kw * (2 * DB * 16 * 64);
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sums[((2 * db) * 16 + r) * 64 + lane] = dkacc[db][r];
        sums[((2 * db + 1) * 16 + r) * 64 + lane] = dvacc[db][r];
      }
  }
  wait_all_and_barrier();
  if (qh == 0) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dkacc[db][r] += sums[((2 * db) * 16 + r) * 64 + lane];
        dvacc[db][r] += sums[((2 * db + 1) * 16 + r) * 64 + lane];
      }
    // dK and dV leave through LDS as whole rows (stage_rows / store_rows), staged in this
    // wave's own partial-sum area after its last read of it (one wave: the LDS keeps the
    // order). Rows past N_kv are not stored.
    static_assert(2 * 32 * staged_row_bytes<D>() <= 2 * DB * 16 * 64 * 4, "dK/dV staging fits");
    lds_u8* const own = (lds_u8*)smem + kw * (2 * DB * 16 * 64 * 4);
    stage_rows<D, E>(own, dkacc, p.scale, lane);
    stage_rows<D, E>(own + 32 * staged_row_bytes<D>(), dvacc, 1.f, lane);
    store_rows<D>((uint8_t*)p.dk + kbase * T::ROW, T::ROW, own, wk0, p.Nkv, lane);
    store_rows<D>((uint8_t*)p.dv + kbase * T::ROW, T::ROW, own + 32 * staged_row_bytes<D>(), wk0,
                  p.Nkv, lane);
  }
}

template <int D, bool CAUSAL, bool F16>
hipError_t launch_bwd(const BwdParams& p, hipStream_t s) {
  const int bh = p.B * p.H;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL, F16>),
                     dim3((p.Nq + 32 * BW_WAVES - 1) / (32 * BW_WAVES) * bh), dim3(BW_THREADS), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL, F16>),
                     dim3((p.Nkv + 127) / 128 * bh), dim3(64 * KV_WAVES), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, bool causal, bool fp16, hipStream_t s) {
  if (causal) return fp16 ? launch_bwd<D, true, true>(p, s) : launch_bwd<D, true, false>(p, s);
  return fp16 ? launch_bwd<D, false, true>(p, s) : launch_bwd<D, false, false>(p, s);
}

}  // namespace

hipError_t launch_bwd16(const BwdParams& p, int d, bool causal, bool fp16, hipStream_t stream) {
  if (d == 64) return launch_bwd_d<64>(p, causal, fp16, stream);
  if (d == 128) return launch_bwd_d<128>(p, causal, fp16, stream);
  return hipErrorInvalidValue;
}

}  // namespace exattn
