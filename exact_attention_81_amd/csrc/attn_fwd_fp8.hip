// Fused exact-attention forward for gfx950 on OCP e4m3 (fp8) operands.
//
// Inputs are the codes and per-block descales written by the quantiser: Q and
// K [B,H,N,128] (optionally rotated by the same random-sign Hadamard matrix,
// which cancels in Q K^T), V transposed [B,H,128,N_kv], and one float32 descale
// per 128 tokens of each (b, h). Both products run on
// v_mfma_f32_32x32x64_f8f6f4 at twice the 16-bit rate, with P itself rounded
// to e4m3 ("FlashAttention 3 and 4: When the Bottleneck Moves", section 2.2;
// "Attention at Scale - From FlashAttention to FlashAttention-4", section "The
// Evolution", FlashAttention-3's FP8 path).
//
// The schedule is the one of the 16-bit kernel: 8 waves of 32 query rows,
// key tiles streamed into 3-stage LDS rings by direct-to-LDS loads, one
// barrier per tile, and two wave groups half an iteration apart so that one
// wave of every SIMD computes exponentials while the other feeds the matrix
// core.
//
// Scales. A 128-key tile is one descale block of K and V and a wave's 32
// query rows inside one 128-query block, so the score of a tile is
//     s * log2(e) = (scale * log2(e) * dq * dk) * (codes_q . codes_k),
// one scalar per wave and tile times the MFMA result. P is taken as
//     p = 2^(s - m_ref + PBIAS) * (dv / dv_ref),
// where dv is the tile's V descale and dv_ref the largest V descale of the
// head: the ratio folds V's dequantisation into the exponent (no per-tile
// rescale of the accumulator), and O = dv_ref * acc / l at the end. The row
// sum l adds the e4m3-rounded p, the very weights the PV product uses, divided
// by dv / dv_ref: the final weights p / l then sum to one exactly. With three
// mantissa bits, summing the unrounded p instead would leave every row off by
// the rounding of its largest weights (up to 2^-4), which on rows dominated by
// a few keys moves O by that share of |v|. The sum comes from the matrix core:
// one more e4m3 product per 64 keys, an all-ones A operand against the same
// P^T operand, gives every lane its query's sum over the 64 keys (the vector
// ALU, the busier unit here, is spared one add per score).
// The running maximum m_ref is re-based when the row maximum grows by more
// than TAU doublings (section 3.2 of the first page), so every p is at most
// 2^(TAU + PBIAS) = 256, inside e4m3's range (448), while a row's largest
// entries sit at 2^6 or above, far from e4m3's subnormals.
//
// Key order inside the PV product. Lane l of the S^T accumulator holds, for
// query l % 32, keys 8q + 4(l/32) + (0..3) of both 32-key halves of the tile.
// The B operand of O^T += V^T P^T needs lane half h to hold keys 32h..32h+31.
// After packing to e4m3 (4 keys per dword) one v_permlane32_swap per dword
// pair exchanges the halves, which leaves every lane with its 32 keys in
// natural order; the V^T operand is then 32 contiguous bytes of a dim row.
#include <type_traits>

#include "device.h"
#include "fp8_ops.h"
#include "mfma16.h"
#include "tile_io.h"

namespace exattn {
namespace {

constexpr int F8_BLOCK_M = 256;
constexpr int F8_BLOCK_N = 128;
constexpr int F8_NWAVES = 8;
constexpr int F8_NTHREADS = 64 * F8_NWAVES;
constexpr int F8_ROWS = F8_BLOCK_M / F8_NWAVES;  // 32 query rows per wave
constexpr int F8_D = 128;                          // d_qk = d_v
constexpr int F8_SBLOCK = 128;                     // tokens per descale block
constexpr int F8_TAU = 2;                          // re-base threshold, doublings
constexpr float F8_PBIAS = 6.f;                    // p <= 2^(F8_TAU + F8_PBIAS) = 256

static_assert(F8_SBLOCK % F8_BLOCK_N == 0 && F8_SBLOCK % F8_ROWS == 0 && F8_BLOCK_M % F8_SBLOCK == 0,
              "tiles and wave rows must not straddle descale blocks");

template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(F8_NTHREADS, F8_NTHREADS),
                          amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8_kernel(const FwdParams p) {
  constexpr int BLOCK_N = F8_BLOCK_N;
  constexpr int NWAVES = F8_NWAVES;
  constexpr int D = F8_D;
  constexpr int K_STAGE = BLOCK_N * D;   // 128 key rows x 128 B
  constexpr int VT_ROW = BLOCK_N;        // one dim row of the V^T tile: 128 keys
  constexpr int V_STAGE = D * VT_ROW;    // 128 dim rows x 128 B
  constexpr int NSTAGE = 3;
  constexpr int NKB = BLOCK_N / 32;      // 32-key blocks of S^T
  constexpr int NKC = BLOCK_N / 64;      // 64-key steps of the PV product
  constexpr int K_PER = K_STAGE / 1024 / NWAVES;  // 1 KB loads per wave and tile
  constexpr int V_PER = V_STAGE / 1024 / NWAVES;
  constexpr int LOADS_PER_TILE = K_PER + V_PER;
  static_assert(K_STAGE % (1024 * NWAVES) == 0 && V_STAGE % (1024 * NWAVES) == 0, "even loads");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * (K_STAGE + V_STAGE)];
  lds_u8* const k_lds = (lds_u8*)smem;
  lds_u8* const v_lds = (lds_u8*)smem + NSTAGE * K_STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const bool group_b = wave >= NWAVES / 2;

  const int BH = p.B * p.H;
  int bh, qt;
  map_block(blockIdx.x, p.n_qtiles, BH, CAUSAL, bh, qt);
  const int q0 = qt * F8_BLOCK_M;
  const int offset = p.Nkv - p.Nq;
  const int nbq = (p.Nq + F8_SBLOCK - 1) / F8_SBLOCK;
  const int nbk = (p.Nkv + F8_SBLOCK - 1) / F8_SBLOCK;

  const uint8_t* __restrict__ qg = (const uint8_t*)p.q + (size_t)bh * p.Nq * D;
  const uint8_t* __restrict__ kg = (const uint8_t*)p.k + (size_t)bh * p.Nkv * D;
  const uint8_t* __restrict__ vg = (const uint8_t*)p.v + (size_t)bh * D * p.Nkv;
  // Descales are read through the constant address space: the compiler may then use
  // scalar loads inside the loop, which the tile loads' memory clobbers would
  // otherwise forbid (a vector load there would wait for every tile load in flight).
  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat* const kds = (cfloat*)(p.k_descale + (size_t)bh * nbk);
  cfloat* const vds = (cfloat*)(p.v_descale + (size_t)bh * nbk);

  int kv_end = p.Nkv;
  if (CAUSAL) kv_end = min(p.Nkv, max(0, q0 + F8_BLOCK_M + offset));
  const int ntiles = (kv_end + BLOCK_N - 1) / BLOCK_N;

  // ---- Q^T fragments (B operand of S^T): query l32, dims 64 ks + 32 half + 0..31.
  const int wq0 = q0 + wave * F8_ROWS;
  const int my_q = wq0 + l32;
  // Rows past N_q repeat row N_q - 1: their results are never stored, and loading
  // unconditionally keeps the compiler from waiting for these loads (to merge them
  // with zeros) before the first tile loads are issued.
  i32x8_t qf[2];
  {
    const uint8_t* src = qg + (size_t)min(my_q, p.Nq - 1) * D + 32 * half;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      qf[ks] = join8(*(const u32x4_t*)(src + 64 * ks), *(const u32x4_t*)(src + 64 * ks + 16));
  }
  // The wave's rows share one Q descale block (a wave past N_q reads the last one).
  const float dq = ((cfloat*)p.q_descale)[(size_t)bh * nbq + min(wq0, p.Nq - 1) / F8_SBLOCK];
  // dv_ref: the head's largest V descale. The first 64 descales are loaded here and
  // reduced after the first tile barrier (see the prologue below).
  float dv_ref = lane < nbk ? vds[lane] : 0.f;
  float log2_dv_ref = 0.f;
  const float c = p.scale_log2 * dq;

  // ---- Direct-to-LDS tile loads; wave w fills bytes [1024 w, 1024 w + 1024) of a stage.
  // Both stages hold rows of 128 B (K: 128 key rows; V^T: 128 dim rows of 128 keys),
  // chunk c of row r at position c ^ ((r >> 1) & 7). Load t of wave w fills rows
  // 8 (w + 8 t) .. 8 (w + 8 t) + 7.
  int k_off[K_PER], v_off[V_PER], v_key[V_PER];
#pragma unroll
  for (int t = 0; t < K_PER; ++t) {
    const int r = (wave + t * NWAVES) * 8 + lane / 8;
    k_off[t] = r * D + ((lane % 8) ^ ((r >> 1) & 7)) * 16;
  }
#pragma unroll
  for (int t = 0; t < V_PER; ++t) {
    const int r = (wave + t * NWAVES) * 8 + lane / 8;
    const int cc = (lane % 8) ^ ((r >> 1) & 7);
    v_key[t] = cc * 16;  // first key of the lane's chunk within the tile
    v_off[t] = r * p.Nkv + v_key[t];
  }
  const unsigned v_bytes = (unsigned)(D * p.Nkv);
  const i32x4_t v_rs = make_rsrc(vg, v_bytes);
  // Tiles j >= ntiles (past N_kv, or past the causal diagonal of the query tile) go
  // through an empty resource or past its end: they read zeros and touch no memory.
  auto k_rsrc = [&](int j) {
    const int key0 = min(j * BLOCK_N, p.Nkv);
    return make_rsrc(kg + (size_t)key0 * D, j < ntiles ? (unsigned)(p.Nkv - key0) * D : 0u);
  };
  // V^T rows continue into the next dim row, so chunks past N_kv (N_kv is a multiple
  // of 16) are pointed past the end of the resource, which reads them as zeros.
  auto v_voff = [&](int j, int t) {
    const int key0 = j * BLOCK_N;
    return (j < ntiles && key0 + v_key[t] < p.Nkv) ? v_off[t] + key0 : (int)v_bytes;
  };
  auto issue_k = [&](int j, auto stage) {
    const i32x4_t rs = k_rsrc(j);
#pragma unroll
    for (int t = 0; t < K_PER; ++t)
      buffer_load_lds16(rs, k_lds + int(stage) * K_STAGE + (wave + t * NWAVES) * 1024, k_off[t]);
  };
  auto issue_v = [&](int j, auto stage) {
#pragma unroll
    for (int t = 0; t < V_PER; ++t)
      buffer_load_lds16(v_rs, v_lds + int(stage) * V_STAGE + (wave + t * NWAVES) * 1024, v_voff(j, t));
  };

  // ---- Per-lane LDS read offsets.
  // K operand of S^T, key block kb, K-step ks: row 32 kb + l32, chunks 4 ks + 2 half + u.
  int koff[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int u = 0; u < 2; ++u) koff[ks][u] = l32 * D + ((4 * ks + 2 * half + u) ^ ((l32 >> 1) & 7)) * 16;
  // V^T operand of O^T, dim block db, key step kc: row 32 db + l32, chunks
  // 4 kc + 2 half + u.
  int voff[NKC][2];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
    for (int u = 0; u < 2; ++u) voff[kc][u] = l32 * VT_ROW + ((4 * kc + 2 * half + u) ^ ((l32 >> 1) & 7)) * 16;

  f32x16_t oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  f32x16_t sacc[NKB];
  i32x8_t pf[NKC];           // P^T B operands (e4m3) between softmax and PV
  float m_ref = -INFINITY;   // running reference max, log2 units (bias excluded)
  float l_row = 0.f;         // the query's row sum (the same in both lane halves)
  float tile_inv_ratio = 1.f;  // dv_ref / dv of the tile between its softmax and PV
  float tile_alpha = 1.f;      // the tile's re-base factor for O, applied in its PV phase

  // S(j): S^T = K_j Q^T. Operands are read one product ahead of their MFMA.
  auto s_phase = [&](auto stage) {
    const lds_u8* st = k_lds + int(stage) * K_STAGE;
    constexpr int STEPS = 2 * NKB;  // step = ks * NKB + kb
    auto kread = [&](int step) {
      const int ks = step / NKB, kb = step % NKB;
      return join8(lds_read128(st + koff[ks][0] + kb * 32 * D), lds_read128(st + koff[ks][1] + kb * 32 * D));
    };
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
    i32x8_t kf = kread(0);
#pragma unroll
    for (int step = 0; step < STEPS; ++step) {
      const i32x8_t cur = kf;
      if (step + 1 < STEPS) kf = kread(step + 1);
      sacc[step % NKB] = mfma_f8(cur, qf[step / NKB], sacc[step % NKB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // PV(j): O^T += V_j^T P_j^T, operands two products ahead; hook(step) issues tile loads.
  // The row sum of the rounded P comes from two more products, ones^T P^T (every A
  // byte 1.0 in e4m3, 0x38), issued with the first PV products and read at the end.
  // The softmax's re-base factor is applied to each accumulator block right before its
  // first product of the tile, on every tile (a factor of 1 when no row grew, which is
  // exact). A wave-uniform branch around 64 multiplies in the softmax instead splits the
  // accumulators' live ranges, and the kernel spilled 56-68 B per lane around it.
  auto pv_phase = [&](auto stage, auto hook) {
    __builtin_amdgcn_s_setprio(0);  // the matrix phase yields to the softmax wave
    const lds_u8* st = v_lds + int(stage) * V_STAGE;
    constexpr int STEPS = 4 * NKC;  // step = kc * 4 + db
    auto vread = [&](int step) {
      const int kc = step / 4, db = step % 4;
      return join8(lds_read128(st + voff[kc][0] + db * 32 * VT_ROW), lds_read128(st + voff[kc][1] + db * 32 * VT_ROW));
    };
    i32x8_t vf[2] = {vread(0), vread(1)};
    const int one = 0x38383838;
    const i32x8_t ones = {one, one, one, one, one, one, one, one};
    f32x16_t lsum;
#pragma unroll
    for (int r = 0; r < 16; ++r) lsum[r] = 0.f;
#pragma unroll
    for (int step = 0; step < STEPS; ++step) {
      const i32x8_t cur = vf[step % 2];
      if (step + 2 < STEPS) vf[step % 2] = vread(step + 2);
      if (step < 4) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[step][r] *= tile_alpha;
      }
      oacc[step % 4] = mfma_f8(cur, pf[step / 4], oacc[step % 4]);
      if (step < NKC) lsum = mfma_f8(ones, pf[step], lsum);
      hook(step);
      __builtin_amdgcn_sched_barrier(0);
    }
    // every row of the ones product holds the query's sum over the tile's keys
    l_row = fmaf(lsum[0], tile_inv_ratio, l_row);
  };
  auto no_hook = [](int) {};

  auto softmax = [&](int j, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // The vector ALU is this kernel's busier unit: while a wave computes its softmax it
    // gets issue priority over the SIMD's other wave, which is then in its matrix phase
    // and needs an issue slot only every few MFMAs (+2.5 %; the opposite order -1.5 %).
    __builtin_amdgcn_s_setprio(1);
    const int blk = (j * BLOCK_N) / F8_SBLOCK;
    // Kept positive (a zero descale or scale gives 1e-30, which moves no score by a
    // representable amount) so that a masked score of -inf gives p = 0 by itself.
    const float ct = fmaxf(c * kds[blk], 1e-30f);
    const float dv = vds[blk];
    // log2(dv / dv_ref) <= 0; a zero block (all codes 0) keeps the bias 0.
    const float vbias = dv > 0.f ? __builtin_amdgcn_logf(dv) - log2_dv_ref : 0.f;
    tile_inv_ratio = __builtin_amdgcn_exp2f(-vbias);
    int room = 0;
    auto visible = [&](int kb, int r) { return kb * 32 + (r >> 2) * 8 + (r & 3) <= room; };
    if constexpr (MASK) {
      const int limit = CAUSAL ? min(p.Nkv - 1, my_q + offset) : p.Nkv - 1;
      room = limit - j * BLOCK_N - half * 4;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!visible(kb, r)) sacc[kb][r] = -INFINITY;
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = max_halves(mx);
    const float mt = (mx == -INFINITY) ? -INFINITY : mx * ct;
    const bool grow = mt > m_ref + (float)F8_TAU;
    tile_alpha = grow ? __builtin_amdgcn_exp2f(m_ref - mt) : 1.f;
    m_ref = grow ? mt : m_ref;
    l_row *= tile_alpha;
    const float nm = ((m_ref == -INFINITY) ? 0.f : -m_ref) + F8_PBIAS + vbias;
    unsigned w[NKB][4];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pv[r] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], ct, nm));
#pragma unroll
      for (int q = 0; q < 4; ++q) w[kb][q] = pack4_fp8(pv[4 * q], pv[4 * q + 1], pv[4 * q + 2], pv[4 * q + 3]);
    }
    // For each 64 keys (blocks 2 kc, 2 kc + 1): lanes 0-31 keep block 2 kc and receive
    // the partner's dwords of it; lanes 32-63 keep block 2 kc + 1 likewise.
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const auto r = __builtin_amdgcn_permlane32_swap(w[2 * kc][q], w[2 * kc + 1][q], false, false);
        pf[kc][2 * q] = (int)r[0];
        pf[kc][2 * q + 1] = (int)r[1];
      }
  };

  int j_plain = min(ntiles, p.Nkv / BLOCK_N);
  if (CAUSAL) j_plain = min(j_plain, max(0, (q0 + offset + 1) / BLOCK_N));
  const int wave_last_key = wq0 + F8_ROWS - 1 + offset;
  auto active = [&](int j) { return !CAUSAL || j * BLOCK_N <= wave_last_key; };
  constexpr std::false_type PLAIN{};
  constexpr std::true_type MASKED{};

  // Same barrier protocol as the 16-bit kernel: barrier j needs K(j) and V(j-1);
  // K(j+2) and V(j+1) are issued after it.
  auto pin_s = [&]() {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) asm volatile("" : "+v"(sacc[kb]));
  };
  auto pin_p = [&]() {
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) asm volatile("" : "+v"(pf[kc]));
  };
  auto barrier_and_issue = [&](int j, auto k_next, auto v_next) {
    tile_barrier<LOADS_PER_TILE>();
    issue_k(j + 2, k_next);
    issue_v(j + 1, v_next);
  };
  // The loads of an unrolled iteration go out between its PV products.
  constexpr int ISSUE_GAP = 4 * NKC / LOADS_PER_TILE;
  static_assert(ISSUE_GAP >= 1, "one load per PV product at most");
  auto spread_issue = [&](int j, auto k_next, auto v_next) {
    const i32x4_t krs = k_rsrc(j + 2);
    lds_u8* kdst = k_lds + int(k_next) * K_STAGE + wave * 1024;
    lds_u8* vdst = v_lds + int(v_next) * V_STAGE + wave * 1024;
    int vo[V_PER];
#pragma unroll
    for (int t = 0; t < V_PER; ++t) vo[t] = v_voff(j + 1, t);
    return [=](int step) {
      if (step % ISSUE_GAP != 0) return;
      const int li = step / ISSUE_GAP;
      if (li < K_PER) buffer_load_lds16(krs, kdst + li * NWAVES * 1024, k_off[li]);
      else if (li < LOADS_PER_TILE) buffer_load_lds16(v_rs, vdst + (li - K_PER) * NWAVES * 1024, vo[li - K_PER]);
    };
  };
  auto plain_iter = [&](int j, auto r_tag) {
    constexpr int R = decltype(r_tag)::value;
    constexpr std::integral_constant<int, R> k_cur{};
    constexpr std::integral_constant<int, (R + 2) % NSTAGE> v_prev{};
    constexpr std::integral_constant<int, (R + 2) % NSTAGE> k_next{};
    constexpr std::integral_constant<int, (R + 1) % NSTAGE> v_next{};
    if (group_b) {
      tile_barrier<LOADS_PER_TILE>();
      pin_s();
    }
    softmax(j - 1, PLAIN);
    if (!group_b) {
      pin_p();
      tile_barrier<LOADS_PER_TILE>();
    }
    pv_phase(v_prev, spread_issue(j, k_next, v_next));
    s_phase(k_cur);
  };
  auto any_iter = [&](int j) {
    const int r = j % NSTAGE;
    if (group_b) {
      barrier_and_issue(j, (r + 2) % NSTAGE, (r + 1) % NSTAGE);
      pin_s();
    }
    if (active(j - 1)) {
      if (j - 1 < j_plain) softmax(j - 1, PLAIN); else softmax(j - 1, MASKED);
    }
    if (!group_b) {
      pin_p();
      barrier_and_issue(j, (r + 2) % NSTAGE, (r + 1) % NSTAGE);
    }
    if (active(j - 1)) pv_phase((r + 2) % NSTAGE, no_hook);
    if (active(j)) s_phase(r);
  };
  if (ntiles > 0) {
    issue_k(0, 0);
    issue_k(1, 1);
    issue_v(0, 0);
    tile_barrier<LOADS_PER_TILE>();
    // The compiler waits for its own loads (the Q fragments, the V descales) at their
    // first use, and since it does not see the tile loads it waits for every load
    // (vmcnt(0)). Using them here, before K(2) and V(1) are issued, keeps that wait
    // from covering those two.
    // A negative scale is applied here as -Q (sign bits only, exact) with |scale| in c.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      asm volatile("" : "+v"(qf[ks]));
      qf[ks] ^= (int)p.q_neg;
    }
    for (int i = lane + 64; i < nbk; i += 64) dv_ref = fmaxf(dv_ref, vds[i]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dv_ref = fmaxf(dv_ref, __shfl_xor(dv_ref, off));
    // every lane holds the same maximum: keep it (and its log) in scalar registers
    dv_ref = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(dv_ref)));
    log2_dv_ref = dv_ref > 0.f ? __builtin_amdgcn_logf(dv_ref) : 0.f;
    log2_dv_ref = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(log2_dv_ref)));
    issue_k(2, 2);
    issue_v(1, 1);
    if (active(0)) s_phase(0);
    const int j_last_plain = min(j_plain, ntiles - 1);
    int j = 1;
    for (; j + 2 <= j_last_plain; j += 3) {
      plain_iter(j, std::integral_constant<int, 1>{});
      plain_iter(j + 1, std::integral_constant<int, 2>{});
      plain_iter(j + 2, std::integral_constant<int, 0>{});
    }
    for (; j < ntiles; ++j) any_iter(j);
    if (group_b) tile_barrier<LOADS_PER_TILE>();
    if (active(ntiles - 1)) {
      if (ntiles - 1 < j_plain) softmax(ntiles - 1, PLAIN); else softmax(ntiles - 1, MASKED);
    }
    if (!group_b) tile_barrier<LOADS_PER_TILE>();
    if (active(ntiles - 1)) pv_phase((ntiles - 1) % NSTAGE, no_hook);
  }

  __builtin_amdgcn_s_waitcnt(0x0070);  // no LDS fill may be in flight when the waves end

  // ---- Epilogue: O = dv_ref * acc / l (bf16, RNE), LSE = ln2 * (m_ref - PBIAS + log2 l).
  // The lane's query and half are recomputed from the lane id (mbcnt) rather than kept
  // in registers through the loop, where they would be spilled to scratch.
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int my_q_e = wq0 + (lane_e & 31), half_e = lane_e >> 5;
  const float l = l_row;
  const bool any = l > 0.f;
  const float inv = any ? dv_ref * __builtin_amdgcn_rcpf(l) : 0.f;
  // O leaves through LDS as whole rows (stage_rows / store_rows, bf16 with round to
  // nearest even); the barrier orders the staging writes after every wave's last ring
  // read and fill.
  static_assert(NWAVES * F8_ROWS * staged_row_bytes<D>() <= NSTAGE * (K_STAGE + V_STAGE),
                "O staging fits in the rings");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  lds_u8* const ot = (lds_u8*)smem + wave * F8_ROWS * staged_row_bytes<D>();
  stage_rows<D, Elem<false>>(ot, oacc, inv, lane_e);
  store_rows<D>((uint8_t*)p.o + (size_t)bh * p.Nq * D * 2, D * 2, ot, wq0, p.Nq, lane_e);
  if (my_q_e < p.Nq && half_e == 0)
    p.lse[(size_t)bh * p.Nq + my_q_e] =
        any ? 0.69314718055994531f * (m_ref - F8_PBIAS + __builtin_amdgcn_logf(l)) : -INFINITY;
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdParams& p0, bool causal, hipStream_t stream) {
  FwdParams p = p0;
  p.n_qtiles = (p.Nq + F8_BLOCK_M - 1) / F8_BLOCK_M;
  const int grid = p.n_qtiles * p.B * p.H;
  if (causal)
    hipLaunchKernelGGL(attn_fwd_fp8_kernel<true>, dim3(grid), dim3(F8_NTHREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_fwd_fp8_kernel<false>, dim3(grid), dim3(F8_NTHREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace exattn
