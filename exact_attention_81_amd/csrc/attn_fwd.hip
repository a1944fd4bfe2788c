// Fused exact-attention forward for gfx950 (MI355X), bf16 / fp16 inputs.
//
// O = softmax(scale * Q K^T [+ causal mask]) V and LSE, one workgroup per
// (query tile, head, batch). The query tile stays in registers while K/V tiles
// stream from HBM through LDS rings; an online softmax keeps a running row
// maximum and row sum, so the N_q x N_kv scores never leave the chip
// ("Attention at Scale - From FlashAttention to FlashAttention-4", section
// "The Evolution": tiling and the online softmax). Tiles go straight from
// global memory into LDS (buffer_load_dwordx4 ... lds) two iterations ahead of
// their use, and each barrier waits only for the loads that are due, the
// gfx950 form of overlapping data movement with compute ("FlashAttention 3
// and 4: When the Bottleneck Moves", section 2.1). The row
// maximum used by the exponentials is refreshed only when it grows by more
// than TAU doublings (same page, section 3.2).
//
// Work split and overlap. 8 waves, two per SIMD, each owning 32 query rows
// (BLOCK_M 256); key tiles of BLOCK_N 64. Every wave runs the same sequence
//     S(0) sm(0) | PV(0) S(1) | sm(1) | PV(1) S(2) | sm(2) ... sm(n-1) PV(n-1)
// (S = K Q^T and PV = V^T P^T on the matrix cores, sm = softmax on the vector
// ALU), with one workgroup barrier per key tile. Waves 0-3 (group A) meet the
// barrier between sm(j-1) and their matrix block [PV(j-1) S(j)], waves 4-7
// (group B) before sm(j-1). A SIMD hosts one wave of each group, so after
// every barrier one of its waves feeds the matrix core while the other runs
// the exponentials: the pages' "two tiles, two engines" overlap (section
// 2.1), arranged by the barrier placement instead of warp specialisation.
//
// Products. S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16}: the 32x32
// accumulator gives every lane one query column and 16 keys, so the softmax
// row reductions are in-lane plus one exchange with lane ^ 32. The same
// registers, rounded to 16 bits, are the B operand of O^T += V^T P^T; the key
// order inside an MFMA K-step is the accumulator's row order, and the V^T
// operand is gathered in exactly that order by ds_read_b64_tr_b16 from the
// row-major V tile, so P never moves between lanes.
//
// LDS layout. K and V tiles are stored row-major with their 16-byte chunks
// XOR-swizzled per row, which keeps both the direct-to-LDS writes (1 KB of
// consecutive LDS per wave instruction) and the MFMA operand reads free of
// bank conflicts.
#include <type_traits>

#include "device.h"
#include "mfma16.h"
#include "tile_io.h"

namespace exattn {
namespace {

constexpr int BLOCK_M = 256;
constexpr int BLOCK_N = 64;
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int ROWS_PER_WAVE = BLOCK_M / NWAVES;  // 32: one MFMA column block

template <int DQK, int DV, bool CAUSAL, int TAU, bool F16, bool STRIDED>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const FwdParams p) {
  static_assert(DQK == 64 || DQK == 128 || DQK == 192, "d_qk");
  static_assert(DV == 64 || DV == 128, "d_v");
  typedef Elem<F16> E;
  constexpr int KS = DQK / 16;             // MFMA K-steps of S^T
  constexpr int DB = DV / 32;              // 32-row blocks of O^T
  // K tile: part A holds dims [0, min(DQK,128)), part B (DQK = 192) dims [128, 192).
  constexpr int KA_D = DQK > 128 ? 128 : DQK;
  constexpr int KB_D = DQK - KA_D;
  constexpr bool KA_W16 = KA_D == 128;
  constexpr int KA_ROW = KA_D * 2;         // bytes
  constexpr int KB_ROW = 128;
  constexpr int KA_BYTES = BLOCK_N * KA_ROW;
  constexpr int KB_BYTES = BLOCK_N * KB_D * 2;
  constexpr int K_STAGE = KA_BYTES + KB_BYTES;
  constexpr bool V_W16 = DV == 128;
  constexpr int V_ROW = DV * 2;
  constexpr int V_STAGE = BLOCK_N * V_ROW;
  constexpr int KA_INSTR = KA_BYTES / 1024;  // wave-wide 1 KB direct loads per tile
  constexpr int KB_INSTR = KB_BYTES / 1024;
  constexpr int V_INSTR = V_STAGE / 1024;

  // Three-stage rings: iteration j reads K(j) and V(j-1) while K(j+1), V(j) (issued
  // one iteration earlier) and K(j+2), V(j+1) (issued after its barrier) land.
  constexpr int NSTAGE = 3;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * (K_STAGE + V_STAGE)];
  lds_u8* const k_lds = (lds_u8*)smem;
  lds_u8* const v_lds = (lds_u8*)smem + NSTAGE * K_STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const bool group_b = wave >= NWAVES / 2;

  const int BH = p.B * p.H;
  int bh, qt;
  map_block(blockIdx.x, p.n_qtiles, BH, CAUSAL, bh, qt);
  const int q0 = qt * BLOCK_M;
  const int offset = p.Nkv - p.Nq;  // causal: key j visible to query i iff j <= i + offset

  // Dense BHND, or (STRIDED) element strides along batch, head and row with a dense
  // last dimension. Bytes per row of each tensor:
  const int q_row = STRIDED ? p.q_sn * 2 : DQK * 2;
  const int k_row = STRIDED ? p.k_sn * 2 : DQK * 2;
  const int v_row = STRIDED ? p.v_sn * 2 : DV * 2;
  const int b_ = bh / p.H, h_ = bh - b_ * p.H;
  auto base = [&](const void* t, long long sb, long long sh, int rows, int d) {
    return (const uint8_t*)t + (STRIDED ? (b_ * sb + h_ * sh) * 2 : (size_t)bh * rows * d * 2);
  };
  const uint8_t* __restrict__ qg = base(p.q, p.q_sb, p.q_sh, p.Nq, DQK);
  const uint8_t* __restrict__ kg = base(p.k, p.k_sb, p.k_sh, p.Nkv, DQK);
  const uint8_t* __restrict__ vg = base(p.v, p.v_sb, p.v_sh, p.Nkv, DV);

  int kv_end = p.Nkv;
  if (CAUSAL) kv_end = min(p.Nkv, max(0, q0 + BLOCK_M + offset));
  const int ntiles = (kv_end + BLOCK_N - 1) / BLOCK_N;

  // ---- Q^T fragments (B operand of S^T): lane = query column, 8 consecutive dims.
  const int wq0 = q0 + wave * ROWS_PER_WAVE;
  const int my_q = wq0 + l32;
  u32x4_t qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (my_q < p.Nq) x = *(const u32x4_t*)(qg + (size_t)my_q * q_row + s * 32 + half * 16);
    qf[s] = x;
  }

  // ---- Direct-to-LDS tile loads. Wave instruction i fills LDS bytes [1024 i, 1024 i + 1024)
  // of a ring stage; lane l writes the 16 bytes at 1024 i + 16 l, so each lane loads the
  // global chunk that belongs at that swizzled position. The buffer resource of a tile
  // starts at its first key and ends at N_kv: rows past the end read as zeros. Per-lane
  // offsets do not depend on the tile.
  static_assert(KA_INSTR % NWAVES == 0 && KB_INSTR % NWAVES == 0 && V_INSTR % NWAVES == 0,
                "every wave issues the same number of tile loads");
  constexpr int KA_PER = KA_INSTR / NWAVES;
  constexpr int KB_PER = KB_INSTR / NWAVES;
  constexpr int V_PER = V_INSTR / NWAVES;
  constexpr int LOADS_PER_TILE = KA_PER + KB_PER + V_PER;  // per thread: K(j) + V(j - 1)
  int ka_off[KA_PER], kb_off[KB_PER > 0 ? KB_PER : 1], v_off[V_PER];
#pragma unroll
  for (int t = 0; t < KA_PER; ++t) {
    constexpr int rows_per = 1024 / KA_ROW, cpr = KA_ROW / 16;
    const int i = wave + t * NWAVES;
    const int r = i * rows_per + lane / cpr;
    ka_off[t] = r * k_row + k_swz(lane % cpr, r, KA_W16) * 16;
  }
#pragma unroll
  for (int t = 0; t < KB_PER; ++t) {
    const int i = wave + t * NWAVES;
    const int r = i * 8 + lane / 8;
    kb_off[t] = r * k_row + KA_ROW + k_swz(lane % 8, r, false) * 16;
  }
#pragma unroll
  for (int t = 0; t < V_PER; ++t) {
    constexpr int rows_per = 1024 / V_ROW, cpr = V_ROW / 16;
    const int i = wave + t * NWAVES;
    const int r = i * rows_per + lane / cpr;
    v_off[t] = r * v_row + v_swz(lane % cpr, r, V_W16) * 16;
  }
  // Tiles past the last one (j >= ntiles: past N_kv, or past the causal diagonal of
  // the query tile) are still "loaded" through an empty resource (every lane reads
  // zero bytes and no memory is touched), which keeps the number of loads in flight
  // the same at every barrier; the stages they fill are not read again.
  // `stage` is an int or a std::integral_constant; with the latter every LDS address
  // below is a per-lane register plus an immediate offset.
  auto tile_rsrc = [&](const uint8_t* g, int j, int row) {
    const int key0 = min(j * BLOCK_N, p.Nkv);
    const unsigned bytes = j < ntiles ? (unsigned)(p.Nkv - key0) * (unsigned)row : 0u;
    return make_rsrc(g + (size_t)key0 * row, bytes);
  };
  auto issue_k = [&](int j, auto stage) {
    const i32x4_t rs = tile_rsrc(kg, j, k_row);
    lds_u8* st = k_lds + int(stage) * K_STAGE;
#pragma unroll
    for (int t = 0; t < KA_PER; ++t) buffer_load_lds16(rs, st + (wave + t * NWAVES) * 1024, ka_off[t]);
#pragma unroll
    for (int t = 0; t < KB_PER; ++t)
      buffer_load_lds16(rs, st + KA_BYTES + (wave + t * NWAVES) * 1024, kb_off[t]);
  };
  auto issue_v = [&](int j, auto stage) {
    const i32x4_t rs = tile_rsrc(vg, j, v_row);
    lds_u8* st = v_lds + int(stage) * V_STAGE;
#pragma unroll
    for (int t = 0; t < V_PER; ++t) buffer_load_lds16(rs, st + (wave + t * NWAVES) * 1024, v_off[t]);
  };

  // ---- Per-lane LDS read offsets within a stage.
  // K operand of S^T: lane reads row 32 kb + l32, chunk 2 s + half.
  int koff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int c = 2 * s + half;
    if (c < KA_D / 8) {
      koff[s] = l32 * KA_ROW + k_swz(c, l32, KA_W16) * 16;
    } else {
      koff[s] = KA_BYTES + l32 * KB_ROW + k_swz(c - KA_D / 8, l32, false) * 16;
    }
  }
  // V^T operand of O^T: for 16-key step ks and half h8 (keys +0 / +8), lane j of its
  // 16-lane group reads row 16 ks + 8 h8 + 4 half + j/4, columns 32 db + 16 g16 + 4 (j%4).
  int voff[DB];
  {
    const int j = lane & 15, g16 = (lane >> 4) & 1;
    const int rl = 4 * half + (j >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = 4 * db + 2 * g16 + ((j & 3) >> 1);
      // Absolute LDS address of the lane's chunk in stage 0, kept opaque to the compiler:
      // folded into the immediate offset of each read, the V ring base (past the K ring)
      // plus a stage offset would exceed the 16-bit field and cost an add per read.
      voff[db] = (int)(unsigned)(uintptr_t)v_lds + rl * V_ROW + v_swz(c, rl, V_W16) * 16 + 8 * (j & 1);
      asm volatile("" : "+v"(voff[db]));
    }
  }

  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  f32x16_t sacc[2];          // S^T of a tile between its S and softmax phases
  u32x4_t pf[4];             // P^T B operands of a tile between its softmax and PV phases
  float m_ref = -INFINITY;   // running reference max, log2 units
  float l_part = 0.f;        // this lane's partial row sum
  float tile_alpha = 1.f;    // a tile's re-base factor of O, applied in its PV phase
  bool tile_rebased = false; // some row of the wave re-based in the tile's softmax
  const float c = p.scale_log2;

  // S(j): S^T = K_j Q^T into sacc. Operands are read one K-step ahead of the products;
  // the scheduling fences keep the compiler from hoisting every read above the first
  // product (16 live fragments). The first K-step's fragments come in as arguments: in
  // the unrolled loop they are read during the last products of the PV phase before
  // (K(j) is already in LDS then), so the S phase does not open with a full LDS
  // latency in which the SIMD's other wave is in its softmax (+0.6 % measured).
  auto kread = [&](auto stage, int s_, int kb) {
    const lds_u8* st = k_lds + int(stage) * K_STAGE;
    const int rows = (2 * s_ + half < KA_D / 8) ? kb * 32 * KA_ROW : kb * 32 * KB_ROW;
    return lds_read128(st + koff[s_] + rows);
  };
  u32x4_t kpre0, kpre1;  // K-step 0 of the next S phase, read during the PV phase
  auto s_phase_from = [&](auto stage, u32x4_t kf0, u32x4_t kf1) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t nf0 = kf0, nf1 = kf1;
      if (s + 1 < KS) {
        nf0 = kread(stage, s + 1, 0);
        nf1 = kread(stage, s + 1, 1);
      }
      sacc[0] = E::mfma(kf0, qf[s], sacc[0]);
      sacc[1] = E::mfma(kf1, qf[s], sacc[1]);
      __builtin_amdgcn_sched_barrier(0);
      kf0 = nf0;
      kf1 = nf1;
    }
  };
  auto s_phase = [&](auto stage) { s_phase_from(stage, kread(stage, 0, 0), kread(stage, 0, 1)); };

  // PV(j): O^T += V_j^T P_j^T from pf. A transposing LDS read takes longer than one
  // product, so operands are read PV_AHEAD products ahead (the S accumulators are dead
  // here, which leaves room for the extra fragments). A re-base in the tile's softmax
  // reaches O here, before the first product, behind a wave-uniform branch. The same
  // multiplies inside the softmax's branch, where S (and at d_qk = 192 twelve Q
  // fragments) are live too, cost 56 more registers at d = 128 and made the compiler
  // spill 16-18 at d_qk = 192 (1.7 % slower on B1 H16 N8192 causal). `k_next` is the ring stage of the
  // next S phase's K tile (its first fragments go to kpre0/kpre1 near the end), or
  // std::false_type for none.
  constexpr int PV_STEPS = 4 * DB;
  constexpr int PV_AHEAD = 3;
  auto pv_phase = [&](auto stage, auto hook, auto k_next) {
    lds_u8* const lds0 = (lds_u8*)(uintptr_t)0;  // voff holds absolute LDS addresses
    const lds_u8* st = lds0 + int(stage) * V_STAGE;
    auto vread = [&](int step) {
      const int ks = step / DB, db = step % DB;
      const lds_u8* a = st + voff[db] + ks * 16 * V_ROW;
      const u32x2_t lo = lds_read_tr16(a);
      const u32x2_t hi = lds_read_tr16(a + 8 * V_ROW);
      return (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
    };
    if (__builtin_amdgcn_readfirstlane((int)tile_rebased)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= tile_alpha;
    }
    u32x4_t vf[PV_AHEAD];
#pragma unroll
    for (int i = 0; i < PV_AHEAD; ++i) vf[i] = vread(i);
#pragma unroll
    for (int step = 0; step < PV_STEPS; ++step) {
      const u32x4_t cur = vf[step % PV_AHEAD];
      if (step + PV_AHEAD < PV_STEPS) vf[step % PV_AHEAD] = vread(step + PV_AHEAD);
      oacc[step % DB] = E::mfma(cur, pf[step / DB], oacc[step % DB]);
      hook(step);
      if constexpr (!std::is_same_v<decltype(k_next), std::false_type>) {
        if (step == PV_STEPS - 3) {
          kpre0 = kread(k_next, 0, 0);
          kpre1 = kread(k_next, 0, 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  constexpr std::false_type NO_K{};
  auto no_hook = [](int) {};

  // sm(j): masking (MASK: a key of the tile is past N_kv or past this wave's diagonal),
  // row max, conditional rescale, exponentials, row sum; sacc -> pf.
  auto softmax = [&](int j, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    tile_rebased = false;
    // Row r of key block kb is key j*BLOCK_N + kb*32 + 8*(r>>2) + 4*half + (r&3); it is
    // visible iff its tile-local offset kb*32 + 8*(r>>2) + (r&3) (a constant) is at most
    // `room`. Comparing constants against one per-tile value keeps the mask from
    // holding 32 per-lane offsets in registers.
    int room = 0;
    auto visible = [&](int kb, int r) { return kb * 32 + (r >> 2) * 8 + (r & 3) <= room; };
    if constexpr (MASK) {
      const int limit = CAUSAL ? min(p.Nkv - 1, my_q + offset) : p.Nkv - 1;
      room = limit - j * BLOCK_N - half * 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!visible(kb, r)) sacc[kb][r] = -INFINITY;
    }
    // Exponentials against the current reference into pf (rounded to 16 bits); returns
    // the lane's float32 sum of them.
    auto exps = [&](float nm) {
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c, nm));
          if constexpr (MASK) e = visible(kb, r) ? e : 0.f;
          pv[r] = e;
          ps += e;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          u32x4_t w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = E::pack2(pv[h * 8 + 2 * i], pv[h * 8 + 2 * i + 1]);
          pf[kb * 2 + h] = w;
        }
      }
      return ps;
    };
    // Row max and the re-base of the running state when it grew by more than TAU
    // doublings (l here, O in the PV phase); true when any row of the wave re-based
    // (wave-uniform).
    auto rebase = [&]() {
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = max_halves(mx);
      const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
      const bool grow = mt > m_ref + (float)TAU;
      if (!__any(grow)) return false;
      // only rows past the threshold re-base
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - mt) : 1.f;
      m_ref = grow ? mt : m_ref;
      l_part *= alpha;
      tile_alpha = alpha;
      tile_rebased = true;
      return true;
    };
    auto neg_ref = [&]() { return m_ref == -INFINITY ? 0.f : -m_ref; };
    float psum;
    if constexpr (DQK > 128) {
      // d_qk = 192 has no registers to keep S past its exponentials: max first.
      rebase();
      psum = exps(neg_ref());
    } else {
      // The row max decides the rescale: the reference moves when a score exceeds it
      // by more than TAU doublings, i.e. when some p = 2^(c s - m_ref) exceeds 2^TAU. A
      // lane whose p sum to less than 2^TAU has no such p (a float sum of non-negative
      // terms is at least each term), so the max is needed only where the sum reaches
      // 2^TAU or no reference exists yet; the decisions, and so the results, are those
      // of the max test.
      psum = exps(neg_ref());
      if (__any(!(psum < (float)(1 << TAU)) || m_ref == -INFINITY))
        if (rebase()) psum = exps(neg_ref());
    }
    l_part += psum;
  };

  // Tiles [0, j_plain) need no mask for any wave of the workgroup; a tile that starts
  // after this wave's last visible key (causal) is skipped by the wave. For causal
  // problems every wave still sees tile j_plain.
  int j_plain = min(ntiles, p.Nkv / BLOCK_N);
  if (CAUSAL) j_plain = min(j_plain, max(0, (q0 + offset + 1) / BLOCK_N));
  const int wave_last_key = wq0 + ROWS_PER_WAVE - 1 + offset;
  auto active = [&](int j) { return !CAUSAL || j * BLOCK_N <= wave_last_key; };
  // Tile j needs no mask for this wave: its keys exist and every row of the wave sees them.
  auto wave_plain = [&](int j) {
    return j < j_plain || (j + 1) * BLOCK_N <= (CAUSAL ? min(p.Nkv, wq0 + offset + 1) : p.Nkv);
  };
  constexpr std::false_type PLAIN{};
  constexpr std::true_type MASKED{};

  // Barrier j needs K(j) and V(j-1) and lets the loads issued after barrier j-1, K(j+1)
  // and V(j), stay in flight; after it the wave issues K(j+2) and V(j+1). Every
  // wave runs sm(j-1) PV(j-1) S(j) per iteration; group B meets barrier j before its
  // softmax, group A after it, so group A's matrix block follows the barrier while
  // group B computes exponentials, and the other way round before the next barrier.
  // Compiler-only fences (no instructions): a value "modified" by an empty volatile asm
  // must be complete before it and cannot be computed earlier than it. They pin the
  // softmax to its side of the barrier, which the compiler would otherwise move
  // (exponentials sunk next to the PV products, the row max hoisted above the barrier),
  // putting both wave groups in the same phase.
  auto pin_s = [&]() {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) asm volatile("" : "+v"(sacc[kb]));
  };
  auto pin_p = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(pf[i]));
  };
  auto barrier_and_issue = [&](int j, auto k_next, auto v_next) {
    tile_barrier<LOADS_PER_TILE>();
    issue_k(j + 2, k_next);
    issue_v(j + 1, v_next);
  };
  // The tile loads of an unrolled iteration are spread over its PV products, one every
  // ISSUE_GAP products, instead of all eight waves issuing theirs right after the
  // barrier: the burst (32 KB per workgroup at d = 128) queues in the vector memory
  // pipeline and stalls the waves behind it.
  constexpr int ISSUE_GAP = PV_STEPS / LOADS_PER_TILE;
  static_assert(ISSUE_GAP >= 1, "one load per PV product at most");
  auto spread_issue = [&](int j, auto k_next, auto v_next) {
    const i32x4_t krs = tile_rsrc(kg, j + 2, k_row);
    const i32x4_t vrs = tile_rsrc(vg, j + 1, v_row);
    lds_u8* kst = k_lds + int(k_next) * K_STAGE;
    lds_u8* vst = v_lds + int(v_next) * V_STAGE;
    return [=](int step) {
      if (step % ISSUE_GAP != 0) return;
      const int li = step / ISSUE_GAP;
      if (li < KA_PER) {
        buffer_load_lds16(krs, kst + (wave + li * NWAVES) * 1024, ka_off[li]);
      } else if (li < KA_PER + KB_PER) {
        const int t = li - KA_PER;
        buffer_load_lds16(krs, kst + KA_BYTES + (wave + t * NWAVES) * 1024, kb_off[t]);
      } else if (li < LOADS_PER_TILE) {
        const int t = li - KA_PER - KB_PER;
        buffer_load_lds16(vrs, vst + (wave + t * NWAVES) * 1024, v_off[t]);
      }
    };
  };
  // Iteration j with ring stages known at compile time, R = j % 3: K(j) in stage R,
  // V(j-1) in stage (R+2) % 3; K(j+2) goes to stage (R+2) % 3, V(j+1) to (R+1) % 3.
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
    pv_phase(v_prev, spread_issue(j, k_next, v_next), k_cur);
    s_phase_from(k_cur, kpre0, kpre1);
  };
  // The same with stages computed at run time (tiles that need masking, and the few
  // iterations that do not fill a group of three).
  auto any_iter = [&](int j) {
    const int r = j % NSTAGE;
    if (group_b) {
      barrier_and_issue(j, (r + 2) % NSTAGE, (r + 1) % NSTAGE);
      pin_s();
    }
    if (active(j - 1)) {
      if (wave_plain(j - 1)) softmax(j - 1, PLAIN); else softmax(j - 1, MASKED);
    }
    if (!group_b) {
      pin_p();
      barrier_and_issue(j, (r + 2) % NSTAGE, (r + 1) % NSTAGE);
    }
    if (active(j - 1)) pv_phase((r + 2) % NSTAGE, no_hook, NO_K);
    if (active(j)) s_phase(r);
  };
  if (ntiles > 0) {
    issue_k(0, 0);
    issue_k(1, 1);
    issue_v(0, 0);
    tile_barrier<LOADS_PER_TILE>();
    // The compiler waits for the Q fragments at their first use, and since it does not
    // see the tile loads it waits for every load (vmcnt(0)). Touching the fragments
    // here, before K(2) and V(1) are issued, keeps that wait from covering those two.
    // A negative scale is applied here as -Q (sign bits only, exact) with |scale| in c.
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      asm volatile("" : "+v"(qf[s]));
      qf[s] ^= p.q_neg;
    }
    issue_k(2, 2);
    issue_v(1, 1);
    if (active(0)) s_phase(0);
    // Iterations j <= j_plain have a plain softmax and every wave active.
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
      if (wave_plain(ntiles - 1)) softmax(ntiles - 1, PLAIN); else softmax(ntiles - 1, MASKED);
    }
    if (!group_b) tile_barrier<LOADS_PER_TILE>();
    if (active(ntiles - 1)) pv_phase((ntiles - 1) % NSTAGE, no_hook, NO_K);
  }

  __builtin_amdgcn_s_waitcnt(0x0070);  // no LDS fill may be in flight when the waves end

  // ---- Epilogue: O = acc / l, LSE = ln2 * (m + log2 l). The lane's query and half are
  // recomputed from the lane id (mbcnt) rather than kept in registers through the loop.
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int my_q_e = wq0 + (lane_e & 31), half_e = lane_e >> 5;
  const float l = sum_halves(l_part);
  const bool any = l > 0.f;
  const float inv = any ? __builtin_amdgcn_rcpf(l) : 0.f;
  // O leaves through LDS as whole rows (stage_rows / store_rows); the barrier orders the
  // staging writes after every wave's last ring read and fill (each wave has waited for
  // its own fills above).
  static_assert(NWAVES * ROWS_PER_WAVE * staged_row_bytes<DV>() <= NSTAGE * (K_STAGE + V_STAGE),
                "O staging fits in the rings");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  lds_u8* const ot = (lds_u8*)smem + wave * ROWS_PER_WAVE * staged_row_bytes<DV>();
  stage_rows<DV, E>(ot, oacc, inv, lane_e);
  uint8_t* const obase = STRIDED ? (uint8_t*)p.o + (b_ * p.o_sb + h_ * p.o_sh) * 2
                                 : (uint8_t*)p.o + (size_t)bh * p.Nq * DV * 2;
  store_rows<DV>(obase, STRIDED ? (size_t)p.o_sn * 2 : (size_t)DV * 2, ot, wq0, p.Nq, lane_e);
  if (my_q_e < p.Nq && half_e == 0)
    p.lse[(size_t)bh * p.Nq + my_q_e] =
        any ? 0.69314718055994531f * (m_ref + __builtin_amdgcn_logf(l)) : -INFINITY;
}

// Dense BHND tensors run the kernel with compile-time row sizes; other strides (only
// with the default rescale threshold) run the STRIDED instance.
bool is_dense(const FwdParams& p, int dqk, int dv) {
  const long long rq = p.Nq, rk = p.Nkv;
  return p.q_sn == dqk && p.k_sn == dqk && p.v_sn == dv && p.o_sn == dv && p.q_sh == rq * dqk &&
         p.k_sh == rk * dqk && p.v_sh == rk * dv && p.o_sh == rq * dv &&
         p.q_sb == p.H * rq * dqk && p.k_sb == p.H * rk * dqk && p.v_sb == p.H * rk * dv &&
         p.o_sb == p.H * rq * dv;
}

template <int DQK, int DV, bool CAUSAL, int TAU, bool F16>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int grid = p.n_qtiles * p.B * p.H;
  if (is_dense(p, DQK, DV)) {
    hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, CAUSAL, TAU, F16, false>), dim3(grid),
                       dim3(NTHREADS), 0, stream, p);
  } else if constexpr (TAU == 8) {
    hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, CAUSAL, TAU, F16, true>), dim3(grid),
                       dim3(NTHREADS), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
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
