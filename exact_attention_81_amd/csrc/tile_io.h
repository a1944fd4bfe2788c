// Direct-to-LDS tile loads and partial-wait barriers shared by the gfx950
// attention kernels.
#pragma once

#include "device.h"

namespace exattn {

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource word 3 for raw 32-bit-format buffers on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): stride 0, 32-bit data format. The
// record count is unsigned: one head's slice of a tensor below 2^31 elements of 2 bytes
// can span up to 2^32 - 2 bytes.
__device__ inline i32x4_t make_rsrc(const void* base, unsigned bytes) {
  const unsigned long long a = (unsigned long long)base;
  return (i32x4_t){(int)(unsigned)a, (int)((a >> 32) & 0xffffu), (int)bytes, kBufferFlags};
}

// 16 bytes per lane from `rsrc` at byte offset `voff` into LDS at dst + 16 * lane
// (buffer_load_dwordx4 ... lds, LDS base in m0); offsets at or past the resource
// size read as 0. Written as inline assembly so that the compiler does not track
// these LDS writes: it would otherwise wait for every one of them (vmcnt(0))
// before each ds_read_b64_tr_b16, which defeats loading tiles ahead. The waves
// wait for them explicitly in tile_barrier. No other code in these kernels uses m0.
__device__ inline void buffer_load_lds16(i32x4_t rsrc, lds_u8* dst, int voff) {
  const unsigned lds_addr = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are outstanding and
// its LDS operations are done, then meet the other waves. Unlike __syncthreads
// this leaves the newest N tile loads in flight.
template <int N>
__device__ inline void tile_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  // s_waitcnt: vmcnt[3:0] | expcnt[6:4] (7 = no wait) | lgkmcnt[11:8] | vmcnt[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline u32x4_t lds_read128(const lds_u8* p) {
  return *(const __attribute__((address_space(3))) u32x4_t*)p;
}

// A wave's 32-row result tile leaves the kernel through LDS as whole rows. In the 32x32
// MFMA accumulator layout (lane l: row l % 32; dims 8 g + 4 (l / 32) + 0..3 of each
// 32-dim block, g = 0..3) one store instruction would write 32 rows with 16 bytes each.
// stage_rows writes the tile times `sc`, rounded to 16 bits by E::pack2, into LDS rows of
// 2 D bytes; store_rows reads it back in 16-byte chunks and writes 64 * 16 / (2 D) whole
// rows per wave instruction: rows row0 .. row0 + 31 of a tensor at `base` with
// `row_bytes` between rows, skipping rows at or past `nrows`.
//
// Staged layout: in row r, 16-byte chunk c sits at chunk c ^ s(r), with its two 8-byte
// halves exchanged when bit 4 of r is set; s(r) = (r / RB) mod NCH, where RB rows span
// the 64 banks (256 bytes) and NCH is the number of chunks per row. The 32 lanes of either
// lane half then write distinct (chunk, half) slots of the banks, so each 8-byte write
// instruction covers all 64 banks once per 32 lanes, and 16 consecutive lanes of a read
// cover one 256-byte span.
template <int D>
constexpr int staged_row_bytes() {
  return D * 2;
}
template <int D>
__device__ inline int staged_swz(int r) {
  constexpr int RB = 256 / (D * 2), NCH = D / 8;
  return (r / RB) & (NCH - 1);
}

template <int D, typename E>
__device__ inline void stage_rows(lds_u8* dst, const f32x16_t (&acc)[D / 32], float sc, int lane) {
  static_assert(D == 64 || D == 128, "staged rows of 128 or 256 bytes");
  typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;
  const int row = lane & 31, half = lane >> 5;
  lds_u8* const rbase = dst + row * staged_row_bytes<D>() + 8 * (half ^ ((row >> 4) & 1));
  const int m = staged_swz<D>(row);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2_t w = {E::pack2(acc[db][g * 4 + 0] * sc, acc[db][g * 4 + 1] * sc),
                         E::pack2(acc[db][g * 4 + 2] * sc, acc[db][g * 4 + 3] * sc)};
      *(lds_u32x2*)(rbase + 16 * ((4 * db + g) ^ m)) = w;
    }
}

template <int D>
__device__ inline void store_rows(uint8_t* base, size_t row_bytes, const lds_u8* src, int row0,
                                  int nrows, int lane) {
  constexpr int CPR = D * 2 / 16, RPI = 64 / CPR;  // chunks per row, rows per instruction
  static_assert(16 % RPI == 0, "bit 4 of a staged row is the same across one instruction");
  const int r0 = lane / CPR, p = lane % CPR;  // row within the instruction, staged chunk
  u32x4_t x[32 / RPI];  // every read first, so that their latencies overlap
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) x[i] = lds_read128(src + (i * RPI + r0) * staged_row_bytes<D>() + p * 16);
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + r0;
    const bool swap = ((i * RPI) >> 4) & 1;  // bit 4 of r
    const u32x4_t v = swap ? (u32x4_t){x[i][2], x[i][3], x[i][0], x[i][1]} : x[i];
    if (row0 + r < nrows) *(u32x4_t*)(base + (size_t)(row0 + r) * row_bytes + 16 * (p ^ staged_swz<D>(r))) = v;
  }
}

}  // namespace exattn
