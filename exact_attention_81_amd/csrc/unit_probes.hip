// Unit-rate probes for gfx950 that the attention kernels' design rests on (a separate
// library, libexattn_probes.so; nothing in libexattn.so calls it):
//
//  * exp_fma: independent chains of v_exp_f32 and of unpacked v_fma_f32, issued in a
//    fixed interleaved order by one or two waves per SIMD. It tells whether the
//    hardware exponential runs beside the FMAs (then moving exponentials onto FMAs,
//    "FlashAttention 3 and 4: When the Bottleneck Moves" section 3.2, could pay) or
//    shares their issue (then it cannot).
//  * lds: LDS read throughput per compute unit for ds_read_b128 and the transposing
//    ds_read_b64_tr_b16, alone and with a stream of v_mfma_f32_32x32x16_bf16 in the same
//    wave, at one and two waves per SIMD: how fast one wave can feed its matrix core
//    from LDS.
//  * mfma_clock: a sustained stream of v_mfma_f32_32x32x16_bf16 (or of the e4m3
//    v_mfma_f32_32x32x64_f8f6f4) on every SIMD (two waves each, four independent
//    accumulators per wave), with operands that are constant or pseudo-random (four different operand registers in turn, so the
//    bits on the matrix core's inputs change from product to product as with real
//    data): the matrix rate and the shader clock the chip holds under that load.
//  * stream_read: HBM read bandwidth of a plain streaming kernel (16-byte loads over a
//    1 GiB buffer, grid-stride, a given number of loads in flight per thread and
//    workgroups per CU), the reference for kernels bound by their reads, such as the
//    split-KV decode.
//
// Every probe runs one workgroup per compute unit. Each wave stamps the start and end
// of its loop with the shader clock (s_memtime) and the 100 MHz real-time counter
// (s_memrealtime); a workgroup's time is the span from its first wave's start to its
// last wave's end (waves that share a SIMD need not finish together: the oldest may
// run ahead), averaged over all workgroups.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

namespace probes {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) unsigned char lds_b;

constexpr int kExpFmaIter = 4096;
constexpr int kLdsIter = 2048;
constexpr int kMaxThreads = 512;
constexpr int kPadFloats = 24576;  // 96 KB

// Lane 0 of every wave writes its loop's start and end stamps: 4 values per wave,
// kMaxThreads / 64 wave slots per workgroup.
__device__ inline void stamp(long long* clk, long long t0, long long t1, long long w0, long long w1) {
  if ((threadIdx.x & 63) == 0) {
    long long* c = clk + ((size_t)blockIdx.x * (kMaxThreads / 64) + threadIdx.x / 64) * 4;
    c[0] = t0;
    c[1] = t1;
    c[2] = w0;
    c[3] = w1;
  }
}

// NE exponential chains and NF FMA chains per lane; the volatile asm statements keep
// the issue order fixed: exponential i sits at slot round(i (NE + NF) / NE).
template <int NE, int NF>
__global__ __launch_bounds__(512) void exp_fma_kernel(float* out, float a, float b,
                                                      long long* clk) {
  float e[NE > 0 ? NE : 1], f[NF > 0 ? NF : 1];
#pragma unroll
  for (int i = 0; i < NE; ++i) e[i] = 0.5f + 0.001f * i + 0.0001f * threadIdx.x;
#pragma unroll
  for (int i = 0; i < NF; ++i) f[i] = 0.5f - 0.001f * i + 0.0001f * threadIdx.x;
  const long long t0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < kExpFmaIter; ++it) {
    constexpr int N = NE + NF;
    int ie = 0, jf = 0;
#pragma unroll
    for (int s = 0; s < N; ++s) {
      const bool do_exp = NE > 0 && ie < NE && (NF == 0 || s * NE >= ie * N);
      if (do_exp) {
        asm volatile("v_exp_f32 %0, %0" : "+v"(e[ie]));
        ++ie;
      } else if (jf < NF) {
        asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(f[jf]) : "v"(a), "v"(b));
        ++jf;
      }
    }
  }
  const long long t1 = clock64(), w1 = wall_clock64();
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NE; ++i) sum += e[i];
#pragma unroll
  for (int i = 0; i < NF; ++i) sum += f[i];
  // 96 KB of LDS per workgroup: no compute unit can hold two of them.
  __shared__ float pad[kPadFloats];
  pad[(threadIdx.x * 48) % kPadFloats] = sum;
  __syncthreads();
  out[blockIdx.x * blockDim.x + threadIdx.x] = pad[(threadIdx.x * 48 + 48) % kPadFloats];
  stamp(clk, t0, t1, w0, w1);
}

// MODE 0: ds_read_b128; 1: two ds_read_b64_tr_b16 per step; 2: MFMA only;
// 3: MFMA + ds_read_b128; 4: MFMA + two tr reads. 8 steps per iteration; every read
// stays inside the 64 KB the workgroup holds, conflict-free within a wave. In modes
// 0-4 an iteration's reads are consumed in the same iteration (the loop drains them
// at its end); modes 5 and 6 keep reads in flight across iterations:
// 5: ds_read_b128 through a ring of 8 registers (a read is consumed 8 reads after its
//    issue); 6: MFMA whose A operand is the ds_read_b128 issued 4 products earlier.
template <int MODE>
__global__ __launch_bounds__(512) void lds_kernel(unsigned* out, long long* clk) {
  // 96 KB (one workgroup per compute unit); the loop reads the first 64 KB.
  __shared__ __attribute__((aligned(16))) unsigned char lds[98304];
  const int t = threadIdx.x;
  for (int i = t; i < 65536 / 4; i += blockDim.x) ((unsigned*)lds)[i] = i * 2654435761u;
  __syncthreads();
  const int lane = t & 63, wave = t >> 6;
  const unsigned base = (wave * 4096 + lane * 16) & 0xFFFF;
  u32x4_t acc = {0, 0, 0, 0};
  f32x16_t c0 = {}, c1 = {};
  const u32x4_t a = {(unsigned)t, 1u, 2u, 3u};
  lds_b* const lds0 = (lds_b*)0;
  auto rd = [&](unsigned addr) { return *(const __attribute__((address_space(3))) u32x4_t*)(lds0 + addr); };
  auto step_addr = [&](int it, int u) { return (base + u * 1024 + (it & 7) * 8192) & 0xFFF0; };
  u32x4_t ring[8];
  if constexpr (MODE == 5 || MODE == 6) {
#pragma unroll
    for (int u = 0; u < 8; ++u) ring[u] = rd(step_addr(0, u));
  }
  const long long t0 = clock64(), w0 = wall_clock64();
  if constexpr (MODE == 5) {
    for (int it = 1; it <= kLdsIter; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc ^= ring[u];
        ring[u] = rd(step_addr(it, u));
        __builtin_amdgcn_sched_barrier(0);  // keep the program order: 8 reads in flight
      }
    }
  }
  if constexpr (MODE == 6) {
    for (int it = 1; it <= kLdsIter; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const u32x4_t op = ring[u & 3];
        ring[u & 3] = rd(step_addr(it, u));
        if (u & 1)
          c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, op),
                                                       __builtin_bit_cast(bf16x8_t, a), c1, 0, 0, 0);
        else
          c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, op),
                                                       __builtin_bit_cast(bf16x8_t, a), c0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);  // keep the program order: reads 4 products ahead
      }
    }
  }
  for (int it = 0; it < (MODE <= 4 ? kLdsIter : 0); ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const unsigned addr = (base + u * 1024 + (it & 7) * 8192) & 0xFFF0;
      if constexpr (MODE == 0 || MODE == 3) {
        acc ^= *(const __attribute__((address_space(3))) u32x4_t*)(lds0 + addr);
      }
      if constexpr (MODE == 1 || MODE == 4) {
        const unsigned a2 = addr & 0xFFF8;
        const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(lds0 + a2));
        const i16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(lds0 + (a2 ^ 2048)));
        acc[0] ^= (unsigned)(__builtin_bit_cast(unsigned long long, v1) & 0xFFFFFFFFu);
        acc[1] ^= (unsigned)(__builtin_bit_cast(unsigned long long, v2) >> 32);
      }
      if constexpr (MODE >= 2) {
        if (u & 1)
          c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, a), c1, 0, 0, 0);
        else
          c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, a), c0, 0, 0, 0);
      }
    }
  }
  const long long t1 = clock64(), w1 = wall_clock64();
  float sum = 0.f;
  for (int r = 0; r < 16; ++r) sum += c0[r] + c1[r];
  if constexpr (MODE == 5 || MODE == 6) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= ring[u];
  }
  out[blockIdx.x * blockDim.x + t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3] ^ __float_as_uint(sum);
  stamp(clk, t0, t1, w0, w1);
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

// Launches `launch` twice (the first warms up) on `blocks` workgroups of `threads` and
// returns the mean span in shader cycles from a workgroup's first wave start to its
// last wave end, and the shader clock in GHz.
template <typename F>
int timed(F launch, int blocks, int threads, double* cycles, double* ghz) {
  if (threads <= 0 || threads > kMaxThreads || threads % 64) return -4;
  const int waves = threads / 64;
  const size_t nclk = (size_t)blocks * (kMaxThreads / 64) * 4;
  float* out = nullptr;
  long long* clk = nullptr;
  if (hipMalloc(&out, (size_t)blocks * threads * 4) != hipSuccess) return -1;
  if (hipMalloc(&clk, nclk * 8) != hipSuccess) {
    (void)hipFree(out);
    return -1;
  }
  int rc = 0;
  for (int rep = 0; rep < 2 && rc == 0; ++rep) {
    launch(out, clk);
    if (hipDeviceSynchronize() != hipSuccess) rc = -2;
  }
  std::vector<long long> h(nclk);
  if (rc == 0 && hipMemcpy(h.data(), clk, nclk * 8, hipMemcpyDeviceToHost) != hipSuccess) rc = -3;
  (void)hipFree(out);
  (void)hipFree(clk);
  if (rc) return rc;
  double c = 0, w = 0;
  for (int i = 0; i < blocks; ++i) {
    const long long* b = h.data() + (size_t)i * (kMaxThreads / 64) * 4;
    long long c0 = b[0], c1 = b[1], r0 = b[2], r1 = b[3];
    for (int v = 1; v < waves; ++v) {
      c0 = std::min(c0, b[4 * v]);
      c1 = std::max(c1, b[4 * v + 1]);
      r0 = std::min(r0, b[4 * v + 2]);
      r1 = std::max(r1, b[4 * v + 3]);
    }
    c += (double)(c1 - c0);
    w += (double)(r1 - r0);
  }
  *cycles = c / blocks;
  *ghz = (c / blocks) / ((w / blocks) * 10.0);  // wall_clock64 ticks at 100 MHz
  return 0;
}

template <int NE, int NF>
int run_exp_fma(int waves_per_simd, double* out3) {
  const int cus = device_cus();
  if (cus <= 0) return -1;
  const int threads = 256 * waves_per_simd;  // one workgroup per CU, waves_per_simd per SIMD
  double cyc = 0, ghz = 0;
  const int rc = timed([&](float* o, long long* clk) {
    hipLaunchKernelGGL((exp_fma_kernel<NE, NF>), dim3(cus), dim3(threads), 0, 0, o, 1.0001f, 0.001f, clk);
  }, cus, threads, &cyc, &ghz);
  if (rc) return rc;
  out3[0] = cyc / ((double)kExpFmaIter * (NE + NF) * waves_per_simd);  // cycles per wave instr per SIMD
  out3[1] = ghz;
  out3[2] = cyc;
  return 0;
}

template <int MODE>
int run_lds(int waves_per_simd, double* out3) {
  const int cus = device_cus();
  if (cus <= 0) return -1;
  const int threads = 256 * waves_per_simd;
  double cyc = 0, ghz = 0;
  const int rc = timed([&](float* o, long long* clk) {
    hipLaunchKernelGGL((lds_kernel<MODE>), dim3(cus), dim3(threads), 0, 0, (unsigned*)o, clk);
  }, cus, threads, &cyc, &ghz);
  if (rc) return rc;
  const double waves = threads / 64.0, steps = (double)kLdsIter * 8;
  out3[0] = (MODE == 2) ? 0.0 : steps * waves * 1024.0 / cyc;                  // LDS bytes/clk/CU
  constexpr bool kMfma = MODE == 2 || MODE == 3 || MODE == 4 || MODE == 6;
  out3[1] = kMfma ? cyc / (steps * waves_per_simd) : 0.0;                       // cycles per MFMA per SIMD
  out3[2] = ghz;
  return 0;
}

constexpr int kMfmaClockIter = 65536;  // 8 products each: about 17 M cycles per launch

// Two pseudo-random bf16 values in one word (finite, 2^-8 <= |x| < 1): an integer hash
// of the argument gives each half a sign, 7 mantissa bits and a biased exponent in
// 119..126.
__device__ inline unsigned rand_bf16x2(unsigned h) {
  h ^= h >> 16; h *= 0x7feb352dU; h ^= h >> 15; h *= 0x846ca68bU; h ^= h >> 16;
  const unsigned m = h & 0x807F807Fu;                         // sign, mantissa per half
  const unsigned e = ((h >> 8) & 0x00070007u) + 0x00770077u;  // biased exponents 119..126
  return m | (e << 7);
}

// Four pseudo-random e4m3 codes in one word: sign and 3 mantissa bits from the hash,
// exponent field 6 or 7 (values in [1/4, 1)), never a NaN code.
__device__ inline unsigned rand_e4m3x4(unsigned h) {
  h ^= h >> 16; h *= 0x7feb352dU; h ^= h >> 15; h *= 0x846ca68bU; h ^= h >> 16;
  return (h & 0x8F8F8F8Fu) | 0x30303030u;
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// FP8 false: v_mfma_f32_32x32x16_bf16; true: v_mfma_f32_32x32x64_f8f6f4 on e4m3 (half
// the iterations: each product takes twice the cycles).
template <bool RANDOM, bool FP8>
__global__ __launch_bounds__(512) void mfma_clock_kernel(float* out, long long* clk) {
  const unsigned t = threadIdx.x + blockIdx.x * blockDim.x;
  f32x16_t c[4] = {};
  long long t0, w0;
  if constexpr (!FP8) {
    u32x4_t a[4], b[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        a[k][w] = RANDOM ? rand_bf16x2(t * 32u + k * 8u + w) : 0x3F803F80u;      // 1.0
        b[k][w] = RANDOM ? rand_bf16x2(t * 32u + k * 8u + w + 4u) : 0x3F003F00u;  // 0.5
      }
    t0 = clock64(); w0 = wall_clock64();
    for (int it = 0; it < kMfmaClockIter; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        c[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[u & 3]),
                                                           __builtin_bit_cast(bf16x8_t, b[(u + 1) & 3]),
                                                           c[u & 3], 0, 0, 0);
    }
  } else {
    i32x8_t a[4], b[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        a[k][w] = (int)(RANDOM ? rand_e4m3x4(t * 64u + k * 16u + w) : 0x38383838u);      // 1.0
        b[k][w] = (int)(RANDOM ? rand_e4m3x4(t * 64u + k * 16u + w + 8u) : 0x30303030u);  // 0.5
      }
    t0 = clock64(); w0 = wall_clock64();
    for (int it = 0; it < kMfmaClockIter / 2; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        c[u & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[u & 3], b[(u + 1) & 3], c[u & 3],
                                                                   0, 0, 0, 0, 0, 0);
    }
  }
  const long long t1 = clock64(), w1 = wall_clock64();
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += c[k][r];
  out[t] = sum;
  stamp(clk, t0, t1, w0, w1);
}

// Every thread reads 16-byte chunks i = tid, tid + T, ... of the buffer (T threads in
// the grid), U chunks per loop iteration kept in flight, and folds them into one word
// so that no load can be dropped; the folded words go to `out`.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                          unsigned* __restrict__ out) {
  const size_t T = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * T < n16; i += U * T) {
    u32x4_t v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = src[i + k * T];
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= v[k];
  }
  for (; i < n16; i += T) acc ^= src[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

template <bool RANDOM, bool FP8>
int run_mfma_clock(double* out3) {
  const int cus = device_cus();
  if (cus <= 0) return -1;
  const int threads = 512;  // two waves per SIMD
  double cyc = 0, ghz = 0;
  // `timed` launches twice and keeps the second; four more launches first let the
  // clock settle under the load.
  for (int warm = 0; warm < 4; ++warm) {
    const int rc = timed([&](float* o, long long* clk) {
      hipLaunchKernelGGL((mfma_clock_kernel<RANDOM, FP8>), dim3(cus), dim3(threads), 0, 0, o, clk);
    }, cus, threads, &cyc, &ghz);
    if (rc) return rc;
  }
  const double products = (double)(FP8 ? kMfmaClockIter / 2 : kMfmaClockIter) * 8 * (threads / 64) * cus;
  const double seconds = cyc / (ghz * 1e9);
  out3[0] = products * 2.0 * 32 * 32 * (FP8 ? 64 : 16) / seconds / 1e12;  // TFLOP/s
  out3[1] = ghz;
  out3[2] = out3[0] / (cus * (FP8 ? 8192.0 : 4096.0) * ghz * 1e9 / 1e12);  // of the peak at that clock
  return 0;
}

template <int U>
int run_stream_read(int wg_per_cu, double* out3) {
  const int cus = device_cus();
  if (cus <= 0) return -1;
  constexpr size_t kBytes = size_t(1) << 30;
  const int blocks = cus * wg_per_cu;
  void* buf = nullptr;
  unsigned* out = nullptr;
  if (hipMalloc(&buf, kBytes) != hipSuccess) return -1;
  if (hipMalloc((void**)&out, (size_t)blocks * 256 * sizeof(unsigned)) != hipSuccess) {
    (void)hipFree(buf);
    return -1;
  }
  int rc = hipMemset(buf, 0x5a, kBytes) == hipSuccess ? 0 : -2;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (rc == 0 && (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess)) rc = -2;
  double best = 0, sum = 0;
  const int reps = 6;
  for (int r = 0; r < reps && rc == 0; ++r) {
    if (hipEventRecord(e0, 0) != hipSuccess) { rc = -2; break; }
    hipLaunchKernelGGL((stream_read_kernel<U>), dim3(blocks), dim3(256), 0, 0, (const u32x4_t*)buf, kBytes / 16, out);
    if (hipEventRecord(e1, 0) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) { rc = -2; break; }
    float ms = 0;
    if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0) { rc = -3; break; }
    const double gbs = (double)kBytes / (ms * 1e-3) / 1e9;
    if (r > 0) {  // the first run warms up
      best = std::max(best, gbs);
      sum += gbs;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(out);
  (void)hipFree(buf);
  if (rc) return rc;
  out3[0] = best;
  out3[1] = sum / (reps - 1);
  out3[2] = blocks;
  return 0;
}

}  // namespace probes

extern "C" {

// Cycles per wave instruction per SIMD (out[0]), shader clock in GHz (out[1]) and loop
// cycles (out[2]) for `ne` exponential and `nf` FMA chains per lane, interleaved, at
// `waves_per_simd` (1 or 2) waves per SIMD. Supported (ne, nf): (8,0) (0,8) (0,16) (8,8)
// (8,16) (8,24) (16,16). Returns 0, or a negative code (unsupported pair, HIP failure).
int probe_exp_fma(int ne, int nf, int waves_per_simd, double* out) {
  if (!out || waves_per_simd < 1 || waves_per_simd > 2) return -4;
  if (ne == 8 && nf == 0) return probes::run_exp_fma<8, 0>(waves_per_simd, out);
  if (ne == 0 && nf == 8) return probes::run_exp_fma<0, 8>(waves_per_simd, out);
  if (ne == 0 && nf == 16) return probes::run_exp_fma<0, 16>(waves_per_simd, out);
  if (ne == 8 && nf == 8) return probes::run_exp_fma<8, 8>(waves_per_simd, out);
  if (ne == 8 && nf == 16) return probes::run_exp_fma<8, 16>(waves_per_simd, out);
  if (ne == 8 && nf == 24) return probes::run_exp_fma<8, 24>(waves_per_simd, out);
  if (ne == 16 && nf == 16) return probes::run_exp_fma<16, 16>(waves_per_simd, out);
  return -4;
}

// LDS bytes per clock per CU (out[0]), cycles per MFMA per SIMD (out[1], MFMA modes) and
// the shader clock (out[2]) for `mode` (0: ds_read_b128, 1: ds_read_b64_tr_b16 pairs,
// 2: MFMA only, 3: MFMA + b128 read, 4: MFMA + tr pair, 5: b128 reads kept 8 in flight,
// 6: MFMA fed by the b128 read issued 4 products earlier) at 1 or 2 waves per SIMD.
int probe_lds(int mode, int waves_per_simd, double* out) {
  if (!out || waves_per_simd < 1 || waves_per_simd > 2) return -4;
  switch (mode) {
    case 0: return probes::run_lds<0>(waves_per_simd, out);
    case 1: return probes::run_lds<1>(waves_per_simd, out);
    case 2: return probes::run_lds<2>(waves_per_simd, out);
    case 3: return probes::run_lds<3>(waves_per_simd, out);
    case 4: return probes::run_lds<4>(waves_per_simd, out);
    case 5: return probes::run_lds<5>(waves_per_simd, out);
    case 6: return probes::run_lds<6>(waves_per_simd, out);
    default: return -4;
  }
}

// MFMA stream on every SIMD: TFLOP/s (out[0]), shader clock in GHz (out[1]) and the
// fraction of the peak at that clock (out[2]). `kind` 0: bf16 constant operands, 1: bf16
// pseudo-random operands, 2: e4m3 constant, 3: e4m3 pseudo-random.
int probe_mfma_clock(int kind, double* out) {
  if (!out) return -4;
  switch (kind) {
    case 0: return probes::run_mfma_clock<false, false>(out);
    case 1: return probes::run_mfma_clock<true, false>(out);
    case 2: return probes::run_mfma_clock<false, true>(out);
    case 3: return probes::run_mfma_clock<true, true>(out);
    default: return -4;
  }
}

// Read bandwidth in GB/s (best out[0], mean out[1] of five timed passes over 1 GiB) and
// the grid size (out[2]) of the streaming kernel with `wg_per_cu` workgroups of 256
// threads per CU (1..8) and `in_flight` 16-byte loads per thread per iteration (1, 4, 8).
int probe_stream_read(int wg_per_cu, int in_flight, double* out) {
  if (!out || wg_per_cu < 1 || wg_per_cu > 8) return -4;
  switch (in_flight) {
    case 1: return probes::run_stream_read<1>(wg_per_cu, out);
    case 4: return probes::run_stream_read<4>(wg_per_cu, out);
    case 8: return probes::run_stream_read<8>(wg_per_cu, out);
    default: return -4;
  }
}

}  // extern "C"
