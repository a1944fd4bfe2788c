// Host-side launch interface of the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace exattn {

// Arguments of one attention-forward launch (16-bit or fp8 inputs).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;        // bf16/fp16: [B,H,N_kv,d_v]; fp8: transposed [B,H,d_v,N_kv]
  void* o;
  float* lse;
  const float* q_descale;  // fp8 only: [B,H,ceil(N/128)]
  const float* k_descale;
  const float* v_descale;
  int B, H, Nq, Nkv;
  float scale_log2;     // |softmax scale| * log2(e)
  unsigned q_neg;       // XOR mask for every 32-bit word of Q: the sign bits when scale < 0
  int n_qtiles;         // ceil(N_q / BLOCK_M)
  // 16-bit path: element strides of Q, K, V and O along batch, head and row (the last
  // dim is dense). Row strides times N are below 2^30, so byte offsets of rows fit in
  // 32 bits. The fp8 path reads dense BHND and ignores them.
  long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
  int q_sn, k_sn, v_sn, o_sn;
};

// Arguments of one split-KV decode launch (16-bit inputs, grouped KV heads).
struct DecodeParams {
  const void* q;        // [B, H, N_q, d]
  const void* k;        // [B, H_kv, N_kv, d]
  const void* v;        // [B, H_kv, N_kv, d]
  void* o;              // [B, H, N_q, d]
  float* lse;           // [B, H, N_q]
  float* o_part;        // splits > 1: [splits, B*H*N_q, d] fp32, O_s normalised by its own sum
  float* lse_part;      // splits > 1: [splits, B*H*N_q] fp32
  int B, H, Hkv, Nq, Nkv;
  float scale_log2;     // |softmax scale| * log2(e)
  unsigned q_neg;       // XOR mask for every 32-bit word of Q: the sign bits when scale < 0
  int splits;           // key ranges per (batch, KV head)
  int chunk;            // keys per range, a multiple of 32; splits * chunk >= N_kv
};

// Arguments of one attention backward (16-bit, dense BHND, d_qk = d_v).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;        // forward output
  const void* dout;     // gradient of the loss with respect to O
  const float* lse;     // forward LSE [B, H, N_q]
  void* dq;
  void* dk;
  void* dv;
  float* delta;         // [B, H, N_q]: D = rowsum(dO * O), written by the first kernel
  int B, H, Nq, Nkv;
  float scale;         // any finite value
  float scale_log2;     // scale * log2(e)
};

// Launchers (one per instantiation family); return hipError_t of the launch.
hipError_t launch_fwd16(const FwdParams& p, int d_qk, int d_v, bool causal, bool fp16,
                        int tau, hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdParams& p, bool causal, hipStream_t stream);
hipError_t launch_decode16(const DecodeParams& p, int d, bool causal, bool fp16,
                           hipStream_t stream);
hipError_t launch_bwd16(const BwdParams& p, int d, bool causal, bool fp16, hipStream_t stream);
// Decode workgroups the current device runs at once for head dim d (0 if unknown).
int decode_resident_workgroups(int d);
// The library's static decode scratch: its size, and its device address on the current
// device (looked up once per device with hipGetSymbolAddress; never allocates).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** ptr);
hipError_t launch_quantize_fp8(const void* x, uint8_t* x8, float* descale, int B, int H,
                               int N, const float* signs, bool transpose_out,
                               hipStream_t stream);

}  // namespace exattn
