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
  float scale_log2;     // softmax scale * log2(e), >= 0
  int n_qtiles;         // ceil(N_q / BLOCK_M)
};

// Launchers (one per instantiation family); return hipError_t of the launch.
hipError_t launch_fwd16(const FwdParams& p, int d_qk, int d_v, bool causal, bool fp16,
                        int tau, hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdParams& p, bool causal, hipStream_t stream);
hipError_t launch_quantize_fp8(const void* x, uint8_t* x8, float* descale, int B, int H,
                               int N, const float* signs, bool transpose_out,
                               hipStream_t stream);

}  // namespace exattn
