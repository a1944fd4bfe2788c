/*
 * exattn.h - C ABI of libexattn.so, the fused exact-attention forward for
 * AMD MI355X (gfx950).
 *
 * The operation: for every batch b and head h,
 *     O = softmax(scale * Q K^T [+ causal mask]) V,   LSE = logsumexp rows,
 * computed without materialising the N_q x N_kv score matrix: query tiles are
 * kept on chip while key/value tiles stream through, and an online softmax
 * keeps a running row maximum and a running row sum, rescales the accumulator
 * and divides once at the end ("Attention at Scale - From FlashAttention to
 * FlashAttention-4", sections "The Problem" and "The Evolution"; "FlashAttention
 * 3 and 4: When the Bottleneck Moves", sections 2.1 and 3.2).
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers (memory of the current HIP device) unless
 *     the comment says otherwise. Tensors are dense, contiguous, row-major
 *     [B, H, N, d] ("BHND"): element (b, h, n, c) sits at ((b*H + h)*N + n)*d + c.
 *   - The caller owns every buffer. The library never allocates, frees or
 *     synchronises; it keeps no mutable global state, so calls are reentrant.
 *     Inputs are read-only; outputs must not alias inputs.
 *   - Calls are asynchronous: they validate the arguments, enqueue kernels on
 *     `stream` (a hipStream_t; NULL = the null stream) and return. A fault
 *     inside a kernel surfaces at the caller's next synchronisation.
 *   - Every entry point returns ATTN_OK (0) or a negative error code, checked
 *     in this order: null pointer, shape, head dims, dtype, scale, alignment,
 *     then the launch itself (ATTN_ERR_HIP). On an error nothing is enqueued.
 *   - Inputs holding Inf or NaN propagate NaN into the affected rows; they are
 *     not trapped.
 */
#ifndef EXATTN_H
#define EXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of Q, K, V and O for attn_fwd. */
enum {
    ATTN_BF16 = 0, /* bfloat16 */
    ATTN_FP16 = 1  /* IEEE half */
};

/* Return codes. */
enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,    /* a required pointer is NULL */
    ATTN_ERR_SHAPE = -2,   /* B, H, N_q or N_kv < 1, or a tensor has >= 2^31 elements */
    ATTN_ERR_HEADDIM = -3, /* (d_qk, d_v) not one of (64,64), (128,128), (192,128);
                              for the fp8 entry points only (128,128) */
    ATTN_ERR_DTYPE = -4,   /* dtype is neither ATTN_BF16 nor ATTN_FP16 */
    ATTN_ERR_SCALE = -5,   /* scale is NaN or infinite */
    ATTN_ERR_ALIGN = -6,   /* a tensor pointer is not 16-byte aligned */
    ATTN_ERR_HIP = -7,     /* the kernel launch failed (hipGetLastError) */
    ATTN_ERR_ARG = -8,     /* another argument is out of range (tau, transpose flag) */
    ATTN_ERR_SCRATCH = -9  /* attn_fwd_decode_noalloc: the problem needs more scratch
                              than the library's static buffer holds */
};

/*
 * attn_fwd - fused attention forward, 16-bit inputs.
 *
 *   q    [B, H, N_q,  d_qk]  dtype    queries
 *   k    [B, H, N_kv, d_qk]  dtype    keys
 *   v    [B, H, N_kv, d_v ]  dtype    values
 *   o    [B, H, N_q,  d_v ]  dtype    output, fully written (rounded to nearest even)
 *   lse  [B, H, N_q]         float32  natural-log logsumexp of the scaled scores,
 *                                     ln(sum_j exp(scale * q_i . k_j)) over visible j;
 *                                     fully written
 *   scale   softmax scale, any finite value (usually 1/sqrt(d_qk)); a negative
 *           scale is computed as |scale| applied to -Q (the sign bits of Q are
 *           flipped in registers, which is exact), so that the row maximum the
 *           online softmax keeps is that of the scaled scores
 *   causal  0: every key is visible. 1: key j is visible to query i iff
 *           j <= i + (N_kv - N_q) (bottom-right aligned; the lower triangle
 *           when N_q == N_kv). A query with no visible key gets O = 0 and
 *           LSE = -inf.
 *   dtype   ATTN_BF16 or ATTN_FP16
 *
 * Products run on bf16/fp16 MFMA with fp32 accumulation; softmax statistics
 * are fp32. The row maximum used for the exponentials is refreshed only when
 * it has grown by more than 8 doublings (a factor 256), as in "FlashAttention
 * 3 and 4: When the Bottleneck Moves", section 3.2; the result is the same
 * softmax since every row is divided by its own final sum.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N_q, int N_kv, int d_qk, int d_v,
             float scale, int causal, int dtype, void* stream);

/*
 * attn_fwd_strided - attn_fwd on tensors with arbitrary element strides, e.g. the
 * [B, N, H, d] ("BNHD") layout or a view into a larger buffer. The layout is an
 * interface matter the pages leave open; the arithmetic is attn_fwd's.
 *
 *   q_strides, k_strides, v_strides, o_strides  host pointers to 3 int64 each: the
 *           element strides along batch, head and row of q, k, v and o; the last
 *           dimension is dense (stride 1). Dense BHND is {H*N*d, N*d, d}.
 *   Every stride must be >= 0, row strides at least the row length (d_qk for q and
 *   k, d_v for v and o) and row stride * N below 2^30, batch and head strides below
 *   2^40 (else ATTN_ERR_SHAPE); every stride a multiple of 8 elements (16 bytes, else
 *   ATTN_ERR_ALIGN). lse stays dense [B, H, N_q]. o must not overlap q, k, v or lse,
 *   and no two elements of o may share an address: sorted by stride, each of o's
 *   batch, head and row strides (over dimensions of extent > 1) must be at least the
 *   span of the smaller ones, else ATTN_ERR_SHAPE. q, k and v may overlap (e.g. a
 *   head stride of 0 repeats one K/V head for every query head).
 */
int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int N_q, int N_kv, int d_qk, int d_v,
                     const int64_t* q_strides, const int64_t* k_strides,
                     const int64_t* v_strides, const int64_t* o_strides,
                     float scale, int causal, int dtype, void* stream);

/*
 * attn_fwd_tau - attn_fwd with an explicit rescale threshold, for checking
 * that the conditional rescale leaves the result unchanged.
 *   tau_log2  0: refresh the row maximum whenever it grows (plain online
 *             softmax); 8: the attn_fwd behaviour. Other values: ATTN_ERR_ARG.
 */
int attn_fwd_tau(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N_q, int N_kv, int d_qk, int d_v,
                 float scale, int causal, int dtype, int tau_log2, void* stream);

/*
 * attn_quantize_fp8 - per-block fp8 (OCP e4m3) quantisation, with an optional
 * random-sign Hadamard rotation ("FlashAttention 3 and 4: When the Bottleneck
 * Moves", section 2.2: one scale per block of values; Q and K multiplied by a
 * fixed random rotation, which cancels in Q K^T).
 *
 *   x        [B, H, N, d] bfloat16 input
 *   x8       uint8 e4m3 codes: [B, H, N, d], or [B, H, d, N] when transpose_out = 1
 *   descale  [B, H, ceil(N/128)] float32: a block is 128 consecutive tokens x d
 *   signs    device pointer to d floats, each +1 or -1 (any value >= 0 counts as
 *            +1, any value < 0 as -1), or NULL for no rotation. With signs the block is rotated by
 *            R = diag(signs) H_d / sqrt(d) (H_d the Sylvester Hadamard matrix).
 *   d        must be 128
 *   transpose_out  0 or 1 (1 is the layout attn_fwd_fp8 takes for V)
 *
 * Arithmetic (bit-exact by construction): y = x diag(signs) H_d is summed in
 * float64 (exact for bfloat16 inputs); amax = max|y| over the block;
 * code = e4m3_rne_saturating(float32(y * (448 / amax))) with the product and
 * quotient in float64; descale = float32(amax / (448 * sqrt(d))) with signs,
 * float32(amax / 448) without. An all-zero block gets codes 0 and descale 0.
 * Dequantised values code * descale approximate x R (or x).
 */
int attn_quantize_fp8(const void* x, uint8_t* x8, float* descale,
                      int B, int H, int N, int d, const float* signs,
                      int transpose_out, void* stream);

/*
 * attn_fwd_fp8 - fused attention forward on fp8 e4m3 inputs made by
 * attn_quantize_fp8 (Q and K with the same signs, V with transpose_out = 1).
 *
 *   q8 [B,H,N_q,d_qk], k8 [B,H,N_kv,d_qk], v8t [B,H,d_v,N_kv]  uint8 e4m3 codes
 *   q_descale [B,H,ceil(N_q/128)], k_descale, v_descale [B,H,ceil(N_kv/128)]  float32
 *   o [B,H,N_q,d_v] bfloat16, lse [B,H,N_q] float32: as for attn_fwd
 *   d_qk = d_v = 128.
 *
 * Both products run on the fp8 MFMA (e4m3 x e4m3 -> fp32); the softmax
 * weights are rounded to e4m3 for the second product.
 */
int attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t,
                 const float* q_descale, const float* k_descale, const float* v_descale,
                 void* o, float* lse, int B, int H, int N_q, int N_kv, int d_qk, int d_v,
                 float scale, int causal, void* stream);

/*
 * attn_fwd_decode - split-KV attention forward for decode-shaped problems, with
 * grouped KV heads ("Attention at Scale - From FlashAttention to
 * FlashAttention-4", section "Beyond Training: Attention Kernels for Serving":
 * decode is a few queries per head against a long key sequence; with grouped
 * KV heads the key sequence is split across workgroups to occupy the GPU
 * ("Sequence-Aware Split Heuristic"), and the partial results are combined by
 * an associative merge ("FlashInfer")).
 *
 *   q    [B, H,    N_q,  d]  dtype    queries
 *   k    [B, H_kv, N_kv, d]  dtype    keys
 *   v    [B, H_kv, N_kv, d]  dtype    values
 *   o    [B, H,    N_q,  d]  dtype    output, fully written (rounded to nearest even)
 *   lse  [B, H,    N_q]      float32  natural-log logsumexp, as for attn_fwd
 *   H_kv    KV heads; H must be a multiple of it. Query head h reads KV head
 *           h / (H / H_kv) (consecutive query heads share a KV head).
 *           (H / H_kv) * N_q must be at most 128, else ATTN_ERR_SHAPE.
 *   d_qk = d_v = 64 or 128, else ATTN_ERR_HEADDIM.
 *   scale, causal, dtype   as for attn_fwd (causal is bottom-right aligned).
 *   num_splits  key ranges per (batch, KV head): 0 picks attn_decode_splits'
 *           choice; 1..256 asks for that many (fewer are used when the key
 *           sequence has fewer 32-key tiles). Other values: ATTN_ERR_ARG.
 *   workspace   device memory of at least attn_decode_workspace_bytes(B, H, N_q,
 *           d_v, s) bytes, 16-byte aligned, where s = attn_decode_splits(...);
 *           may be NULL when s = 1. Too small or NULL otherwise: ATTN_ERR_ARG.
 *           Its contents on entry do not matter; on return they are undefined.
 *           Calls that share a workspace must not overlap in time.
 *
 * With s > 1 every split writes its fp32 partial (O normalised by its own sum,
 * and its LSE) to the workspace and a second kernel merges them:
 * LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
 */
int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int H_kv, int N_q, int N_kv, int d_qk, int d_v,
                    float scale, int causal, int dtype, int num_splits,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_splits - the number of key ranges attn_fwd_decode uses for these
 * arguments on the current device (num_splits = 0: its own choice, which gives
 * every resident workgroup slot of the GPU one (batch, KV head, range) while
 * keeping ranges at least two 32-key tiles per wave), or a negative error code
 * for arguments attn_fwd_decode would reject.
 */
int attn_decode_splits(int B, int H, int H_kv, int N_q, int N_kv, int d_qk, int d_v,
                       int num_splits);

/*
 * attn_decode_workspace_bytes - workspace attn_fwd_decode needs with `splits`
 * key ranges: splits * B*H*N_q * (d_v + 1) * 4 bytes, 0 when splits <= 1 or a
 * size is < 1.
 */
size_t attn_decode_workspace_bytes(int B, int H, int N_q, int d_v, int splits);

/*
 * attn_fwd_decode_noalloc - attn_fwd_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Arguments, checks and results are attn_fwd_decode's
 * with the same num_splits; the split partials go to a scratch buffer the
 * library holds as a static device array (one per GPU, kept until the process
 * ends) instead of a caller workspace. The call allocates and frees nothing.
 *
 *   The partials need splits * B*H*N_q * (d_v + 1) * 4 bytes (splits as
 *   attn_decode_splits reports); more than attn_decode_scratch_bytes() (8 MiB)
 *   returns ATTN_ERR_SCRATCH before anything is launched. A call with one
 *   split uses no scratch.
 *   The scratch needs no initial contents (every partial is written before it
 *   is read). All calls on one GPU share it: calls that overlap in time on one
 *   GPU (other streams, other host threads) race and give wrong results;
 *   serialise them, or use attn_fwd_decode with separate workspaces.
 */
int attn_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int H_kv, int N_q, int N_kv, int d_qk, int d_v,
                            float scale, int causal, int dtype, int num_splits, void* stream);

/* attn_decode_scratch_bytes - size of the static scratch attn_fwd_decode_noalloc uses. */
size_t attn_decode_scratch_bytes(void);

/*
 * attn_bwd - gradients of attn_fwd: dQ, dK, dV from Q, K, V, the forward's O and
 * LSE, and dO ("FlashAttention-4: Algorithm and Kernel Pipelining Co-Design for
 * Asymmetric Hardware Scaling", Figure 2: the scores are recomputed from Q, K and
 * the saved LSE, then five matrix products and two elementwise steps:
 * dV = P^T dO, dP = dO V^T, dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q,
 * with D_i = sum_c dO_ic O_ic).
 *
 *   q, k, v, o, dout, dq, dk, dv   dense [B, H, N, d], dtype; o and lse as attn_fwd
 *                                  wrote them for the same q, k, v, scale, causal
 *   lse    [B, H, N_q] float32, as attn_fwd wrote it; a row with no visible key
 *          (LSE = -inf, causal with N_q > N_kv) gets zero gradients. An LSE of -inf
 *          on a row that sees keys is outside this contract (non-finite results).
 *   delta  [B, H, N_q] float32 workspace: D is written there (caller-owned)
 *   d_qk = d_v = 64 or 128, else ATTN_ERR_HEADDIM.
 *   dq, dk, dv are fully written (rounded to nearest even); the result is
 *   deterministic (no atomics): one kernel computes D and dQ, a second dK and dV.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta,
             int B, int H, int N_q, int N_kv, int d_qk, int d_v,
             float scale, int causal, int dtype, void* stream);

/* Static, NUL-terminated description of a return code (never NULL). */
const char* attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* EXATTN_H */
