// C ABI of libexattn.so: argument validation and dispatch to the gfx950 kernels.
// The contract of every entry point is documented in include/exattn.h.
#include "exattn.h"

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "launch.h"

namespace {

using exattn::FwdParams;

constexpr int64_t kMaxElems = int64_t(1) << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool too_big(int64_t a, int64_t b, int64_t c, int64_t d) {
  // a*b*c*d >= 2^31, evaluated without overflow (all factors >= 1).
  int64_t x = a * b;
  if (x >= kMaxElems) return true;
  x *= c;
  if (x >= kMaxElems) return true;
  return x * d >= kMaxElems;
}

bool supported_dims16(int d_qk, int d_v) {
  return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128);
}

int check_shape(int B, int H, int N_q, int N_kv, int d_qk, int d_v) {
  if (B < 1 || H < 1 || N_q < 1 || N_kv < 1) return ATTN_ERR_SHAPE;
  if (too_big(B, H, N_q, d_qk) || too_big(B, H, N_kv, d_qk) || too_big(B, H, N_kv, d_v) ||
      too_big(B, H, N_q, d_v))
    return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

int check_scale(float scale) { return std::isfinite(scale) ? ATTN_OK : ATTN_ERR_SCALE; }

constexpr float kLog2e = 1.4426950408889634f;

// The forward kernels take the row maximum of Q K^T times a non-negative factor. A
// negative scale is carried by negating Q instead: scale * (q . k) = |scale| * ((-q) . k),
// and flipping the sign bit of every Q element in registers is exact. Returns the XOR
// mask the kernels apply to each 32-bit word of Q (two 16-bit or four 8-bit elements).
unsigned q_sign_mask(float scale, bool fp8) {
  if (!std::signbit(scale) || scale == 0.f) return 0u;
  return fp8 ? 0x80808080u : 0x80008000u;
}

// Element strides (batch, head, row) of the four 16-bit tensors, in the order q, k, v, o.
struct Strides16 {
  int64_t v[4][3];
};

Strides16 dense_strides(int H, int N_q, int N_kv, int d_qk, int d_v) {
  Strides16 st;
  const int64_t rows[4] = {N_q, N_kv, N_kv, N_q};
  const int64_t dims[4] = {d_qk, d_qk, d_v, d_v};
  for (int t = 0; t < 4; ++t) {
    st.v[t][2] = dims[t];
    st.v[t][1] = rows[t] * dims[t];
    st.v[t][0] = H * rows[t] * dims[t];
  }
  return st;
}

// Shape checks of a strided call: every stride >= 0, rows at least d elements apart,
// row offsets of a (batch, head) slice below 2^30 elements (32-bit byte offsets).
int check_strides_shape(const Strides16& st, int N_q, int N_kv, int d_qk, int d_v) {
  const int64_t rows[4] = {N_q, N_kv, N_kv, N_q};
  const int64_t dims[4] = {d_qk, d_qk, d_v, d_v};
  for (int t = 0; t < 4; ++t) {
    if (st.v[t][0] < 0 || st.v[t][1] < 0 || st.v[t][2] < dims[t]) return ATTN_ERR_SHAPE;
    if (st.v[t][2] * rows[t] >= (int64_t(1) << 30)) return ATTN_ERR_SHAPE;
    if (st.v[t][0] >= (int64_t(1) << 40) || st.v[t][1] >= (int64_t(1) << 40)) return ATTN_ERR_SHAPE;
  }
  return ATTN_OK;
}

// O is written by many workgroups at once, so no two of its elements may share an
// address: with the dimensions of extent > 1 sorted by stride, each stride must reach
// past every element the smaller ones span (a sufficient condition; a layout that
// interleaves dimensions in some other non-overlapping way is refused too).
bool o_overlaps(const int64_t (&st)[3], int B, int H, int N_q, int d_v) {
  int64_t dims[3][2] = {{st[0], B}, {st[1], H}, {st[2], N_q}};
  // insertion sort of the three (stride, extent) pairs by stride
  for (int i = 1; i < 3; ++i)
    for (int j = i; j > 0 && dims[j][0] < dims[j - 1][0]; --j)
      for (int c = 0; c < 2; ++c) std::swap(dims[j][c], dims[j - 1][c]);
  int64_t span = d_v;  // elements of one row (stride 1)
  for (auto& dm : dims) {
    if (dm[1] <= 1) continue;
    if (dm[0] < span) return true;
    span = dm[0] * (dm[1] - 1) + span;
  }
  return false;
}

// 16-byte loads and stores need every stride to be a multiple of 8 elements.
bool strides_aligned(const Strides16& st) {
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < 3; ++i)
      if (st.v[t][i] % 8) return false;
  return true;
}

int fwd16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_q,
          int N_kv, int d_qk, int d_v, float scale, int causal, int dtype, int tau,
          const Strides16* strided, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (int rc = check_shape(B, H, N_q, N_kv, d_qk, d_v)) return rc;
  const Strides16 st = strided ? *strided : dense_strides(H, N_q, N_kv, d_qk, d_v);
  if (strided) {
    if (int rc = check_strides_shape(st, N_q, N_kv, d_qk, d_v)) return rc;
    if (o_overlaps(st.v[3], B, H, N_q, d_v)) return ATTN_ERR_SHAPE;
  }
  if (!supported_dims16(d_qk, d_v)) return ATTN_ERR_HEADDIM;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  if (int rc = check_scale(scale)) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !strides_aligned(st))
    return ATTN_ERR_ALIGN;
  if (tau != 0 && tau != 8) return ATTN_ERR_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  FwdParams p = {};
  p.q_sb = st.v[0][0], p.q_sh = st.v[0][1], p.q_sn = (int)st.v[0][2];
  p.k_sb = st.v[1][0], p.k_sh = st.v[1][1], p.k_sn = (int)st.v[1][2];
  p.v_sb = st.v[2][0], p.v_sh = st.v[2][1], p.v_sn = (int)st.v[2][2];
  p.o_sb = st.v[3][0], p.o_sh = st.v[3][1], p.o_sn = (int)st.v[3][2];
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.Nq = N_q;
  p.Nkv = N_kv;
  p.scale_log2 = std::fabs(scale) * kLog2e;
  p.q_neg = q_sign_mask(scale, false);
  hipError_t e = exattn::launch_fwd16(p, d_qk, d_v, causal != 0, dtype == ATTN_FP16, tau,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// Split-KV decode: validation shared by attn_decode_splits and attn_fwd_decode.
int check_decode(int B, int H, int H_kv, int N_q, int N_kv, int d_qk, int d_v) {
  if (B < 1 || H < 1 || H_kv < 1 || N_q < 1 || N_kv < 1 || H % H_kv != 0) return ATTN_ERR_SHAPE;
  if ((int64_t)(H / H_kv) * N_q > 128) return ATTN_ERR_SHAPE;
  if (too_big(B, H, N_q, d_qk) || too_big(B, H_kv, N_kv, d_qk) || too_big(B, H_kv, N_kv, d_v) ||
      too_big(B, H, N_q, d_v + 1))
    return ATTN_ERR_SHAPE;
  if (d_qk != d_v || (d_qk != 64 && d_qk != 128)) return ATTN_ERR_HEADDIM;
  return ATTN_OK;
}

constexpr int kDecodeTile = 32;      // keys per decode tile
constexpr int kDecodeMaxSplits = 256;

// Keys per split for `splits` requested ranges: whole tiles, every range non-empty.
int decode_chunk(int N_kv, int splits) {
  const int tiles = (N_kv + kDecodeTile - 1) / kDecodeTile;
  return (tiles + splits - 1) / splits * kDecodeTile;
}

// Split count for num_splits = 0: enough (batch, KV head, split) workgroups to give
// every resident workgroup slot of the device one, but no split shorter than two
// tiles per wave of a row block.
int decode_auto_splits(int B, int H, int H_kv, int N_q, int N_kv, int d) {
  const int slots = exattn::decode_resident_workgroups(d);
  const int groups = B * H_kv;
  if (slots <= 0 || groups >= slots) return 1;
  const int rows = H / H_kv * N_q;
  const int kv_waves = rows <= 32 ? 4 : rows <= 64 ? 2 : 1;  // waves sharing one row block
  const int max_splits = std::max(1, N_kv / (2 * kDecodeTile * kv_waves));
  return std::min({(slots + groups - 1) / groups, max_splits, kDecodeMaxSplits});
}

size_t decode_workspace(int B, int H, int N_q, int d_v, int splits) {
  if (splits <= 1) return 0;
  return (size_t)splits * B * H * N_q * (size_t)(d_v + 1) * sizeof(float);
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int N_q, int N_kv, int d_qk, int d_v, float scale, int causal, int dtype,
             void* stream) {
  return fwd16(q, k, v, o, lse, B, H, N_q, N_kv, d_qk, d_v, scale, causal, dtype, 8, nullptr,
               stream);
}

int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int N_q, int N_kv, int d_qk, int d_v, const int64_t* q_strides,
                     const int64_t* k_strides, const int64_t* v_strides,
                     const int64_t* o_strides, float scale, int causal, int dtype, void* stream) {
  if (!q_strides || !k_strides || !v_strides || !o_strides) return ATTN_ERR_NULL;
  Strides16 st;
  const int64_t* src[4] = {q_strides, k_strides, v_strides, o_strides};
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < 3; ++i) st.v[t][i] = src[t][i];
  return fwd16(q, k, v, o, lse, B, H, N_q, N_kv, d_qk, d_v, scale, causal, dtype, 8, &st, stream);
}

int attn_fwd_tau(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N_q, int N_kv, int d_qk, int d_v, float scale, int causal, int dtype,
                 int tau_log2, void* stream) {
  return fwd16(q, k, v, o, lse, B, H, N_q, N_kv, d_qk, d_v, scale, causal, dtype, tau_log2,
               nullptr, stream);
}

int attn_quantize_fp8(const void* x, uint8_t* x8, float* descale, int B, int H, int N, int d,
                      const float* signs, int transpose_out, void* stream) {
  if (!x || !x8 || !descale) return ATTN_ERR_NULL;
  if (check_shape(B, H, N, N, d, d)) return ATTN_ERR_SHAPE;
  if (d != 128) return ATTN_ERR_HEADDIM;
  if (!aligned16(x) || !aligned16(x8) || !aligned16(descale)) return ATTN_ERR_ALIGN;
  if (signs && !aligned16(signs)) return ATTN_ERR_ALIGN;
  if (transpose_out != 0 && transpose_out != 1) return ATTN_ERR_ARG;
  if (transpose_out && (N % 16) != 0) return ATTN_ERR_SHAPE;
  hipError_t e = exattn::launch_quantize_fp8(x, x8, descale, B, H, N, signs, transpose_out != 0,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t, const float* q_descale,
                 const float* k_descale, const float* v_descale, void* o, float* lse, int B, int H,
                 int N_q, int N_kv, int d_qk, int d_v, float scale, int causal, void* stream) {
  if (!q8 || !k8 || !v8t || !q_descale || !k_descale || !v_descale || !o || !lse)
    return ATTN_ERR_NULL;
  if (int rc = check_shape(B, H, N_q, N_kv, d_qk, d_v)) return rc;
  if (d_qk != 128 || d_v != 128) return ATTN_ERR_HEADDIM;
  if (int rc = check_scale(scale)) return rc;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_ALIGN;
  if ((N_kv % 16) != 0) return ATTN_ERR_SHAPE;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  FwdParams p = {};
  p.q = q8;
  p.k = k8;
  p.v = v8t;
  p.o = o;
  p.lse = lse;
  p.q_descale = q_descale;
  p.k_descale = k_descale;
  p.v_descale = v_descale;
  p.B = B;
  p.H = H;
  p.Nq = N_q;
  p.Nkv = N_kv;
  p.scale_log2 = std::fabs(scale) * kLog2e;
  p.q_neg = q_sign_mask(scale, true);
  hipError_t e = exattn::launch_fwd_fp8(p, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_decode_splits(int B, int H, int H_kv, int N_q, int N_kv, int d_qk, int d_v,
                       int num_splits) {
  if (int rc = check_decode(B, H, H_kv, N_q, N_kv, d_qk, d_v)) return rc;
  if (num_splits < 0 || num_splits > kDecodeMaxSplits) return ATTN_ERR_ARG;
  const int want = num_splits ? num_splits : decode_auto_splits(B, H, H_kv, N_q, N_kv, d_qk);
  const int chunk = decode_chunk(N_kv, want);
  return (N_kv + chunk - 1) / chunk;
}

size_t attn_decode_workspace_bytes(int B, int H, int N_q, int d_v, int splits) {
  if (B < 1 || H < 1 || N_q < 1 || d_v < 1) return 0;
  return decode_workspace(B, H, N_q, d_v, splits);
}

int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                    int H_kv, int N_q, int N_kv, int d_qk, int d_v, float scale, int causal,
                    int dtype, int num_splits, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (int rc = check_decode(B, H, H_kv, N_q, N_kv, d_qk, d_v)) return rc;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  if (int rc = check_scale(scale)) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      (workspace && !aligned16(workspace)))
    return ATTN_ERR_ALIGN;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  const int splits = attn_decode_splits(B, H, H_kv, N_q, N_kv, d_qk, d_v, num_splits);
  if (splits < 0) return splits;
  const size_t need = decode_workspace(B, H, N_q, d_v, splits);
  if (need && (!workspace || workspace_bytes < need)) return ATTN_ERR_ARG;
  exattn::DecodeParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  if (need) {
    p.o_part = static_cast<float*>(workspace);
    p.lse_part = p.o_part + (size_t)splits * B * H * N_q * d_v;
  }
  p.B = B;
  p.H = H;
  p.Hkv = H_kv;
  p.Nq = N_q;
  p.Nkv = N_kv;
  p.scale_log2 = std::fabs(scale) * kLog2e;
  p.q_neg = q_sign_mask(scale, false);
  p.splits = splits;
  p.chunk = decode_chunk(N_kv, splits);
  hipError_t e = exattn::launch_decode16(p, d_qk, causal != 0, dtype == ATTN_FP16,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int H_kv, int N_q, int N_kv, int d_qk, int d_v,
                            float scale, int causal, int dtype, int num_splits, void* stream) {
  // The same checks as attn_fwd_decode, in the same order, before the scratch is sized.
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (int rc = check_decode(B, H, H_kv, N_q, N_kv, d_qk, d_v)) return rc;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  if (int rc = check_scale(scale)) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_ALIGN;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  const int splits = attn_decode_splits(B, H, H_kv, N_q, N_kv, d_qk, d_v, num_splits);
  if (splits < 0) return splits;
  const size_t need = decode_workspace(B, H, N_q, d_v, splits);
  if (need > exattn::decode_scratch_bytes()) return ATTN_ERR_SCRATCH;
  void* ws = nullptr;
  if (need && exattn::decode_scratch(&ws) != hipSuccess) return ATTN_ERR_HIP;
  return attn_fwd_decode(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d_qk, d_v, scale, causal, dtype,
                         num_splits, ws, need, stream);
}

size_t attn_decode_scratch_bytes(void) { return exattn::decode_scratch_bytes(); }

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N_q,
             int N_kv, int d_qk, int d_v, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta) return ATTN_ERR_NULL;
  if (int rc = check_shape(B, H, N_q, N_kv, d_qk, d_v)) return rc;
  if (d_qk != d_v || (d_qk != 64 && d_qk != 128)) return ATTN_ERR_HEADDIM;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  if (int rc = check_scale(scale)) return rc;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv, delta};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTN_ERR_ALIGN;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  exattn::BwdParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = delta;
  p.B = B;
  p.H = H;
  p.Nq = N_q;
  p.Nkv = N_kv;
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;  // the backward uses the saved LSE, no row maximum
  hipError_t e = exattn::launch_bwd16(p, d_qk, causal != 0, dtype == ATTN_FP16,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape (a size < 1, a tensor with >= 2^31 elements, or N not a multiple of 16 where required)";
    case ATTN_ERR_HEADDIM: return "unsupported head dimensions";
    case ATTN_ERR_DTYPE: return "unsupported dtype";
    case ATTN_ERR_SCALE: return "scale must be finite";
    case ATTN_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case ATTN_ERR_HIP: return "HIP kernel launch failed";
    case ATTN_ERR_ARG: return "argument out of range";
    case ATTN_ERR_SCRATCH:
      return "the split partials need more than the library's static decode scratch "
             "(attn_decode_scratch_bytes(); pass a workspace to attn_fwd_decode instead)";
    default: return "unknown error code";
  }
}

}  // extern "C"
