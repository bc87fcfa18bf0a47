// C-ABI of libfp8attn: argument checks on the host, launch sizing from the host copy of
// cu_seqlens, and error reporting. Every call only enqueues on the caller's stream.
// Behaviour of each entry point is specified in include/fp8attn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "fp8attn.h"
#include "api_internal.h"
#include "launch.h"

static_assert(sizeof(fp8attn_state) == 1280, "fp8attn_state is part of the ABI");
static_assert(offsetof(fp8attn_state, cur) % 64 == 0, "each stripe is a 64-byte line");

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return FP8ATTN_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FP8ATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int64_t padded_keys(int64_t T, int num_seqs) { return round_up(T, 128) + 128 * (int64_t)num_seqs; }

struct Varlen {
  int64_t T = 0;
  int max_seqlen = 0;
  int64_t Tp = 0;
  size_t ws_bytes = 0;
};

// Checks shared by fp8attn_quantize and fp8attn_forward.
int check_varlen(const char* fn, const void* q, const void* k, const void* v,
                 const int32_t* cu, const int32_t* cu_host, int num_seqs, int num_heads,
                 int head_dim, Varlen* out) {
  if (!cu || !cu_host)
    return fail(FP8ATTN_EINVAL, "%s: cu_seqlens and cu_seqlens_host must be non-NULL", fn);
  if (num_seqs < 1) return fail(FP8ATTN_EINVAL, "%s: num_seqs must be >= 1 (got %d)", fn, num_seqs);
  if (num_heads < 1) return fail(FP8ATTN_EINVAL, "%s: num_heads must be >= 1 (got %d)", fn, num_heads);
  if (head_dim != 128)
    return fail(FP8ATTN_EUNSUPPORTED, "%s: head_dim %d is not supported (only 128)", fn, head_dim);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(FP8ATTN_EINVAL, "%s: q, k and v must be 16-byte aligned", fn);
  if (cu_host[0] != 0) return fail(FP8ATTN_EINVAL, "%s: cu_seqlens[0] must be 0 (got %d)", fn, cu_host[0]);
  int max_len = 0;
  for (int i = 0; i < num_seqs; ++i) {
    const int64_t len = (int64_t)cu_host[i + 1] - cu_host[i];
    if (len < 0)
      return fail(FP8ATTN_EINVAL, "%s: cu_seqlens decreases at index %d (%d -> %d)", fn, i,
                  cu_host[i], cu_host[i + 1]);
    if (len > max_len) max_len = (int)len;
  }
  const int64_t T = cu_host[num_seqs];
  // an empty batch reads no tensor element: q, k, v may then be NULL
  if (T > 0 && (!q || !k || !v)) return fail(FP8ATTN_EINVAL, "%s: q, k and v must be non-NULL", fn);
  // token indices and per-head element offsets are kept in 32/64-bit ranges
  if (T * num_heads > ((int64_t)1 << 31) - 1)
    return fail(FP8ATTN_EINVAL, "%s: total_tokens * num_heads = %lld exceeds 2^31-1", fn,
                (long long)(T * num_heads));
  // the attention kernels address one sequence of one tensor, and one head's V8t rows, with
  // 32-bit buffer offsets
  if ((int64_t)max_len * num_heads * head_dim > ((int64_t)1 << 31) - 1)
    return fail(FP8ATTN_EUNSUPPORTED,
                "%s: longest sequence x num_heads x head_dim = %lld exceeds 2^31-1", fn,
                (long long)max_len * num_heads * head_dim);
  if ((int64_t)head_dim * padded_keys(T, num_seqs) > ((int64_t)1 << 31) - 1)
    return fail(FP8ATTN_EUNSUPPORTED, "%s: head_dim x padded tokens exceeds 2^31-1", fn);
  out->T = T;
  out->max_seqlen = max_len;
  out->Tp = padded_keys(T, num_seqs);
  out->ws_bytes = fp8attn_workspace_bytes(T, num_seqs, num_heads, head_dim);
  return FP8ATTN_OK;
}

}  // namespace

namespace fp8attn {

int hip_result(hipError_t e, const char* what) { return hip_status(e, what); }

int forward_impl(const char* fn, void* state, const void* q, const void* k, const void* v,
                 const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int num_seqs,
                 int num_heads, int head_dim, float softmax_scale, unsigned flags,
                 void* workspace, size_t workspace_bytes, void* out, void* stream,
                 int (*acquire_scratch)(void** workspace)) {
  const bool scratch = acquire_scratch != nullptr;
  if (flags & ~(FP8ATTN_SKIP | FP8ATTN_OBSERVE))
    return fail(FP8ATTN_EINVAL, "%s: unknown flag bits 0x%x", fn, flags);
  if ((flags & FP8ATTN_SKIP) && (flags & FP8ATTN_OBSERVE))
    return fail(FP8ATTN_EINVAL, "%s: FP8ATTN_OBSERVE and FP8ATTN_SKIP exclude each other", fn);
  Varlen vl;
  int rc = check_varlen(fn, q, k, v, cu_seqlens, cu_seqlens_host, num_seqs, num_heads, head_dim, &vl);
  if (rc != FP8ATTN_OK) return rc;
  if ((vl.T > 0 && !out) || !aligned16(out))
    return fail(FP8ATTN_EINVAL, "%s: out must be non-NULL and 16-byte aligned", fn);
  if (!std::isfinite(softmax_scale))
    return fail(FP8ATTN_EINVAL, "%s: softmax_scale must be finite", fn);
  const bool skip = (flags & FP8ATTN_SKIP) != 0;
  // the BF16 kernel addresses one sequence of a bf16 tensor with 32-bit byte offsets
  if (skip && (int64_t)vl.max_seqlen * num_heads * head_dim * 2 > ((int64_t)1 << 31) - 1)
    return fail(FP8ATTN_EUNSUPPORTED,
                "%s: the BF16 path needs longest sequence x num_heads x head_dim x 2 bytes < 2^31", fn);
  if (!skip) {
    if (!state) return fail(FP8ATTN_EINVAL, "%s: the FP8 path needs a state", fn);
    if (scratch && workspace_bytes < vl.ws_bytes)
      return fail(FP8ATTN_EINVAL,
                  "%s: this call needs %zu bytes of workspace; the library's fixed scratch "
                  "holds %zu", fn, vl.ws_bytes, workspace_bytes);
    // every argument is checked: only now look up the fixed scratch array
    if (scratch && (rc = acquire_scratch(&workspace)) != FP8ATTN_OK) return rc;
    if (!workspace || !aligned16(workspace))
      return fail(FP8ATTN_EINVAL, "%s: workspace must be non-NULL and 16-byte aligned", fn);
    if (workspace_bytes < vl.ws_bytes)
      return fail(FP8ATTN_EINVAL, "%s: workspace of %zu bytes is smaller than the %zu needed",
                  fn, workspace_bytes, vl.ws_bytes);
  }
  const bool observe = (flags & FP8ATTN_OBSERVE) != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (vl.T == 0) {
    if (!observe) return ok();
    return hip_status(fp8attn::launch_scales(static_cast<fp8attn_state*>(state), FP8ATTN_DYNAMIC,
                                             nullptr, 0.0f, s),
                      fn);
  }
  const float sm = softmax_scale > 0.0f ? softmax_scale
                                        : (float)(1.0 / std::sqrt((double)head_dim));
  fp8attn::AttnLaunch a;
  a.cu = cu_seqlens;
  a.num_seqs = num_seqs;
  a.H = num_heads;
  a.T = vl.T;
  a.Tp = vl.Tp;
  a.max_seqlen = vl.max_seqlen;
  a.softmax_scale = sm;
  a.out = static_cast<uint16_t*>(out);
  if (skip) {
    return hip_status(fp8attn::launch_attn_bf16(a, static_cast<const uint16_t*>(q),
                                                static_cast<const uint16_t*>(k),
                                                static_cast<const uint16_t*>(v), s),
                      fn);
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int64_t n = vl.T * num_heads * head_dim;
  const fp8attn_state* st = static_cast<const fp8attn_state*>(state);
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  hipError_t e =
      observe ? fp8attn::launch_quantize_dynamic(static_cast<fp8attn_state*>(state), q16, k16, v16,
                                                 cu_seqlens, num_seqs, vl.T, num_heads, ws,
                                                 ws + n, ws + 2 * n, vl.Tp, s)
              : fp8attn::launch_quantize(st, q16, k16, v16, cu_seqlens, num_seqs, vl.T,
                                         num_heads, ws, ws + n, ws + 2 * n, vl.Tp, s);
  if (e != hipSuccess) return hip_status(e, fn);
  return hip_status(fp8attn::launch_attn_fp8(a, st, ws, ws + n, ws + 2 * n, s),
                    fn);
}

}  // namespace fp8attn

extern "C" {

size_t fp8attn_state_bytes(void) { return sizeof(fp8attn_state); }

const char* fp8attn_last_error(void) { return g_last_error.c_str(); }

int fp8attn_state_reset(void* state, void* stream) {
  if (!state) return fail(FP8ATTN_EINVAL, "fp8attn_state_reset: state must be non-NULL");
  return hip_status(fp8attn::launch_state_reset(static_cast<fp8attn_state*>(state),
                                                static_cast<hipStream_t>(stream)),
                    "fp8attn_state_reset");
}

int fp8attn_observe_amax(void* state, const void* q, const void* k, const void* v, int64_t n,
                         void* stream) {
  if (!state) return fail(FP8ATTN_EINVAL, "fp8attn_observe_amax: state must be non-NULL");
  if (n < 0) return fail(FP8ATTN_EINVAL, "fp8attn_observe_amax: n must be >= 0 (got %lld)", (long long)n);
  if (n > 0 && (!q || !k || !v))
    return fail(FP8ATTN_EINVAL, "fp8attn_observe_amax: q, k and v must be non-NULL");
  if (n > 0 && (!aligned16(q) || !aligned16(k) || !aligned16(v)))
    return fail(FP8ATTN_EINVAL, "fp8attn_observe_amax: q, k and v must be 16-byte aligned");
  return hip_status(fp8attn::launch_amax(static_cast<fp8attn_state*>(state),
                                         static_cast<const uint16_t*>(q),
                                         static_cast<const uint16_t*>(k),
                                         static_cast<const uint16_t*>(v), n,
                                         static_cast<hipStream_t>(stream)),
                    "fp8attn_observe_amax");
}

int fp8attn_scales(void* state, int mode, const float* static_amax_host, float margin,
                   void* stream) {
  if (!state) return fail(FP8ATTN_EINVAL, "fp8attn_scales: state must be non-NULL");
  if (mode != FP8ATTN_DYNAMIC && mode != FP8ATTN_STATIC)
    return fail(FP8ATTN_EINVAL, "fp8attn_scales: unknown mode %d", mode);
  if (mode == FP8ATTN_STATIC) {
    if (!static_amax_host)
      return fail(FP8ATTN_EINVAL, "fp8attn_scales: static mode needs static_amax_host[3]");
    for (int t = 0; t < 3; ++t)
      if (!std::isfinite(static_amax_host[t]) || static_amax_host[t] < 0.0f)
        return fail(FP8ATTN_EINVAL, "fp8attn_scales: static amax[%d] = %g must be finite and >= 0",
                    t, (double)static_amax_host[t]);
    if (!std::isfinite(margin) || !(margin > 0.0f))
      return fail(FP8ATTN_EINVAL, "fp8attn_scales: margin %g must be finite and > 0", (double)margin);
    // the scales kernel forms A = fp32(amax * margin); an overflow to inf would give a zero
    // inverse scale (every code 0) and NaN attention output
    for (int t = 0; t < 3; ++t) {
      volatile float a = static_amax_host[t] * margin;   // the binary32 product, as on the device
      if (!std::isfinite(a))
        return fail(FP8ATTN_EINVAL,
                    "fp8attn_scales: static amax[%d] x margin = %g x %g overflows binary32", t,
                    (double)static_amax_host[t], (double)margin);
    }
  }
  return hip_status(fp8attn::launch_scales(static_cast<fp8attn_state*>(state), mode,
                                           mode == FP8ATTN_STATIC ? static_amax_host : nullptr,
                                           margin, static_cast<hipStream_t>(stream)),
                    "fp8attn_scales");
}

size_t fp8attn_workspace_bytes(int64_t total_tokens, int num_seqs, int num_heads,
                               int head_dim) {
  if (total_tokens < 0 || num_seqs < 1 || num_heads < 1 || head_dim < 1) return 0;
  if (total_tokens > ((int64_t)1 << 40) || num_seqs > (1 << 30) || num_heads > (1 << 20) ||
      head_dim > (1 << 16))
    return 0;
  const int64_t hd = (int64_t)num_heads * head_dim;
  const int64_t Tp = padded_keys(total_tokens, num_seqs);
  return (size_t)(2 * total_tokens * hd + hd * Tp);
}

int fp8attn_quantize(const void* state, const void* q, const void* k, const void* v,
                     const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int num_seqs,
                     int num_heads, int head_dim, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const char* fn = "fp8attn_quantize";
  if (!state) return fail(FP8ATTN_EINVAL, "%s: state must be non-NULL", fn);
  Varlen vl;
  int rc = check_varlen(fn, q, k, v, cu_seqlens, cu_seqlens_host, num_seqs, num_heads, head_dim, &vl);
  if (rc != FP8ATTN_OK) return rc;
  if (!workspace || !aligned16(workspace))
    return fail(FP8ATTN_EINVAL, "%s: workspace must be non-NULL and 16-byte aligned", fn);
  if (workspace_bytes < vl.ws_bytes)
    return fail(FP8ATTN_EINVAL, "%s: workspace of %zu bytes is smaller than the %zu needed", fn,
                workspace_bytes, vl.ws_bytes);
  if (vl.T == 0) return ok();
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int64_t n = vl.T * num_heads * head_dim;
  return hip_status(
      fp8attn::launch_quantize(static_cast<const fp8attn_state*>(state),
                               static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                               static_cast<const uint16_t*>(v), cu_seqlens, num_seqs, vl.T,
                               num_heads, ws, ws + n, ws + 2 * n, vl.Tp,
                               static_cast<hipStream_t>(stream)),
      fn);
}

int fp8attn_quantize_dynamic(void* state, const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                             int num_seqs, int num_heads, int head_dim, void* workspace,
                             size_t workspace_bytes, void* stream) {
  const char* fn = "fp8attn_quantize_dynamic";
  if (!state) return fail(FP8ATTN_EINVAL, "%s: state must be non-NULL", fn);
  Varlen vl;
  int rc = check_varlen(fn, q, k, v, cu_seqlens, cu_seqlens_host, num_seqs, num_heads, head_dim, &vl);
  if (rc != FP8ATTN_OK) return rc;
  if (!workspace || !aligned16(workspace))
    return fail(FP8ATTN_EINVAL, "%s: workspace must be non-NULL and 16-byte aligned", fn);
  if (workspace_bytes < vl.ws_bytes)
    return fail(FP8ATTN_EINVAL, "%s: workspace of %zu bytes is smaller than the %zu needed", fn,
                workspace_bytes, vl.ws_bytes);
  fp8attn_state* st = static_cast<fp8attn_state*>(state);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // no tokens: the observation is 0 and only the ring moves, as with observe + scales
  if (vl.T == 0) return hip_status(fp8attn::launch_scales(st, FP8ATTN_DYNAMIC, nullptr, 0.0f, s), fn);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int64_t n = vl.T * num_heads * head_dim;
  return hip_status(
      fp8attn::launch_quantize_dynamic(st, static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(k),
                                       static_cast<const uint16_t*>(v), cu_seqlens, num_seqs,
                                       vl.T, num_heads, ws, ws + n, ws + 2 * n, vl.Tp, s),
      fn);
}

int fp8attn_attend(const void* state, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                   int num_seqs, int num_heads, int head_dim, float softmax_scale,
                   const void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const char* fn = "fp8attn_attend";
  // q, k, v are not read: pass the (aligned, non-NULL) workspace in their place for the
  // shared checks.
  if (!workspace || !aligned16(workspace))
    return fail(FP8ATTN_EINVAL, "%s: workspace must be non-NULL and 16-byte aligned", fn);
  Varlen vl;
  int rc = check_varlen(fn, workspace, workspace, workspace, cu_seqlens, cu_seqlens_host,
                        num_seqs, num_heads, head_dim, &vl);
  if (rc != FP8ATTN_OK) return rc;
  if (!state) return fail(FP8ATTN_EINVAL, "%s: state must be non-NULL", fn);
  if (workspace_bytes < vl.ws_bytes)
    return fail(FP8ATTN_EINVAL, "%s: workspace of %zu bytes is smaller than the %zu needed", fn,
                workspace_bytes, vl.ws_bytes);
  if (!out || !aligned16(out))
    return fail(FP8ATTN_EINVAL, "%s: out must be non-NULL and 16-byte aligned", fn);
  if (!std::isfinite(softmax_scale))
    return fail(FP8ATTN_EINVAL, "%s: softmax_scale must be finite", fn);
  if (vl.T == 0) return ok();
  fp8attn::AttnLaunch a;
  a.cu = cu_seqlens;
  a.num_seqs = num_seqs;
  a.H = num_heads;
  a.T = vl.T;
  a.Tp = vl.Tp;
  a.max_seqlen = vl.max_seqlen;
  a.softmax_scale = softmax_scale > 0.0f ? softmax_scale : (float)(1.0 / std::sqrt((double)head_dim));
  a.out = static_cast<uint16_t*>(out);
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  const int64_t n = vl.T * num_heads * head_dim;
  return hip_status(fp8attn::launch_attn_fp8(a, static_cast<const fp8attn_state*>(state), ws,
                                              ws + n, ws + 2 * n, static_cast<hipStream_t>(stream)),
                    fn);
}

int fp8attn_forward(void* state, const void* q, const void* k, const void* v,
                    const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int num_seqs,
                    int num_heads, int head_dim, float softmax_scale, unsigned flags,
                    void* workspace, size_t workspace_bytes, void* out, void* stream) {
  return fp8attn::forward_impl("fp8attn_forward", state, q, k, v, cu_seqlens, cu_seqlens_host,
                               num_seqs, num_heads, head_dim,
                               softmax_scale, flags, workspace, workspace_bytes, out, stream,
                               nullptr);
}

}  // extern "C"
