// fp8attn_forward_noalloc: fp8attn_forward for callers that cannot allocate device memory
// (code under HIP graph capture, serving loops or harnesses that forbid hipMalloc). The
// FP8 path's workspace (Q8 | K8 | V8t) lives in one fixed device array of this library
// instead of a caller's buffer; everything else, kernels included, is fp8attn_forward's.
//
// The array exists once per GPU the library runs on, from the moment the library's code
// object is loaded on that GPU until the process ends. Its device address is looked up
// once per device (hipGetSymbolAddress, on the first call that device makes) and kept: the
// array's name is only a host-side handle, never a device address. Nothing here allocates.
// Every call on one GPU shares that GPU's array, so calls that overlap in time on one GPU
// (two streams, two host threads) race on it; nothing needs to start at zero (the quantise
// kernels write every byte the attention reads, V8t's zero padding included).
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"
#include "fp8attn.h"

namespace {

static_assert(FP8ATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

__device__ __align__(256) uint8_t scratch[FP8ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on first use).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fp8attn::hip_result(e, "fp8attn_forward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fp8attn::hip_result(hipErrorInvalidDevice, "fp8attn_forward_noalloc: device index");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
      return fp8attn::hip_result(e, "fp8attn_forward_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FP8ATTN_OK;
}

}  // namespace

extern "C" int fp8attn_forward_noalloc(void* state, const void* q, const void* k,
                                       const void* v, const int32_t* cu_seqlens,
                                       const int32_t* cu_seqlens_host, int num_seqs,
                                       int num_heads, int head_dim, float softmax_scale,
                                       unsigned flags, void* out, void* stream) {
  // the scratch address is looked up only after every argument has been checked, and only
  // on the FP8 path (the BF16 path uses no workspace)
  return fp8attn::forward_impl("fp8attn_forward_noalloc", state, q, k, v, cu_seqlens,
                               cu_seqlens_host, num_seqs, num_heads, head_dim, softmax_scale,
                               flags, nullptr, FP8ATTN_NOALLOC_SCRATCH_BYTES, out, stream,
                               scratch_address);
}
