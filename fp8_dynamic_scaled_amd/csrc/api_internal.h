// Host-side pieces of the C-ABI shared between its source files (internal to libfp8attn).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8attn {

// The whole of fp8attn_forward (argument checks, then the launches). `fn` names the entry
// point in error messages. With acquire_scratch == nullptr the caller's workspace is used;
// otherwise the FP8 path's workspace is a fixed array of workspace_bytes bytes whose device
// address acquire_scratch provides (returning an FP8ATTN_ status), called only after every
// argument, the needed size included, has passed its check.
int forward_impl(const char* fn, void* state, const void* q, const void* k, const void* v,
                 const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int num_seqs,
                 int num_heads, int head_dim, float softmax_scale, unsigned flags,
                 void* workspace, size_t workspace_bytes, void* out, void* stream,
                 int (*acquire_scratch)(void** workspace));

// FP8ATTN_OK for hipSuccess; otherwise FP8ATTN_EHIP with "<what>: <HIP message>" as the
// calling thread's last error.
int hip_result(hipError_t e, const char* what);

}  // namespace fp8attn
