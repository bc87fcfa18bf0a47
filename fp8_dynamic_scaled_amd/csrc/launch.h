// Host-side launchers of the gfx950 kernels (internal to libfp8attn; the C-ABI in
// fp8attn_api.cpp validates arguments and calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8attn.h"

namespace fp8attn {

hipError_t launch_state_reset(fp8attn_state* st, hipStream_t s);

hipError_t launch_amax(fp8attn_state* st, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, int64_t n, hipStream_t s);

hipError_t launch_scales(fp8attn_state* st, int mode, const float static_amax[3],
                         float margin, hipStream_t s);

// Q, K -> E4M3 [T][H][D]; V -> E4M3 key-contiguous V8t [H][D][Tp].
hipError_t launch_quantize(const fp8attn_state* st, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const int32_t* cu, int num_seqs, int64_t T,
                           int H, uint8_t* q8, uint8_t* k8, uint8_t* v8t, int64_t Tp,
                           hipStream_t s);

// Dynamic forward in one pass over Q/K/V when the window maximum does not move: quantise
// with the scale of the ring's other 15 slots while observing this forward's amax, run the
// scales kernel (dynamic), then re-quantise the tensors whose window maximum changed. The
// state's pending observation (cur) must be clear, as every scales call leaves it.
hipError_t launch_quantize_dynamic(fp8attn_state* st, const uint16_t* q, const uint16_t* k,
                                   const uint16_t* v, const int32_t* cu, int num_seqs,
                                   int64_t T, int H, uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                                   int64_t Tp, hipStream_t s);

struct AttnLaunch {
  const int32_t* cu;     // device cu_seqlens
  int num_seqs;
  int H;
  int64_t T;
  int64_t Tp;            // padded key columns of V8t (FP8 path)
  int max_seqlen;        // from the host copy: sizes the grid
  float softmax_scale;
  uint16_t* out;
};

hipError_t launch_attn_fp8(const AttnLaunch& a, const fp8attn_state* st, const uint8_t* q8,
                           const uint8_t* k8, const uint8_t* v8t, hipStream_t s);

hipError_t launch_attn_bf16(const AttnLaunch& a, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, hipStream_t s);

}  // namespace fp8attn
