// Per-tensor amax observation and the scale update (vLLM docs "FP8 ViT Encoder
// Attention", section "Usage": every dynamic forward observes the Q/K/V amax, and a
// circular buffer of the last 16 observations drives that forward's scale; static
// scales are calibrated amax values times a margin, default 1.5).
//
// amax_kernel: one launch reads Q, K and V (bf16) once; HBM-bound. Each thread keeps a
// packed 16-bit max of |x| (the bf16 bit pattern with the sign cleared orders like the
// magnitude), the block reduces through a wave shuffle and LDS, and at most one atomicMax
// per block and tensor folds it into the block's stripe of state->cur as the fp32 bit image
// (non-negative floats order like their bits).
// scales_kernel: one wave; gathers tensor t's observation from its stripes into ring slot
// count mod 16, takes the window maximum and writes scale = A/448, inv = 448/A (IEEE
// division), clears the stripes, and records
// in `moved` which tensors' window maximum this observation raised.
#include "device_common.h"
#include "launch.h"

namespace fp8attn {

namespace {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxVec = 8;  // uint4 loads in flight per thread per iteration

__device__ __forceinline__ us2 abs_pk(uint32_t w) {
  uint32_t m = w & 0x7fff7fffu;
  return *reinterpret_cast<us2*>(&m);
}

__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(fp8attn_state* st,
                                                             const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             int64_t n) {
  const int t = blockIdx.y;
  const uint16_t* x = t == 0 ? q : (t == 1 ? k : v);
  const int64_t nvec = n / 8;  // uint4 = 8 bf16
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  us2 acc = {0, 0};
  const int64_t stride = (int64_t)gridDim.x * kAmaxThreads;
  int64_t i = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
  // main loop: kAmaxVec independent 16-byte loads per iteration
  for (; i + (kAmaxVec - 1) * stride < nvec; i += kAmaxVec * stride) {
    uint4 r[kAmaxVec];
#pragma unroll
    for (int u = 0; u < kAmaxVec; ++u) r[u] = xv[i + u * stride];
#pragma unroll
    for (int u = 0; u < kAmaxVec; ++u) {
      acc = __builtin_elementwise_max(acc, abs_pk(r[u].x));
      acc = __builtin_elementwise_max(acc, abs_pk(r[u].y));
      acc = __builtin_elementwise_max(acc, abs_pk(r[u].z));
      acc = __builtin_elementwise_max(acc, abs_pk(r[u].w));
    }
  }
  for (; i < nvec; i += stride) {
    uint4 r = xv[i];
    acc = __builtin_elementwise_max(acc, abs_pk(r.x));
    acc = __builtin_elementwise_max(acc, abs_pk(r.y));
    acc = __builtin_elementwise_max(acc, abs_pk(r.z));
    acc = __builtin_elementwise_max(acc, abs_pk(r.w));
  }
  uint32_t m = acc.x > acc.y ? acc.x : acc.y;
  // scalar tail (n not a multiple of 8)
  if (blockIdx.x == 0) {
    for (int64_t j = nvec * 8 + threadIdx.x; j < n; j += kAmaxThreads) {
      uint32_t b = x[j] & 0x7fffu;
      m = b > m ? b : m;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(m, off);
    m = o > m ? o : m;
  }
  __shared__ uint32_t red[kAmaxThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = red[0];
#pragma unroll
    for (int w = 1; w < kAmaxThreads / 64; ++w) b = red[w] > b ? red[w] : b;
    // bf16 magnitude -> fp32 bit image, then fold into this block's stripe of the pending
    // observation
    fold_max(&st->cur[blockIdx.x % FP8ATTN_CUR_STRIPES][t], b << 16);
  }
}

__global__ void scales_kernel(fp8attn_state* st, int mode, float s0, float s1, float s2,
                              float margin) {
  const int t = threadIdx.x;
  uint32_t count = st->count;
  bool moved = false;
  if (t < 3) {
    if (mode == FP8ATTN_DYNAMIC) {
      // window maximum of the slots that stay, then with this forward's observation
      const uint32_t slot = count % FP8ATTN_RING_SLOTS;
      moved = dynamic_update(st, t, slot, ring_max_except(st, t, slot),
                             take_observation(st, t));
    } else {
      const float cal = t == 0 ? s0 : (t == 1 ? s1 : s2);
      const float A = cal * margin;
      st->amax[t] = A;
      st->scale[t] = scale_from_amax(A);
      st->inv_scale[t] = inv_scale_from_amax(A);
      take_observation(st, t);   // cleared; a static update does not use it
    }
  }
  const uint32_t mask = (uint32_t)(__builtin_amdgcn_ballot_w64(moved) & 7u);
  __syncthreads();
  if (t == 0) {
    st->moved = mask;
    if (mode == FP8ATTN_DYNAMIC) st->count = count + 1;
  }
}

__global__ void state_reset_kernel(uint32_t* words, int nwords) {
  const int i = threadIdx.x;
  if (i < nwords) words[i] = 0u;
}

}  // namespace

hipError_t launch_state_reset(fp8attn_state* st, hipStream_t s) {
  const int nwords = (int)(sizeof(fp8attn_state) / 4);
  hipLaunchKernelGGL(state_reset_kernel, dim3(1), dim3(64 * ((nwords + 63) / 64)), 0, s,
                     reinterpret_cast<uint32_t*>(st), nwords);
  return hipGetLastError();
}

hipError_t launch_amax(fp8attn_state* st, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;  // amax of an empty tensor is the cleared 0
  const int64_t nvec = n / 8;
  // ~2 blocks per CU and tensor (grid-stride loops, kAmaxVec 16-byte loads in flight per
  // thread): few enough that the per-block atomics stay cheap
  int64_t blocks = (nvec + (int64_t)kAmaxThreads * kAmaxVec - 1) / ((int64_t)kAmaxThreads * kAmaxVec);
  if (blocks > 512) blocks = 512;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks, 3), dim3(kAmaxThreads), 0, s, st, q,
                     k, v, n);
  return hipGetLastError();
}

hipError_t launch_scales(fp8attn_state* st, int mode, const float static_amax[3],
                         float margin, hipStream_t s) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f;
  if (static_amax) {
    a0 = static_amax[0];
    a1 = static_amax[1];
    a2 = static_amax[2];
  }
  hipLaunchKernelGGL(scales_kernel, dim3(1), dim3(64), 0, s, st, mode, a0, a1, a2, margin);
  return hipGetLastError();
}

}  // namespace fp8attn
