// HBM stream kernels for the benchmark (libfp8attn_stream.so, not part of the C-ABI of
// libfp8attn): the practical memory ceiling that the HBM-bound kernels of the library are
// measured against, and a read-only sweep that evicts the Infinity Cache without leaving
// dirty lines behind.
//
// stream_kernel reads `rd` 16-byte vectors per unit and writes `wr` (0 or 1) per unit,
// over `units` units, grid-stride with U units' loads in flight per thread:
//   rd = 1, wr = 0: read-only (the amax pass's pattern);
//   rd = 1, wr = 1: copy;
//   rd = 2, wr = 1: two bytes read per byte written (the quantise pass's pattern).
// A read-only sweep folds its data into one word per block so that nothing is dead code.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

template <int RD, int WR, int kUnroll>
__global__ __launch_bounds__(kThreads) void stream_kernel(const uint4* __restrict__ src,
                                                          uint4* __restrict__ dst,
                                                          int64_t units,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; u + (kUnroll - 1) * stride < units; u += kUnroll * stride) {
    uint4 r[kUnroll][RD];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j)
#pragma unroll
      for (int i = 0; i < RD; ++i) r[j][i] = src[(u + j * stride) * RD + i];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      if (WR == 0) {
#pragma unroll
        for (int i = 0; i < RD; ++i) acc ^= r[j][i].x ^ r[j][i].y ^ r[j][i].z ^ r[j][i].w;
      } else {
#pragma unroll
        for (int i = 0; i < WR; ++i) {
          uint4 w = r[j][i % RD];
          if (RD > WR) w.x ^= r[j][RD - 1].y;
          dst[(u + j * stride) * WR + i] = w;
        }
      }
    }
  }
  for (; u < units; u += stride) {
    uint4 r[RD];
#pragma unroll
    for (int i = 0; i < RD; ++i) r[i] = src[u * RD + i];
    if (WR == 0) {
#pragma unroll
      for (int i = 0; i < RD; ++i) acc ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
    } else {
#pragma unroll
      for (int i = 0; i < WR; ++i) {
        uint4 w = r[i % RD];
        if (RD > WR) w.x ^= r[RD - 1].y;
        dst[u * WR + i] = w;
      }
    }
  }
  if (WR == 0 && acc == 0x9e3779b9u) sink[blockIdx.x] = acc;   // keeps the reads live
}

template <int RD, int WR>
hipError_t launch(int unroll, int blocks, hipStream_t st, const uint4* s, uint4* d, int64_t units,
                  uint32_t* k) {
  if (unroll == 1)
    hipLaunchKernelGGL((stream_kernel<RD, WR, 1>), dim3(blocks), dim3(kThreads), 0, st, s, d, units, k);
  else if (unroll == 2)
    hipLaunchKernelGGL((stream_kernel<RD, WR, 2>), dim3(blocks), dim3(kThreads), 0, st, s, d, units, k);
  else if (unroll == 4)
    hipLaunchKernelGGL((stream_kernel<RD, WR, 4>), dim3(blocks), dim3(kThreads), 0, st, s, d, units, k);
  else
    hipLaunchKernelGGL((stream_kernel<RD, WR, 8>), dim3(blocks), dim3(kThreads), 0, st, s, d, units, k);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Stream `units` units of rd 16-byte reads and wr 16-byte writes with `blocks` blocks of 256
// threads (blocks <= 0: 2 per compute unit of the current device), each thread keeping
// `unroll` (1, 2, 4 or 8) units' loads in flight. src must hold units * rd and dst
// units * wr 16-byte vectors, both 16-byte aligned; sink holds `blocks` words (only the
// read-only form writes it, and practically never). Returns 0, -1 for an unsupported
// (rd, wr, unroll), or the HIP error code of the launch.
int stream_probe(const void* src, void* dst, int64_t units, int rd, int wr, int unroll,
                 int blocks, void* sink, void* stream) {
  if (units < 0 || (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8)) return -1;
  if (blocks <= 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return -1;
    blocks = 2 * cus;
  }
  const uint4* s = static_cast<const uint4*>(src);
  uint4* d = static_cast<uint4*>(dst);
  uint32_t* k = static_cast<uint32_t*>(sink);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (rd == 1 && wr == 0)
    e = launch<1, 0>(unroll, blocks, st, s, d, units, k);
  else if (rd == 1 && wr == 1)
    e = launch<1, 1>(unroll, blocks, st, s, d, units, k);
  else if (rd == 2 && wr == 1)
    e = launch<2, 1>(unroll, blocks, st, s, d, units, k);
  else
    return -1;
  return (int)e;
}

}  // extern "C"
