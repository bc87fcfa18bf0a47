// Per-tensor BF16 -> E4M3 quantisation of Q, K and V in one launch (vLLM-Omni "Quantized
// KV Cache", "Overview": Q/K/V are quantised on the fly right before the attention
// operator; vLLM docs "FP8 ViT Encoder Attention": per-tensor scales).
//
// q8 = E4M3(fp32(x * inv_scale[t])): one IEEE fp32 multiply, a clamp to +-448 (the
// converter would turn values beyond 464 into NaN), then the hardware RNE converter.
//
// Blocks [0, nb_qk) stream Q and K element-wise into [T][H][D] (16 bytes in, 8 out per
// thread step). Blocks [nb_qk, nb_qk + nb_v) each take one head and one 128-column tile
// of the padded key axis of V8t [H][D][Tp] (see fp8attn.h): they load 128 tokens x 128
// channels of V, quantise, transpose through LDS and write 128 channel rows of 128
// contiguous key bytes. Columns outside every sequence are written as 0 so the
// attention kernel can read whole tiles without bounds checks on V.
#include "device_common.h"
#include "launch.h"

namespace fp8attn {

namespace {

constexpr int kThreads = 256;
constexpr int kQkPerThread = 2;                                 // uint4 groups per thread
constexpr int kQkPerBlock = kThreads * kQkPerThread * 8;        // elements per block
constexpr int kVTile = 128;                                     // keys per V tile
constexpr int kLdsRow = kVTile + 16;                            // bytes per LDS row (16B aligned)

__device__ __forceinline__ uint2 quant8(uint4 r, float inv) {
  // 8 bf16 -> 8 E4M3 bytes, element order preserved
  int lo = cvt_pk_e4m3<false>(clamp_e4m3(bf16_lo(r.x) * inv), clamp_e4m3(bf16_hi(r.x) * inv), 0);
  lo = cvt_pk_e4m3<true>(clamp_e4m3(bf16_lo(r.y) * inv), clamp_e4m3(bf16_hi(r.y) * inv), lo);
  int hi = cvt_pk_e4m3<false>(clamp_e4m3(bf16_lo(r.z) * inv), clamp_e4m3(bf16_hi(r.z) * inv), 0);
  hi = cvt_pk_e4m3<true>(clamp_e4m3(bf16_lo(r.w) * inv), clamp_e4m3(bf16_hi(r.w) * inv), hi);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

__device__ __forceinline__ float bf16_at(const uint4& r, int c) {
  // channel c (0..7) of 8 packed bf16
  uint32_t w = c < 2 ? r.x : (c < 4 ? r.y : (c < 6 ? r.z : r.w));
  return (c & 1) ? bf16_hi(w) : bf16_lo(w);
}

__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const fp8attn_state* __restrict__ st, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu, int num_seqs, int64_t n, int H, uint8_t* __restrict__ q8,
    uint8_t* __restrict__ k8, uint8_t* __restrict__ v8t, int64_t Tp, int nb_qk) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kHeadDim * kLdsRow];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < nb_qk) {
    // ---- Q and K: element-wise stream over the concatenation [Q | K] of 2n elements
    const float inv_q = st->inv_scale[0];
    const float inv_k = st->inv_scale[1];
    const int64_t base = (int64_t)blockIdx.x * kQkPerBlock;
#pragma unroll
    for (int u = 0; u < kQkPerThread; ++u) {
      const int64_t e = base + ((int64_t)u * kThreads + tid) * 8;
      if (e >= 2 * n) break;
      const bool is_k = e >= n;                 // n is a multiple of 128: no group straddles
      const int64_t off = is_k ? e - n : e;
      const uint4 r = *reinterpret_cast<const uint4*>((is_k ? k : q) + off);
      const uint2 o = quant8(r, is_k ? inv_k : inv_q);
      *reinterpret_cast<uint2*>((is_k ? k8 : q8) + off) = o;
    }
    return;
  }
  // ---- V: one (padded key tile, head)
  const float inv_v = st->inv_scale[2];
  const int vb = (int)blockIdx.x - nb_qk;
  const int h = vb % H;
  const int64_t col0 = (int64_t)(vb / H) * kVTile;  // first padded key column of the tile
  // sequence whose padded region holds col0: largest i with pad_start(i) <= col0
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pad_start(cu[mid], mid) <= col0) lo = mid; else hi = mid - 1;
  }
  const int seq = lo;
  const int64_t seq_begin = cu[seq];
  const int64_t seq_len = (int64_t)cu[seq + 1] - seq_begin;
  const int64_t j0 = col0 - pad_start(seq_begin, seq);  // key offset inside the sequence

  // thread -> 4 consecutive keys x 16 channels; 8 threads cover one 256-byte token row
  const int cc = tid & 7;           // channel chunk: channels 16cc .. 16cc+15
  const int kg = tid >> 3;          // key group: keys 4kg .. 4kg+3 of the tile
  float x[4][16];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t j = j0 + 4 * kg + r;
    if (j < seq_len) {
      const uint16_t* src = v + ((seq_begin + j) * H + h) * kHeadDim + 16 * cc;
      const uint4 a = *reinterpret_cast<const uint4*>(src);
      const uint4 b = *reinterpret_cast<const uint4*>(src + 8);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        x[r][c] = clamp_e4m3(bf16_at(a, c) * inv_v);
        x[r][8 + c] = clamp_e4m3(bf16_at(b, c) * inv_v);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) x[r][c] = 0.0f;
    }
  }
  // Transpose through LDS: row = channel, one dword = 4 keys of one channel. The dword
  // column is XORed with 4 * (row / 16) so that the 8 channel chunks of a wave land in
  // different banks; 16-byte chunks stay contiguous (chunk' = chunk ^ (row / 16)).
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    int w = cvt_pk_e4m3<false>(x[0][c], x[1][c], 0);
    w = cvt_pk_e4m3<true>(x[2][c], x[3][c], w);
    const int row = 16 * cc + c;
    *reinterpret_cast<int*>(&tile[row * kLdsRow + 4 * (kg ^ (4 * cc))]) = w;
  }
  __syncthreads();
  // write 128 rows x 128 bytes: 8 threads per row, 16 bytes each, 4 rows per thread
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = it * 32 + (tid >> 3);
    const int chunk = tid & 7;
    const int pchunk = chunk ^ ((row >> 4) & 7);
    const uint4 d = *reinterpret_cast<const uint4*>(&tile[row * kLdsRow + 16 * pchunk]);
    *reinterpret_cast<uint4*>(v8t + ((int64_t)h * kHeadDim + row) * Tp + col0 + 16 * chunk) = d;
  }
}

}  // namespace

hipError_t launch_quantize(const fp8attn_state* st, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const int32_t* cu, int num_seqs, int64_t T,
                           int H, uint8_t* q8, uint8_t* k8, uint8_t* v8t, int64_t Tp,
                           hipStream_t s) {
  const int64_t n = T * H * kHeadDim;
  const int64_t nb_qk = (2 * n + kQkPerBlock - 1) / kQkPerBlock;
  const int64_t nb_v = (Tp / kVTile) * H;
  const int64_t blocks = nb_qk + nb_v;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, st, q, k,
                     v, cu, num_seqs, n, H, q8, k8, v8t, Tp, (int)nb_qk);
  return hipGetLastError();
}

}  // namespace fp8attn
