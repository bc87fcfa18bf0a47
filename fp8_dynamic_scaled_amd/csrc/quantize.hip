// Per-tensor BF16 -> E4M3 quantisation of Q, K and V in one launch (vLLM-Omni "Quantized
// KV Cache", "Overview": Q/K/V are quantised on the fly right before the attention
// operator; vLLM docs "FP8 ViT Encoder Attention": per-tensor scales, and in "Usage" the
// dynamic mode whose 16-slot amax ring drives every forward's scale).
//
// q8 = E4M3(fp32(x * inv_scale[t])): one IEEE fp32 multiply, a clamp to +-448 (the
// converter would turn values beyond 464 into NaN), then the hardware RNE converter.
//
// Work split (grid-stride, so the grid stays small whatever the batch): blocks
// [0, nb_qk) stream Q and K element-wise into [T][H][D] (two groups of 16 elements in
// flight per thread, each 32 bytes read and 16 written at once); blocks
// [nb_qk, nb_qk + nb_v) each take a contiguous run of (head, 128-column tile) pairs of the
// padded key axis of V8t [H][D][Tp] (see fp8attn.h), the tiles of one head consecutive,
// so that a block's successive tiles extend the same V8t rows and the sequence that holds
// a tile is found once per run and head and then stepped; each pair loads 128 tokens x 128
// channels of V, quantises, transposes through LDS and writes 128 channel rows of 128
// contiguous key bytes. Columns outside every sequence are written as 0 so the attention
// kernel can read whole tiles without bounds checks on V.
//
// Three modes share that kernel:
//  * kPlain: scale from the state (written by the scales kernel).
//  * kObserve (speculative dynamic forward): this forward's window maximum will be
//    A = max(A_pred, amax), A_pred = max of the ring slots other than the one its
//    observation replaces. The kernel quantises with A_pred's scale and, in the same pass
//    over the input, observes amax into the state's pending slot (as the amax kernel
//    does). The scales kernel then runs as usual.
//  * kRedo (after the scales kernel): re-quantises a tensor only when the scales kernel
//    recorded that its window maximum moved (this forward's amax exceeded A_pred);
//    otherwise its blocks return after one load.
// The bytes are therefore exactly those of amax + scales + plain quantise, while in steady
// state Q, K and V are read once instead of twice.
#include "device_common.h"
#include "launch.h"

namespace fp8attn {

namespace {

constexpr int kThreads = 256;
constexpr int kQkGroups = 2;                                    // 16-element groups per thread step
constexpr int kVTile = 128;                                     // keys per V tile
constexpr int kLdsRow = kVTile + 16;                            // bytes per LDS row (16B aligned)
constexpr int kMaxBlocksPerPart = 1024;                         // Q/K blocks, V blocks

enum QuantMode { kPlain = 0, kObserve = 1, kRedo = 2 };

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

// max of |x| over 8 packed bf16, as the 16-bit pattern with the sign cleared (which orders
// like the magnitude), folded into m
__device__ __forceinline__ uint32_t absmax8(uint32_t m, const uint4& r) {
  us2 a = {(unsigned short)(m), (unsigned short)(m)};
  const uint32_t w[4] = {r.x & 0x7fff7fffu, r.y & 0x7fff7fffu, r.z & 0x7fff7fffu,
                         r.w & 0x7fff7fffu};
#pragma unroll
  for (int i = 0; i < 4; ++i) a = __builtin_elementwise_max(a, *reinterpret_cast<const us2*>(&w[i]));
  return a.x > a.y ? a.x : a.y;
}

// Block-wide max of per-thread 16-bit magnitudes; thread 0 folds the result into the
// block's stripe of the pending observation state->cur (fp32 bit image, post_max).
__device__ __forceinline__ void publish_max(fp8attn_state* st, int t, uint32_t m, uint32_t* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(m, off);
    m = o > m ? o : m;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();                          // red may still be read from a previous call
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) b = red[w] > b ? red[w] : b;
    post_max(&st->cur[blockIdx.x % FP8ATTN_CUR_STRIPES][t], b << 16);
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    fp8attn_state* __restrict__ st, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu, int num_seqs, int64_t n, int H, uint8_t* __restrict__ q8,
    uint8_t* __restrict__ k8, uint8_t* __restrict__ v8t, int64_t Tp, int nb_qk, int nb_v) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kHeadDim * kLdsRow];
  __shared__ uint32_t red[kThreads / 64];
  const int tid = threadIdx.x;

  // ---- the scale of each tensor, and (re-quantise mode) which tensors need the work
  float inv[3];
  bool work[3] = {true, true, true};
  if (MODE == kObserve) {
    const uint32_t slot = st->count % FP8ATTN_RING_SLOTS;
#pragma unroll
    for (int t = 0; t < 3; ++t) inv[t] = inv_scale_from_amax(ring_max_except(st, t, slot));
  } else {
#pragma unroll
    for (int t = 0; t < 3; ++t) inv[t] = st->inv_scale[t];
    if (MODE == kRedo) {
      const uint32_t moved = st->moved;             // written by the scales kernel
#pragma unroll
      for (int t = 0; t < 3; ++t) work[t] = (moved >> t) & 1u;
    }
  }

  if ((int)blockIdx.x < nb_qk) {
    // ---- Q and K: element-wise stream over the concatenation [Q | K] of 2n elements
    if (MODE == kRedo && !work[0] && !work[1]) return;
    const int64_t groups = 2 * n / 16;                // n is a multiple of 128
    const int64_t step = (int64_t)nb_qk * kThreads * kQkGroups;
    uint32_t mq = 0, mk = 0;
    for (int64_t g0 = (int64_t)blockIdx.x * kThreads * kQkGroups; g0 < groups; g0 += step) {
      uint4 r[kQkGroups][2];
#pragma unroll
      for (int u = 0; u < kQkGroups; ++u) {
        const int64_t g = g0 + u * kThreads + tid;
        if (g < groups) {
          const int64_t e = g * 16;
          const bool is_k = e >= n;
          const uint4* p = reinterpret_cast<const uint4*>((is_k ? k : q) + (is_k ? e - n : e));
          r[u][0] = p[0];
          r[u][1] = p[1];
        }
      }
#pragma unroll
      for (int u = 0; u < kQkGroups; ++u) {
        const int64_t g = g0 + u * kThreads + tid;
        if (g < groups) {
          const int64_t e = g * 16;
          const bool is_k = e >= n;
          if (MODE == kObserve) {
            if (is_k) mk = absmax8(absmax8(mk, r[u][0]), r[u][1]);
            else mq = absmax8(absmax8(mq, r[u][0]), r[u][1]);
          }
          if (MODE != kRedo || work[is_k ? 1 : 0]) {
            const uint2 a = quant8(r[u][0], inv[is_k ? 1 : 0]);
            const uint2 b = quant8(r[u][1], inv[is_k ? 1 : 0]);
            *reinterpret_cast<uint4*>((is_k ? k8 : q8) + (is_k ? e - n : e)) =
                make_uint4(a.x, a.y, b.x, b.y);
          }
        }
      }
    }
    if (MODE == kObserve) {
      publish_max(st, 0, mq, red);
      publish_max(st, 1, mk, red);
    }
    return;
  }

  // ---- V: (head, padded key tile) pairs; each block takes a contiguous run of them, in
  // which, within one head, the key tile -- and so the sequence -- only moves forward
  if (MODE == kRedo && !work[2]) return;
  const float inv_v = inv[2];
  const int64_t tiles = (Tp / kVTile) * H;
  const int64_t run = (tiles + nb_v - 1) / nb_v;
  const int64_t vb_begin = ((int64_t)blockIdx.x - nb_qk) * run;
  const int64_t vb_end = vb_begin + run < tiles ? vb_begin + run : tiles;
  const int cc = tid & 7;           // channel chunk: channels 16cc .. 16cc+15
  const int kg = tid >> 3;          // key group: keys 4kg .. 4kg+3 of the tile
  uint32_t mv = 0;
  int seq = -1;
  for (int64_t vb = vb_begin; vb < vb_end; ++vb) {
    const int64_t ntile = Tp / kVTile;
    const int h = (int)(vb / ntile);
    const int64_t col0 = (vb % ntile) * kVTile;      // first padded key column of the tile
    if (col0 == 0) seq = -1;                         // a new head: search again
    // sequence whose padded region holds col0: the largest i with pad_start(i) <= col0
    // (starts increase strictly); a binary search for the run's first tile, then steps
    if (seq < 0) {
      int lo = 0, hi = num_seqs - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pad_start(cu[mid], mid) <= col0) lo = mid; else hi = mid - 1;
      }
      seq = lo;
    } else {
      while (seq + 1 < num_seqs && pad_start(cu[seq + 1], seq + 1) <= col0) ++seq;
    }
    const int64_t seq_begin = cu[seq];
    const int64_t seq_len = (int64_t)cu[seq + 1] - seq_begin;
    const int64_t j0 = col0 - pad_start(seq_begin, seq);  // key offset inside the sequence

    // thread -> 4 consecutive keys x 16 channels; 8 threads cover one 256-byte token row
    float x[4][16];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t j = j0 + 4 * kg + r;
      if (j < seq_len) {
        const uint16_t* src = v + ((seq_begin + j) * H + h) * kHeadDim + 16 * cc;
        const uint4 a = *reinterpret_cast<const uint4*>(src);
        const uint4 b = *reinterpret_cast<const uint4*>(src + 8);
        if (MODE == kObserve) mv = absmax8(absmax8(mv, a), b);
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
    __syncthreads();                      // the tile buffer is rewritten by the next pair
  }
  if (MODE == kObserve) publish_max(st, 2, mv, red);
}

template <int MODE>
hipError_t launch_mode(fp8attn_state* st, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const int32_t* cu, int num_seqs, int64_t T, int H,
                       uint8_t* q8, uint8_t* k8, uint8_t* v8t, int64_t Tp, hipStream_t s) {
  const int64_t n = T * H * kHeadDim;
  const int64_t per_block = (int64_t)kThreads * kQkGroups * 16;
  int64_t nb_qk = (2 * n + per_block - 1) / per_block;
  // the re-quantise pass keeps the full grid: when it works (the first forward of a layer,
  // or a new window maximum -- with amax varying between forwards, one of Q/K/V does so in
  // several forwards of 16) it must run at full speed, and its blocks exit after one load
  // when it does not
  const int64_t cap = kMaxBlocksPerPart;
  if (nb_qk > cap) nb_qk = cap;
  int64_t nb_v = (Tp / kVTile) * H;
  if (nb_v > cap) nb_v = cap;
  // A small batch (few V tiles) gets one round of resident blocks (4 waves per SIMD: 4
  // blocks per CU, 1024 on the chip) instead of a partial second round: its Q/K blocks take
  // more groups each. 3 x 784 tokens x 16 heads: 15.9 -> 14.7 us per dynamic forward.
  constexpr int64_t kOneRound = 1024;
  if (nb_qk + nb_v > kOneRound && nb_v < kOneRound - 64) nb_qk = kOneRound - nb_v;
  if (nb_qk + nb_v <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_kernel<MODE>, dim3((unsigned)(nb_qk + nb_v)), dim3(kThreads), 0,
                     s, st, q, k, v, cu, num_seqs, n, H, q8, k8, v8t, Tp, (int)nb_qk,
                     (int)nb_v);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const fp8attn_state* st, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const int32_t* cu, int num_seqs, int64_t T,
                           int H, uint8_t* q8, uint8_t* k8, uint8_t* v8t, int64_t Tp,
                           hipStream_t s) {
  // the plain mode only reads the state
  return launch_mode<kPlain>(const_cast<fp8attn_state*>(st), q, k, v, cu, num_seqs, T, H, q8,
                             k8, v8t, Tp, s);
}

hipError_t launch_quantize_dynamic(fp8attn_state* st, const uint16_t* q, const uint16_t* k,
                                   const uint16_t* v, const int32_t* cu, int num_seqs,
                                   int64_t T, int H, uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                                   int64_t Tp, hipStream_t s) {
  hipError_t e = launch_mode<kObserve>(st, q, k, v, cu, num_seqs, T, H, q8, k8, v8t, Tp, s);
  if (e != hipSuccess) return e;
  e = launch_scales(st, FP8ATTN_DYNAMIC, nullptr, 0.0f, s);
  if (e != hipSuccess) return e;
  return launch_mode<kRedo>(st, q, k, v, cu, num_seqs, T, H, q8, k8, v8t, Tp, s);
}

}  // namespace fp8attn
