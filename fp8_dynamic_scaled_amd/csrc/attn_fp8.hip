// FP8 varlen non-causal flash-attention forward for gfx950 (CDNA4).
//
// What it computes (vLLM-Omni "Quantized KV Cache", "Overview"; vLLM docs "FP8 ViT
// Encoder Attention", first paragraph and "Performance"; Korean wiki "FP8 ViT 인코더
// 어텐션", "Requirements": varlen FP8 attention with per-tensor scales): for each packed
// sequence i, head h and query row r, over the keys j of sequence i only,
//   s_j  = (q8 . k8_j) * scale_q * scale_k * softmax_scale,
//   m    = running row maximum of s over the key tiles seen so far,
//   p8_j = E4M3(exp(s_j - m) * 448)          (fixed scale 448, so p8 <= 448),
//   O    = scale_v * sum_j p8_j v8_j / sum_j p8_j, rescaled by exp(m_old - m_new) when
//          the running maximum grows (online softmax), stored as bf16.
//
// Mapping onto the matrix cores (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulate):
//   * a block owns 128 queries of one (sequence, head); each of its 4 waves owns 32;
//   * scores are produced transposed, S^T = K Q^T, so that in the accumulator layout a
//     lane holds ONE query (column l % 32) and 16 keys per 32x32 block; the row maximum
//     is then a per-lane reduction plus one exchange with lane l ^ 32;
//   * the K rows of a tile are stored in LDS in a permuted order so that lane half g
//     ends up holding the 32 consecutive keys g*32 .. g*32+31 of the 64-key tile; the
//     packed E4M3 probabilities are then directly the B operand of O^T = V^T P^T, and the
//     A operand is 32 consecutive key bytes of one channel row of V8t (keys contiguous,
//     as written by the quantise kernel) -- no LDS round trip for P;
//   * O^T in the accumulator layout again puts one query per lane, so the online-softmax
//     rescale is a per-lane multiply; it is skipped for the whole wave when no lane's
//     maximum grew (exact: the factor would be 1);
//   * the row sum of the quantised weights comes from one extra MFMA with an all-ones
//     A operand (keeps it off the vector ALU, which the exp2 already saturates);
//   * K and V8t tiles are double-buffered in LDS with a register prefetch of the next
//     tile; LDS chunks are XOR-swizzled so operand reads are bank-conflict free;
//   * exp(x - m) * 448 is computed as exp2(s * c - (m * c - log2 448)), c = scales *
//     log2(e): one FMA and one v_exp_f32 per score;
//   * block -> work mapping is XCD-aware: consecutive work units (q-tiles of one
//     (sequence, head)) go to the same XCD so its L2 keeps that head's K/V.
#include "device_common.h"
#include "launch.h"

namespace fp8attn {

namespace {

constexpr int kBM = 128;                 // queries per block
constexpr int kBN = FP8ATTN_KV_BLOCK;     // keys per tile = online-softmax block
constexpr int kThreads = 256;
constexpr int kKTileBytes = kBN * kHeadDim;   // K tile: 64 rows x 128 B
constexpr int kVTileBytes = kHeadDim * kBN;   // V8t tile: 128 rows x 64 B
constexpr int kStageBytes = kKTileBytes + kVTileBytes;
constexpr uint32_t kOnesE4M3 = 0x38383838u;   // four E4M3 1.0

// LDS row of key kappa (0..63) in the K tile: the MFMA A row m of key block kb that
// yields, in the accumulator layout, key g*32 + kb*16 + i in register i of lane half g.
__device__ __forceinline__ int k_lds_row(int kappa) {
  const int g = kappa >> 5, kb = (kappa >> 4) & 1, i = kappa & 15;
  return kb * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
}

__device__ __forceinline__ v8i lds_load32(const uint8_t* p0, const uint8_t* p1) {
  const v4i a = *reinterpret_cast<const v4i*>(p0);
  const v4i b = *reinterpret_cast<const v4i*>(p1);
  v8i r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fp8_kernel(const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8,
                     const uint8_t* __restrict__ v8t, const int32_t* __restrict__ cu,
                     int num_seqs, int H, int64_t Tp, int qtiles, int units_per_xcd,
                     const fp8attn_state* __restrict__ st, float sm_scale,
                     uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];

  // ---- work unit: XCD-aware decode, q-tile fastest
  const int L = blockIdx.x;
  const int unit = (L & 7) * units_per_xcd + (L >> 3);
  const int qt = unit % qtiles;
  const int sh = unit / qtiles;
  const int head = sh % H;
  const int seq = sh / H;
  if (seq >= num_seqs) return;
  const int seq_begin = cu[seq];
  const int S = cu[seq + 1] - seq_begin;
  if (qt * kBM >= S) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int64_t row_stride = (int64_t)H * kHeadDim;

  // ---- Q^T operand (B of S^T = K Q^T): lane = query n, 32 channel bytes of half g
  const int q_local = qt * kBM + wave * 32 + n;
  const int q_row = seq_begin + (q_local < S ? q_local : S - 1);
  const uint8_t* qp = q8 + (int64_t)q_row * row_stride + head * kHeadDim;
  v8i qb[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const v4i a = *reinterpret_cast<const v4i*>(qp + s * 64 + g * 32);
    const v4i b = *reinterpret_cast<const v4i*>(qp + s * 64 + g * 32 + 16);
    qb[s][0] = a[0]; qb[s][1] = a[1]; qb[s][2] = a[2]; qb[s][3] = a[3];
    qb[s][4] = b[0]; qb[s][5] = b[1]; qb[s][6] = b[2]; qb[s][7] = b[3];
  }

  const float scale_q = st->scale[0], scale_k = st->scale[1], scale_v = st->scale[2];
  const float c = scale_q * scale_k * sm_scale * kLog2e;  // score -> log2 domain

  // ---- tile loaders: each thread moves 2 K chunks and 2 V8t chunks of 16 bytes
  const uint8_t* kbase = k8 + (int64_t)seq_begin * row_stride + head * kHeadDim;
  const uint8_t* vbase = v8t + (int64_t)head * kHeadDim * Tp + pad_start(seq_begin, seq);
  const int k_key0 = tid >> 3, k_ch = tid & 7;        // keys k_key0, k_key0 + 32
  const int v_row0 = tid >> 2, v_ch = tid & 3;        // channel rows v_row0, v_row0 + 64
  const int kR0 = k_lds_row(k_key0), kR1 = k_lds_row(k_key0 + 32);
  const int k_off0 = kR0 * kHeadDim + ((k_ch ^ (kR0 & 7)) << 4);
  const int k_off1 = kR1 * kHeadDim + ((k_ch ^ (kR1 & 7)) << 4);
  const int v_off0 = kKTileBytes + v_row0 * kBN + ((v_ch ^ ((v_row0 >> 1) & 3)) << 4);
  const int v_off1 = kKTileBytes + (v_row0 + 64) * kBN + ((v_ch ^ (((v_row0 + 64) >> 1) & 3)) << 4);
  const uint8_t* vsrc0 = vbase + (int64_t)v_row0 * Tp + (v_ch << 4);
  const uint8_t* vsrc1 = vbase + (int64_t)(v_row0 + 64) * Tp + (v_ch << 4);
  uint4 kreg0, kreg1, vreg0, vreg1;
#define FP8ATTN_LOAD_TILE(k0_)                                                              \
  do {                                                                                      \
    const int ka_ = (k0_) + k_key0 < S ? (k0_) + k_key0 : S - 1;                            \
    const int kb_ = (k0_) + k_key0 + 32 < S ? (k0_) + k_key0 + 32 : S - 1;                  \
    kreg0 = *reinterpret_cast<const uint4*>(kbase + (int64_t)ka_ * row_stride + (k_ch << 4)); \
    kreg1 = *reinterpret_cast<const uint4*>(kbase + (int64_t)kb_ * row_stride + (k_ch << 4)); \
    vreg0 = *reinterpret_cast<const uint4*>(vsrc0 + (k0_));                                 \
    vreg1 = *reinterpret_cast<const uint4*>(vsrc1 + (k0_));                                 \
  } while (0)
#define FP8ATTN_STORE_TILE(stage_)                                                          \
  do {                                                                                      \
    uint8_t* b_ = smem + (stage_) * kStageBytes;                                            \
    *reinterpret_cast<uint4*>(b_ + k_off0) = kreg0;                                         \
    *reinterpret_cast<uint4*>(b_ + k_off1) = kreg1;                                         \
    *reinterpret_cast<uint4*>(b_ + v_off0) = vreg0;                                         \
    *reinterpret_cast<uint4*>(b_ + v_off1) = vreg1;                                         \
  } while (0)

  // ---- per-lane state for query n
  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  v16f o[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[cb][i] = 0.0f;
  v8i ones;
#pragma unroll
  for (int r = 0; r < 8; ++r) ones[r] = (int)kOnesE4M3;
  const v16f zero16 = {};

  // lane-invariant parts of the operand addresses
  const int a_row = n;                                   // MFMA A row of this lane
  const int ntiles = (S + kBN - 1) / kBN;

  FP8ATTN_LOAD_TILE(0);
  FP8ATTN_STORE_TILE(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const bool has_next = t + 1 < ntiles;
    if (has_next) FP8ATTN_LOAD_TILE((t + 1) * kBN);
    const uint8_t* kt = smem + (t & 1) * kStageBytes;
    const uint8_t* vt = kt + kKTileBytes;

    // S^T = K Q^T for two 32-key blocks
    v16f sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int R = kb * 32 + a_row;
      const uint8_t* rowp = kt + R * kHeadDim;
      v16f acc = zero16;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c0 = s * 4 + g * 2;
        const v8i a = lds_load32(rowp + ((c0 ^ (R & 7)) << 4), rowp + (((c0 + 1) ^ (R & 7)) << 4));
        acc = mfma_e4m3_32x32x64(a, qb[s], acc);
      }
      sacc[kb] = acc;
    }

    // mask keys beyond the sequence (last tile only)
    const int k0 = t * kBN;
    if (k0 + kBN > S) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (k0 + g * 32 + kb * 16 + i >= S) sacc[kb][i] = -__builtin_inff();
    }

    // running maximum of this lane's query
    float mx = sacc[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = __builtin_fmaxf(mx, sacc[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, sacc[1][i]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = __builtin_fmaxf(m_run, mx);
    if (t > 0 && wave_any(m_new > m_run)) {
      const float alpha = fast_exp2((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[cb][i] *= alpha;
    }
    m_run = m_new;

    // p = exp(s - m) * 448 = exp2(s*c - (m*c - log2 448)), packed to E4M3
    const float mc = m_run * c - kLog2E4M3Max;
    v8i p;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int kb = r >> 2, i0 = (r & 3) * 4;
      const float e0 = fast_exp2(__builtin_fmaf(sacc[kb][i0 + 0], c, -mc));
      const float e1 = fast_exp2(__builtin_fmaf(sacc[kb][i0 + 1], c, -mc));
      const float e2 = fast_exp2(__builtin_fmaf(sacc[kb][i0 + 2], c, -mc));
      const float e3 = fast_exp2(__builtin_fmaf(sacc[kb][i0 + 3], c, -mc));
      int w = cvt_pk_e4m3<false>(e0, e1, 0);
      p[r] = cvt_pk_e4m3<true>(e2, e3, w);
    }

    // row sum of the quantised weights on the matrix core
    const v16f rs = mfma_e4m3_32x32x64(ones, p, zero16);
    l_run += rs[0];

    // O^T += V^T P^T over 4 blocks of 32 channels
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int R = cb * 32 + a_row;
      const uint8_t* rowp = vt + R * kBN;
      const int sw = (R >> 1) & 3;
      const v8i a = lds_load32(rowp + (((2 * g) ^ sw) << 4), rowp + (((2 * g + 1) ^ sw) << 4));
      o[cb] = mfma_e4m3_32x32x64(a, p, o[cb]);
    }

    if (has_next) FP8ATTN_STORE_TILE((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = O * scale_v / l, bf16, one query row per lane
  if (q_local < S) {
    const float f = scale_v / l_run;
    uint16_t* op = out + (int64_t)(seq_begin + q_local) * row_stride + head * kHeadDim;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        const f2 x0 = {o[cb][i4 * 4 + 0] * f, o[cb][i4 * 4 + 1] * f};
        const f2 x1 = {o[cb][i4 * 4 + 2] * f, o[cb][i4 * 4 + 3] * f};
        const b2 y0 = __builtin_convertvector(x0, b2);
        const b2 y1 = __builtin_convertvector(x1, b2);
        uint2 w;
        w.x = *reinterpret_cast<const uint32_t*>(&y0);
        w.y = *reinterpret_cast<const uint32_t*>(&y1);
        const int ch = cb * 32 + i4 * 8 + g * 4;
        *reinterpret_cast<uint2*>(op + ch) = w;
      }
  }
#undef FP8ATTN_LOAD_TILE
#undef FP8ATTN_STORE_TILE
}

}  // namespace

hipError_t launch_attn_fp8(const AttnLaunch& a, const fp8attn_state* st, const uint8_t* q8,
                           const uint8_t* k8, const uint8_t* v8t, hipStream_t s) {
  if (a.max_seqlen <= 0) return hipSuccess;
  const int qtiles = (a.max_seqlen + kBM - 1) / kBM;
  const int64_t units = (int64_t)a.num_seqs * a.H * qtiles;
  const int64_t per_xcd = (units + 7) / 8;
  if (per_xcd * 8 > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_fp8_kernel, dim3((unsigned)(per_xcd * 8)), dim3(kThreads), 0, s, q8,
                     k8, v8t, a.cu, a.num_seqs, a.H, a.Tp, qtiles, (int)per_xcd, st,
                     a.softmax_scale, a.out);
  return hipGetLastError();
}

}  // namespace fp8attn
