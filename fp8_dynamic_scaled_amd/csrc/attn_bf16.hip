// BF16 varlen non-causal flash-attention forward for gfx950: the native-dtype path of
// the step/layer skip selectors (vLLM-Omni "Quantized KV Cache", "Overview": attention
// runs in the native dtype when FP8 is not requested; "Parameters": listed steps or
// layers stay in the native dtype) and the same-hardware baseline of the FP8 kernel.
//
// O = softmax(Q K^T * softmax_scale) V per packed sequence with fp32 accumulation and an
// fp32 online softmax; P is rounded to bf16 for the PV product, and the row sum is the
// fp32 sum of the unrounded P.
//
// Same schedule as the FP8 kernel (128 queries per block, 4 waves of 32, 64-key tiles
// double-buffered in LDS, S^T = K Q^T so one lane owns one query, permuted K rows so
// that lane half g holds keys g*32 .. g*32+31, XCD-aware block mapping), on
// v_mfma_f32_32x32x16_bf16. The caller's V is token-major ([T][H][D]); the PV product
// needs keys along k, so each tile of V is transposed while it is written to LDS
// (4 keys x 8 channels per thread, packed into 8-byte channel rows).
#include "device_common.h"
#include "launch.h"

namespace fp8attn {

namespace {

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;
constexpr int kRowBytes = kHeadDim * 2;               // 256 B per token row (bf16)
constexpr int kKTileBytes = kBN * kRowBytes;          // 16 KB
constexpr int kVRowBytes = kBN * 2;                   // 128 B per channel row of V^T
constexpr int kVTileBytes = kHeadDim * kVRowBytes;    // 16 KB
constexpr int kStageBytes = kKTileBytes + kVTileBytes;

__device__ __forceinline__ int k_lds_row(int kappa) {
  const int g = kappa >> 5, kb = (kappa >> 4) & 1, i = kappa & 15;
  return kb * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
}

// swizzle of the 16-byte chunks of a V^T row (8 chunks of 128 B rows)
__device__ __forceinline__ int v_swz(int row) { return (row ^ (row >> 3)) & 7; }

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f2 x = {a, b};
  const b2 y = __builtin_convertvector(x, b2);
  return *reinterpret_cast<const uint32_t*>(&y);
}

// Write 4 keys x 8 channels of V (vreg r = key 4*kq + r, channels 8*cc .. 8*cc+7) into
// the V^T tile: 8 channel rows, each receiving the 4 keys as one 8-byte run.
__device__ __forceinline__ void store_vt(uint8_t* vt, const uint4& r0, const uint4& r1,
                                         const uint4& r2, const uint4& r3, int cc, int kq) {
  const uint32_t a0[4] = {r0.x, r0.y, r0.z, r0.w};
  const uint32_t a1[4] = {r1.x, r1.y, r1.z, r1.w};
  const uint32_t a2[4] = {r2.x, r2.y, r2.z, r2.w};
  const uint32_t a3[4] = {r3.x, r3.y, r3.z, r3.w};
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const int d = x >> 1;
    const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;  // high or low bf16 halves
    uint2 pk;
    pk.x = __builtin_amdgcn_perm(a1[d], a0[d], sel);
    pk.y = __builtin_amdgcn_perm(a3[d], a2[d], sel);
    const int row = 8 * cc + x;
    const int off = row * kVRowBytes + (((kq >> 1) ^ v_swz(row)) << 4) + ((kq & 1) << 3);
    *reinterpret_cast<uint2*>(vt + off) = pk;
  }
}

__device__ __forceinline__ v8bf as_v8bf(const uint4& u) {
  return *reinterpret_cast<const v8bf*>(&u);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                      const uint16_t* __restrict__ v, const int32_t* __restrict__ cu,
                      int num_seqs, int H, int qtiles, int units_per_xcd, float sm_scale,
                      uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];

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
  const int64_t row_stride = (int64_t)H * kHeadDim;   // elements

  // ---- Q^T operand: 8 k-steps of 16 channels; lane half g holds channels s*16+g*8..+7
  const int q_local = qt * kBM + wave * 32 + n;
  const int q_row = seq_begin + (q_local < S ? q_local : S - 1);
  const uint16_t* qp = q + (int64_t)q_row * row_stride + head * kHeadDim;
  uint4 qb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qb[s] = *reinterpret_cast<const uint4*>(qp + s * 16 + g * 8);

  const float c = sm_scale * kLog2e;

  // ---- tile loaders
  const uint16_t* kbase = k + (int64_t)seq_begin * row_stride + head * kHeadDim;
  const uint16_t* vbase = v + (int64_t)seq_begin * row_stride + head * kHeadDim;
  // K: 64 keys x 16 chunks; thread -> chunk k_ch of keys k_key0 + 16 j (j = 0..3)
  const int k_key0 = tid >> 4, k_ch = tid & 15;
  const int kR0 = k_lds_row(k_key0), kR1 = k_lds_row(k_key0 + 16);
  const int kR2 = k_lds_row(k_key0 + 32), kR3 = k_lds_row(k_key0 + 48);
  const int k_off0 = kR0 * kRowBytes + ((k_ch ^ (kR0 & 7)) << 4);
  const int k_off1 = kR1 * kRowBytes + ((k_ch ^ (kR1 & 7)) << 4);
  const int k_off2 = kR2 * kRowBytes + ((k_ch ^ (kR2 & 7)) << 4);
  const int k_off3 = kR3 * kRowBytes + ((k_ch ^ (kR3 & 7)) << 4);
  // V: thread -> keys 4*v_kq .. +3, channels 8*v_cc .. +7 (16 threads cover a token row)
  const int v_cc = tid & 15, v_kq = tid >> 4;
  uint4 kreg0, kreg1, kreg2, kreg3, vreg0, vreg1, vreg2, vreg3;
#define FP8ATTN_KROW(k_) (kbase + (int64_t)((k_) < S ? (k_) : S - 1) * row_stride + k_ch * 8)
#define FP8ATTN_VROW(k_) (vbase + (int64_t)((k_) < S ? (k_) : S - 1) * row_stride + v_cc * 8)
#define FP8ATTN_LOAD_TILE(k0_)                                                           \
  do {                                                                                   \
    kreg0 = *reinterpret_cast<const uint4*>(FP8ATTN_KROW((k0_) + k_key0));               \
    kreg1 = *reinterpret_cast<const uint4*>(FP8ATTN_KROW((k0_) + k_key0 + 16));          \
    kreg2 = *reinterpret_cast<const uint4*>(FP8ATTN_KROW((k0_) + k_key0 + 32));          \
    kreg3 = *reinterpret_cast<const uint4*>(FP8ATTN_KROW((k0_) + k_key0 + 48));          \
    vreg0 = *reinterpret_cast<const uint4*>(FP8ATTN_VROW((k0_) + 4 * v_kq + 0));         \
    vreg1 = *reinterpret_cast<const uint4*>(FP8ATTN_VROW((k0_) + 4 * v_kq + 1));         \
    vreg2 = *reinterpret_cast<const uint4*>(FP8ATTN_VROW((k0_) + 4 * v_kq + 2));         \
    vreg3 = *reinterpret_cast<const uint4*>(FP8ATTN_VROW((k0_) + 4 * v_kq + 3));         \
  } while (0)
#define FP8ATTN_STORE_TILE(stage_)                                                       \
  do {                                                                                   \
    uint8_t* b_ = smem + (stage_) * kStageBytes;                                         \
    *reinterpret_cast<uint4*>(b_ + k_off0) = kreg0;                                      \
    *reinterpret_cast<uint4*>(b_ + k_off1) = kreg1;                                      \
    *reinterpret_cast<uint4*>(b_ + k_off2) = kreg2;                                      \
    *reinterpret_cast<uint4*>(b_ + k_off3) = kreg3;                                      \
    store_vt(b_ + kKTileBytes, vreg0, vreg1, vreg2, vreg3, v_cc, v_kq);                  \
  } while (0)

  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  v16f o[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[cb][i] = 0.0f;
  const v16f zero16 = {};
  const int ntiles = (S + kBN - 1) / kBN;

  FP8ATTN_LOAD_TILE(0);
  FP8ATTN_STORE_TILE(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const bool has_next = t + 1 < ntiles;
    if (has_next) FP8ATTN_LOAD_TILE((t + 1) * kBN);
    const uint8_t* kt = smem + (t & 1) * kStageBytes;
    const uint8_t* vt = kt + kKTileBytes;

    v16f sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int R = kb * 32 + n;
      const uint8_t* rowp = kt + R * kRowBytes;
      v16f acc = zero16;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint4 a = *reinterpret_cast<const uint4*>(rowp + (((2 * s + g) ^ (R & 7)) << 4));
        acc = mfma_bf16_32x32x16(as_v8bf(a), as_v8bf(qb[s]), acc);
      }
      sacc[kb] = acc;
    }

    const int k0 = t * kBN;
    if (k0 + kBN > S) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (k0 + g * 32 + kb * 16 + i >= S) sacc[kb][i] = -__builtin_inff();
    }

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

    // P^T operand: k-step ks covers keys g*32 + ks*8 .. +7 = sacc[ks/2][(ks%2)*8 ..]
    const float mc = m_run * c;
    uint4 pb[4];
    float psum = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = ks >> 1, i0 = (ks & 1) * 8;
      float e[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        e[x] = fast_exp2(__builtin_fmaf(sacc[kb][i0 + x], c, -mc));
        psum += e[x];
      }
      pb[ks].x = pack_bf16(e[0], e[1]);
      pb[ks].y = pack_bf16(e[2], e[3]);
      pb[ks].z = pack_bf16(e[4], e[5]);
      pb[ks].w = pack_bf16(e[6], e[7]);
    }
    psum += __shfl_xor(psum, 32);
    l_run += psum;

#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int R = cb * 32 + n;
      const uint8_t* rowp = vt + R * kVRowBytes;
      const int sw = v_swz(R);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(rowp + (((4 * g + ks) ^ sw) << 4));
        o[cb] = mfma_bf16_32x32x16(as_v8bf(a), as_v8bf(pb[ks]), o[cb]);
      }
    }

    if (has_next) FP8ATTN_STORE_TILE((t + 1) & 1);
    __syncthreads();
  }

  if (q_local < S) {
    const float f = 1.0f / l_run;
    uint16_t* op = out + (int64_t)(seq_begin + q_local) * row_stride + head * kHeadDim;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        uint2 w;
        w.x = pack_bf16(o[cb][i4 * 4 + 0] * f, o[cb][i4 * 4 + 1] * f);
        w.y = pack_bf16(o[cb][i4 * 4 + 2] * f, o[cb][i4 * 4 + 3] * f);
        *reinterpret_cast<uint2*>(op + cb * 32 + i4 * 8 + g * 4) = w;
      }
  }
#undef FP8ATTN_KROW
#undef FP8ATTN_VROW
#undef FP8ATTN_LOAD_TILE
#undef FP8ATTN_STORE_TILE
}

}  // namespace

hipError_t launch_attn_bf16(const AttnLaunch& a, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, hipStream_t s) {
  if (a.max_seqlen <= 0) return hipSuccess;
  const int qtiles = (a.max_seqlen + kBM - 1) / kBM;
  const int64_t units = (int64_t)a.num_seqs * a.H * qtiles;
  const int64_t per_xcd = (units + 7) / 8;
  if (per_xcd * 8 > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_bf16_kernel, dim3((unsigned)(per_xcd * 8)), dim3(kThreads), 0, s, q,
                     k, v, a.cu, a.num_seqs, a.H, qtiles, (int)per_xcd, a.softmax_scale,
                     a.out);
  return hipGetLastError();
}

}  // namespace fp8attn
