// BF16 varlen non-causal flash-attention forward for gfx950: the native-dtype path of
// the step/layer skip selectors (vLLM-Omni "Quantized KV Cache", "Overview": attention
// runs in the native dtype when FP8 is not requested; "Parameters": listed steps or
// layers stay in the native dtype) and the same-hardware baseline of the FP8 kernel.
//
// O = softmax(Q K^T * softmax_scale) V per packed sequence with fp32 accumulation and an
// fp32 online softmax over 64-key tiles; P is rounded to bf16 for the PV product and the
// row sum is the fp32 sum of those rounded weights (so the weights used sum to 1).
//
// Mapping onto the matrix cores (v_mfma_f32_32x32x16_bf16, 8 k-steps of 16 channels per
// 32-key block):
//   * a block owns 128 queries of one (sequence, head), 4 waves of 32 queries; scores are
//     produced transposed, S^T = K Q^T, so one lane holds one query; the K rows of a tile
//     sit in LDS in the permuted order of the FP8 kernel, so lane half g holds keys
//     g*32 .. g*32+31 and the bf16-packed P is directly the B operand of O^T = V^T P^T;
//   * V stays token-major in LDS: the A operand of the PV product (8 consecutive keys of
//     one channel per lane) is read with ds_read_b64_tr_b16, which transposes 16x4 blocks
//     of 16-bit elements across each group of 16 lanes -- output lane i, element r is
//     element i % 4 of the 8 bytes addressed by lane 4r + i/4 -- so lane 4r + q points
//     at 4 channels of key r and every lane receives 4 keys of one channel;
//   * K and V tiles go global -> LDS with buffer loads that write LDS directly, two-stage
//     rings, one barrier per tile; rows past the end of the sequence read as zero;
//   * the same software pipeline as the FP8 kernel: iteration t runs the softmax of tile
//     t on the vector ALU while the matrix core runs PV of tile t-1 and the scores of
//     tile t+1 (here 32 MFMAs per tile: at d = 128 the BF16 matrix core, not the vector
//     ALU, is the bound); the region is written in issue order, groups of 4 MFMAs each
//     followed by one softmax chunk, kept in place by sched_barrier; the loop runs in
//     pairs of tiles so every LDS stage offset is an instruction immediate;
//   * the rescale for tile t-1's maximum runs at the top of iteration t; it is skipped for
//     the whole wave when no lane's maximum grew; XCD-aware block -> work mapping.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace fp8attn {

namespace {

constexpr int kBM = 128;                     // queries per block
constexpr int kBN = 64;                      // keys per tile
constexpr int kThreads = 256;
constexpr int kRowBytes = kHeadDim * 2;      // 256 B per token row (bf16)
constexpr int kTileBytes = kBN * kRowBytes;  // 16 KB per K or V tile
constexpr int kKBase = 0;                    // K stages at [0, 32 KB)
constexpr int kVBase = 2 * kTileBytes;       // V stages at [32 KB, 64 KB)
constexpr int kBufferFlags = 0x00020000;     // raw buffer resource, dword 3 (gfx9)

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4s lds_v4s;

// LDS row of key kappa (0..63) in the K tile and its inverse (same order as the FP8
// kernel: S^T register i of block kb in lane half g is key g*32 + kb*16 + i).
__device__ __forceinline__ int k_row_key(int R) {
  const int kb = R >> 5, m = R & 31;
  return ((m >> 2) & 1) * 32 + kb * 16 + (m >> 3) * 4 + (m & 3);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f2 x = {a, b};
  const b2 y = __builtin_convertvector(x, b2);
  return *reinterpret_cast<const uint32_t*>(&y);
}

__device__ __forceinline__ v8bf as_v8bf(const uint4& u) { return *reinterpret_cast<const v8bf*>(&u); }

typedef uint32_t v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 join(const v4s& a, const v4s& b) {
  const v2u x = __builtin_bit_cast(v2u, a), y = __builtin_bit_cast(v2u, b);
  return make_uint4(x[0], x[1], y[0], y[1]);
}

// Maximum over the two lane halves (lanes l and l ^ 32 hold the two key halves).
__device__ __forceinline__ float half_swap_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Scores i0 .. i0+3 of a 16-score block -> 2 dwords of bf16 weights exp2(s*c - mc); the
// weights as rounded are added to psum (fp32 dot product with ones).
__device__ __forceinline__ uint2 quant4(const v16f& s, int i0, float c, float mc, float& psum) {
  uint2 w;
  w.x = pack_bf16(fast_exp2(__builtin_fmaf(s[i0], c, -mc)), fast_exp2(__builtin_fmaf(s[i0 + 1], c, -mc)));
  w.y = pack_bf16(fast_exp2(__builtin_fmaf(s[i0 + 2], c, -mc)), fast_exp2(__builtin_fmaf(s[i0 + 3], c, -mc)));
  const b2 one = {(__bf16)1.0f, (__bf16)1.0f};
  psum = __builtin_amdgcn_fdot2_f32_bf16(*reinterpret_cast<const b2*>(&w.x), one, psum, false);
  psum = __builtin_amdgcn_fdot2_f32_bf16(*reinterpret_cast<const b2*>(&w.y), one, psum, false);
  return w;
}

// The same for a masked tile: keys at or past key_lim get weight 0 (exp2 of -inf; the
// argument, not the score, is replaced).
__device__ __forceinline__ uint2 quant4_masked(const v16f& s, int i0, int key0, int key_lim,
                                               float c, float mc, float& psum) {
  float e[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const float a = __builtin_fmaf(s[i0 + x], c, -mc);
    e[x] = fast_exp2(key0 + x >= key_lim ? -__builtin_inff() : a);
  }
  uint2 w;
  w.x = pack_bf16(e[0], e[1]);
  w.y = pack_bf16(e[2], e[3]);
  const b2 one = {(__bf16)1.0f, (__bf16)1.0f};
  psum = __builtin_amdgcn_fdot2_f32_bf16(*reinterpret_cast<const b2*>(&w.x), one, psum, false);
  psum = __builtin_amdgcn_fdot2_f32_bf16(*reinterpret_cast<const b2*>(&w.y), one, psum, false);
  return w;
}

// Wait for this thread's older LDS-bound loads, then a bare barrier (see the FP8 kernel:
// __syncthreads' fence would wait for every outstanding load).
__device__ __forceinline__ void loads_barrier() {
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void pin(const uint4* p) {
  asm volatile("" ::"v"(p[0].x), "v"(p[0].y), "v"(p[0].z), "v"(p[0].w), "v"(p[1].x),
               "v"(p[1].y), "v"(p[1].z), "v"(p[1].w));
  asm volatile("" ::"v"(p[2].x), "v"(p[2].y), "v"(p[2].z), "v"(p[2].w), "v"(p[3].x),
               "v"(p[3].y), "v"(p[3].z), "v"(p[3].w));
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                      const uint16_t* __restrict__ v, const int32_t* __restrict__ cu,
                      int num_seqs, int H, int vtiles, int units_per_xcd, float sm_scale,
                      uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kTileBytes];

  // ---- work unit: XCD-aware decode, virtual tile fastest (vtile_seq), then head
  const int L = blockIdx.x;
  const int unit = (L & 7) * units_per_xcd + (L >> 3);
  const int vt = unit % vtiles;
  const int head = unit / vtiles;
  if (head >= H) return;
  const int seq = vtile_seq(cu, num_seqs, vt);
  const int qt = vt - vtile_start(cu, seq);
  const int seq_begin = cu[seq];
  const int S = cu[seq + 1] - seq_begin;
  if (qt * kBM >= S) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int row_bytes = H * kRowBytes;                  // bytes per token row of Q/K/V
  const int ntiles = (S + kBN - 1) / kBN;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // ---- tile loaders (buffer loads into LDS; lane L of a wave's instruction fills bytes
  // 16 L of a 1 KB run = 4 rows of 256 B; wave w fills rows 16 w .. 16 w + 15)
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(k) + (int64_t)seq_begin * row_bytes + head * kRowBytes;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(v) + (int64_t)seq_begin * row_bytes + head * kRowBytes;
  int kvo[4], vvo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int R = 16 * wv + 4 * i + (lane >> 4);       // LDS row
    const int pc = lane & 15;                          // physical 16-byte chunk
    kvo[i] = k_row_key(R) * row_bytes + ((pc ^ (R & 15)) << 4);
    vvo[i] = R * row_bytes + ((pc ^ ((R & 3) << 2)) << 4);
  }
  auto load_k = [&](int j, int stage) __attribute__((always_inline)) {
    const int k0 = (j < ntiles ? j : ntiles - 1) * kBN;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (int64_t)k0 * row_bytes), (short)0, (S - k0) * row_bytes, kBufferFlags);
    uint8_t* dst = smem + kKBase + stage * kTileBytes + wv * 4096;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + 1024 * i), 16, kvo[i], 0, 0, 0);
  };
  auto load_v = [&](int j, int stage) __attribute__((always_inline)) {
    const int k0 = (j < ntiles ? j : ntiles - 1) * kBN;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (int64_t)k0 * row_bytes), (short)0, (S - k0) * row_bytes, kBufferFlags);
    uint8_t* dst = smem + kVBase + stage * kTileBytes + wv * 4096;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + 1024 * i), 16, vvo[i], 0, 0, 0);
  };
  load_k(0, 0);
  load_k(1, 1);

  // ---- Q^T operand: 8 k-steps of 16 channels; lane half g holds channels s*16+g*8..+7
  const int q_local = qt * kBM + wave * 32 + n;
  const int q_row = seq_begin + (q_local < S ? q_local : S - 1);
  const uint16_t* qp = q + (int64_t)q_row * H * kHeadDim + head * kHeadDim;
  uint4 qb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qb[s] = *reinterpret_cast<const uint4*>(qp + s * 16 + g * 8);
  const float c = sm_scale * kLog2e;

  // ---- per-lane LDS read addresses (stage and block offsets are immediates)
  // K operand (A of S^T): row R = kb*32 + n, logical chunk 2s + g, physical chunk
  // (2s + g) ^ (R & 15) = 2 (s ^ (x >> 1)) + (g ^ (x & 1)) with x = n & 15
  const int xk = n & 15;
  const int kaddr0 = n * kRowBytes + ((g ^ (xk & 1)) << 4);
  int kaddr[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kaddr[s] = kaddr0 + ((s ^ (xk >> 1)) << 5);
  // V operand (A of O^T, transposed read): 16-lane group G -> channels m0 = (G&1)*16 of the
  // 32-channel block, keys kh*32.. (kh = G >> 1); lane 4r + q of the group points at key
  // r (+ 8 ks + 4 half) and channels m0 + 4q .. m0 + 4q + 3 of block cb; chunk swizzle of
  // V rows is XOR ((key & 3) << 2) = 4r, so block cb sits in chunk group cb ^ r.
  const int gi = lane & 15, G = lane >> 4;
  const int vr = gi >> 2, vq = gi & 3;
  const int vaddr0 = ((G >> 1) * 32 + vr) * kRowBytes + ((((G & 1) * 2) + (vq >> 1)) << 4) + ((vq & 1) << 3);
  int vaddr[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) vaddr[cb] = vaddr0 + ((cb ^ vr) << 6);

  auto ldsk = [&](int stage, int kb, int s) __attribute__((always_inline)) {
    return *reinterpret_cast<const uint4*>(smem + kKBase + stage * kTileBytes +
                                           kb * 32 * kRowBytes + kaddr[s]);
  };
  auto ldsv = [&](int stage, int cb, int ks) __attribute__((always_inline)) {
    const __attribute__((address_space(3))) uint8_t* b =
        (const __attribute__((address_space(3))) uint8_t*)smem + kVBase + stage * kTileBytes +
        ks * 8 * kRowBytes + vaddr[cb];
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)b);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(b + 4 * kRowBytes));
    return join(lo, hi);
  };

  // ---- per-lane state
  float m_prev = -__builtin_inff(), m_ref = -__builtin_inff();
  float l_run = 0.0f, ps_prev = 0.0f;
  v16f o0 = {}, o1 = {}, o2 = {}, o3 = {};
  v16f sa0, sa1, sb0, sb1;
  uint4 p_prev[4];
  const v16f zero16 = {};
  const int last_lim = S - (ntiles - 1) * kBN;

  auto scores = [&](int stage, v16f& s0, v16f& s1) __attribute__((always_inline)) {
    s0 = zero16;
    s1 = zero16;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      s0 = mfma_bf16_32x32x16(as_v8bf(ldsk(stage, 0, s)), as_v8bf(qb[s]), s0);
      s1 = mfma_bf16_32x32x16(as_v8bf(ldsk(stage, 1, s)), as_v8bf(qb[s]), s1);
    }
  };
  auto pv = [&](int stage, const uint4* p) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      o0 = mfma_bf16_32x32x16(as_v8bf(ldsv(stage, 0, ks)), as_v8bf(p[ks]), o0);
      o1 = mfma_bf16_32x32x16(as_v8bf(ldsv(stage, 1, ks)), as_v8bf(p[ks]), o1);
      o2 = mfma_bf16_32x32x16(as_v8bf(ldsv(stage, 2, ks)), as_v8bf(p[ks]), o2);
      o3 = mfma_bf16_32x32x16(as_v8bf(ldsv(stage, 3, ks)), as_v8bf(p[ks]), o3);
    }
  };
  auto catch_up = [&]() __attribute__((always_inline)) {
    if (wave_any(m_prev > m_ref)) {
      const float alpha = fast_exp2(__builtin_fmaxf((m_ref - m_prev) * c, -1.0e30f));
      l_run *= alpha;
      o0 *= alpha;
      o1 *= alpha;
      o2 *= alpha;
      o3 *= alpha;
    }
    m_ref = m_prev;
  };

  loads_barrier();
  scores(0, sa0, sa1);

  // Iteration t < ntiles - 1 with compile-time stage parity P = t & 1: softmax of tile t
  // (scores cur), scores of tile t+1 (K stage P ^ 1) into nxt, PV of tile t-1 (V stage
  // P ^ 1) when t > 0. Top: the previous iteration's loads (K(t+1), V(t-1)) have landed;
  // then K(t+2) and V(t) go into the stages freed by iteration t-1.
  auto iteration = [&](int t, v16f& cur0, v16f& cur1, v16f& nxt0, v16f& nxt1, auto parity,
                       auto do_pv) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    constexpr bool PV = decltype(do_pv)::value;
    constexpr int sk = P ^ 1, sv = P ^ 1;
    loads_barrier();
    load_k(t + 2, P);
    load_v(t, P);
    if (PV) {
      catch_up();
      l_run += ps_prev;
    }
    uint4 p[4];
    float psum = 0.0f;
    uint4 va[4], vb[4];
    // group 0: PV k-step 0 + max over cur0
    if (PV) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) va[cb] = ldsv(sv, cb, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // raised issue priority while the iteration's MFMAs issue: of the two waves on a SIMD,
    // the one with matrix-core work pending gets the vector ALU for the chunks between them
    __builtin_amdgcn_s_setprio(1);
    if (PV) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) vb[cb] = ldsv(sv, cb, 1);
      o0 = mfma_bf16_32x32x16(as_v8bf(va[0]), as_v8bf(p_prev[0]), o0);
      o1 = mfma_bf16_32x32x16(as_v8bf(va[1]), as_v8bf(p_prev[0]), o1);
      o2 = mfma_bf16_32x32x16(as_v8bf(va[2]), as_v8bf(p_prev[0]), o2);
      o3 = mfma_bf16_32x32x16(as_v8bf(va[3]), as_v8bf(p_prev[0]), o3);
    }
    float mx = __builtin_fmaxf(cur0[0], cur0[1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = __builtin_fmaxf(mx, cur0[i]);
    __builtin_amdgcn_sched_barrier(0);
    // group 1: PV k-step 1 + max over cur1, exchange
    if (PV) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) va[cb] = ldsv(sv, cb, 2);
      o0 = mfma_bf16_32x32x16(as_v8bf(vb[0]), as_v8bf(p_prev[1]), o0);
      o1 = mfma_bf16_32x32x16(as_v8bf(vb[1]), as_v8bf(p_prev[1]), o1);
      o2 = mfma_bf16_32x32x16(as_v8bf(vb[2]), as_v8bf(p_prev[1]), o2);
      o3 = mfma_bf16_32x32x16(as_v8bf(vb[3]), as_v8bf(p_prev[1]), o3);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, cur1[i]);
    const float m_cur = __builtin_fmaxf(m_prev, half_swap_max(mx));
    const float mc = m_cur * c;
    __builtin_amdgcn_sched_barrier(0);
    // group 2: PV k-step 2 + weights of keys g*32 + 0..7 (P k-step 0, low half)
    if (PV) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) vb[cb] = ldsv(sv, cb, 3);
      o0 = mfma_bf16_32x32x16(as_v8bf(va[0]), as_v8bf(p_prev[2]), o0);
      o1 = mfma_bf16_32x32x16(as_v8bf(va[1]), as_v8bf(p_prev[2]), o1);
      o2 = mfma_bf16_32x32x16(as_v8bf(va[2]), as_v8bf(p_prev[2]), o2);
      o3 = mfma_bf16_32x32x16(as_v8bf(va[3]), as_v8bf(p_prev[2]), o3);
    }
    {
      const uint2 a = quant4(cur0, 0, c, mc, psum), b = quant4(cur0, 4, c, mc, psum);
      p[0] = make_uint4(a.x, a.y, b.x, b.y);
    }
    __builtin_amdgcn_sched_barrier(0);
    // group 3: PV k-step 3 + P k-step 1
    uint4 ka0, kb0, ka1, kb1;
    ka0 = ldsk(sk, 0, 0);
    kb0 = ldsk(sk, 1, 0);
    if (PV) {
      o0 = mfma_bf16_32x32x16(as_v8bf(vb[0]), as_v8bf(p_prev[3]), o0);
      o1 = mfma_bf16_32x32x16(as_v8bf(vb[1]), as_v8bf(p_prev[3]), o1);
      o2 = mfma_bf16_32x32x16(as_v8bf(vb[2]), as_v8bf(p_prev[3]), o2);
      o3 = mfma_bf16_32x32x16(as_v8bf(vb[3]), as_v8bf(p_prev[3]), o3);
    }
    {
      const uint2 a = quant4(cur0, 8, c, mc, psum), b = quant4(cur0, 12, c, mc, psum);
      p[1] = make_uint4(a.x, a.y, b.x, b.y);
    }
    __builtin_amdgcn_sched_barrier(0);
    // groups 4..7: scores of tile t+1, 2 k-steps (4 MFMAs) each, + P k-steps 2, 3 and
    // the row-sum exchange
    nxt0 = zero16;
    nxt1 = zero16;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int s = 2 * grp;
      ka1 = ldsk(sk, 0, s + 1);
      kb1 = ldsk(sk, 1, s + 1);
      nxt0 = mfma_bf16_32x32x16(as_v8bf(ka0), as_v8bf(qb[s]), nxt0);
      nxt1 = mfma_bf16_32x32x16(as_v8bf(kb0), as_v8bf(qb[s]), nxt1);
      if (grp < 3) {
        ka0 = ldsk(sk, 0, s + 2);
        kb0 = ldsk(sk, 1, s + 2);
      }
      nxt0 = mfma_bf16_32x32x16(as_v8bf(ka1), as_v8bf(qb[s + 1]), nxt0);
      nxt1 = mfma_bf16_32x32x16(as_v8bf(kb1), as_v8bf(qb[s + 1]), nxt1);
      if (grp == 0) {
        const uint2 a = quant4(cur1, 0, c, mc, psum), b = quant4(cur1, 4, c, mc, psum);
        p[2] = make_uint4(a.x, a.y, b.x, b.y);
      } else if (grp == 1) {
        const uint2 a = quant4(cur1, 8, c, mc, psum), b = quant4(cur1, 12, c, mc, psum);
        p[3] = make_uint4(a.x, a.y, b.x, b.y);
      } else if (grp == 2) {
        psum = half_swap_sum(psum);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    pin(p);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) p_prev[ks] = p[ks];
    ps_prev = psum;
    m_prev = m_cur;
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  // ---- main loop over t = 0 .. ntiles-2 (scores alternate a <-> b; stage parity t & 1)
  int t = 0;
  if (ntiles > 1) {
    iteration(0, sa0, sa1, sb0, sb1, P0{}, F_{});
    t = 1;
    for (; t + 2 < ntiles; t += 2) {
      iteration(t, sb0, sb1, sa0, sa1, P1{}, T_{});
      iteration(t + 1, sa0, sa1, sb0, sb1, P0{}, T_{});
    }
    if (t + 1 < ntiles) {
      iteration(t, sb0, sb1, sa0, sa1, P1{}, T_{});
      ++t;
    } else {
      sa0 = sb0;   // the last tile's scores are in set b
      sa1 = sb1;
    }
  }
  // ---- epilogue (t = ntiles - 1, scores in set a): V(t-1) is in stage (t-1) & 1 (loaded
  // by the last iteration); V(t) still has to come, into stage t & 1, free once every wave
  // has passed the barrier below
  loads_barrier();
  load_v(ntiles - 1, (ntiles - 1) & 1);
  if (ntiles > 1) {
    catch_up();
    l_run += ps_prev;
    if ((ntiles - 2) & 1) pv(1, p_prev);
    else pv(0, p_prev);
  }
  {
    const bool ragged = last_lim != kBN;
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float a = (ragged && g * 32 + i >= last_lim) ? -__builtin_inff() : sa0[i];
      const float b = (ragged && g * 32 + 16 + i >= last_lim) ? -__builtin_inff() : sa1[i];
      mx = __builtin_fmaxf(mx, __builtin_fmaxf(a, b));
    }
    const float m_cur = __builtin_fmaxf(m_prev, half_swap_max(mx));
    const float mc = m_cur * c;
    float psum = 0.0f;
    uint4 p[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const v16f& sc = ks < 2 ? sa0 : sa1;
      const int i0 = (ks & 1) * 8, key0 = g * 32 + (ks >> 1) * 16 + i0;
      const uint2 a = quant4_masked(sc, i0, key0, last_lim, c, mc, psum);
      const uint2 b = quant4_masked(sc, i0 + 4, key0 + 4, last_lim, c, mc, psum);
      p[ks] = make_uint4(a.x, a.y, b.x, b.y);
    }
    psum = half_swap_sum(psum);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) p_prev[ks] = p[ks];
    ps_prev = psum;
    m_prev = m_cur;
  }
  loads_barrier();
  catch_up();
  l_run += ps_prev;
  if ((ntiles - 1) & 1) pv(1, p_prev);
  else pv(0, p_prev);

  // ---- O / l, bf16, one query row per lane
  if (q_local < S) {
    const float f = 1.0f / l_run;
    uint16_t* op = out + (int64_t)(seq_begin + q_local) * H * kHeadDim + head * kHeadDim;
    auto put = [&](const v16f& o, int cb) __attribute__((always_inline)) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        uint2 w;
        w.x = pack_bf16(o[i4 * 4 + 0] * f, o[i4 * 4 + 1] * f);
        w.y = pack_bf16(o[i4 * 4 + 2] * f, o[i4 * 4 + 3] * f);
        *reinterpret_cast<uint2*>(op + cb * 32 + i4 * 8 + g * 4) = w;
      }
    };
    put(o0, 0);
    put(o1, 1);
    put(o2, 2);
    put(o3, 3);
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnLaunch& a, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, hipStream_t s) {
  if (a.max_seqlen <= 0) return hipSuccess;
  static_assert(kBM == 128, "virtual tiles are 128 queries");
  const int64_t vtiles = (a.T + 127) / 128 + a.num_seqs;   // per head, see vtile_start
  const int64_t units = vtiles * a.H;
  const int64_t per_xcd = (units + 7) / 8;
  if (per_xcd * 8 > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_bf16_kernel, dim3((unsigned)(per_xcd * 8)), dim3(kThreads), 0, s, q,
                     k, v, a.cu, a.num_seqs, a.H, (int)vtiles, (int)per_xcd, a.softmax_scale,
                     a.out);
  return hipGetLastError();
}

}  // namespace fp8attn
