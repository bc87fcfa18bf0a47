// FP8 varlen non-causal flash-attention forward for gfx950 (CDNA4).
//
// What it computes (vLLM-Omni "Quantized KV Cache", "Overview"; vLLM docs "FP8 ViT
// Encoder Attention", first paragraph and "Performance"; Korean wiki "FP8 ViT 인코더
// 어텐션", "Requirements": varlen FP8 attention with per-tensor scales): for each packed
// sequence i, head h and query row r, over the keys j of sequence i only,
//   s_j  = (q8 . k8_j) * scale_q * scale_k * softmax_scale,
//   M    = ceil(m * log2 e), m = max_j s_j over ALL keys of the sequence,
//   p8_j = E4M3(448 * 2^(s_j log2 e - M))     (the largest weight in [224, 448]),
//   O    = scale_v * sum_j p8_j v8_j / sum_j p8_j, stored as bf16.
// One pass over the keys: each tile's weights are taken against the running reference
// exponent R_t (the row maximum so far, in log2 units, rounded up), and their PV and
// row-sum products enter the accumulators multiplied by 2^(R_t - R_0) -- the MFMA's E8M0
// scale on the P operand -- so the accumulators keep the first tile's reference R_0 and
// are never rescaled (unless the shift would pass 2^64). Multiplying by a power of two
// commutes with the E4M3 rounding while the weights stay at or above 2^-6, and is exact in
// the fp32 products and sums, so O = sum / row sum is the result of the final reference,
// independent of the tiling; only weights that end below 2^-6 (keys more than ~10 nats
// under the row maximum, seen before it) keep the finer rounding of their provisional
// reference: each differs from its E4M3 code by at most 2^-9 on the weights' scale (where
// the largest weight is 224 to 448).
//
// Mapping onto the matrix cores (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulate):
//   * a block owns 128 queries of one (sequence, head); each of its 4 waves owns 32;
//   * scores are produced transposed, S^T = K Q^T, so that in the accumulator layout a
//     lane holds ONE query (column l % 32) and 16 keys per 32x32 block; the row maximum
//     is a per-lane reduction plus one v_permlane32_swap with the other lane half;
//   * the K rows of a tile are stored in LDS in a permuted order so that lane half g
//     ends up holding the 32 consecutive keys g*32 .. g*32+31 of the 64-key tile; the
//     packed E4M3 probabilities are then directly the B operand of O^T = V^T P^T, and the
//     A operand is 32 consecutive key bytes of one channel row of V8t (keys contiguous,
//     as written by the quantise kernel) -- no LDS round trip for P;
//   * the B operand P^T holds one query per lane, so the per-query shift 2^(R_t - R_0) is
//     the per-lane B scale of v_mfma_scale_f32_32x32x64_f8f6f4 (E8M0 in byte 0 of a VGPR;
//     the B scale of lane l applies to its column l % 32 and key half l / 32);
//   * the row sum of the quantised weights accumulates on the matrix core (one extra MFMA
//     with an all-ones A operand per tile, scaled like the PV products).
//
// Schedule. At d = 128 the vector ALU, not the matrix core, bounds this kernel: per score
// it needs one FMA, one v_exp_f32 (about 2.3 FMA slots), half a v_cvt_pk_fp8_f32 (about
// 1.7 slots) and part of a v_max3, and every MFMA issue blocks the ALU for a few cycles;
// the matrix core needs 1/4 of a 32x32x64 MFMA slot per 64 scores. Keeping both busy
// takes a software pipeline inside each wave plus two waves per SIMD:
//   * iteration t runs the softmax of tile t on the vector ALU while the matrix core runs
//     PV of tile t-1 and the scores of tile t+1; the MFMAs are spread through the VALU
//     stream (sched_barrier), and the new P is pinned before the loop back edge so the
//     compiler cannot sink its exp/convert chain past the next tile's rescale branch;
//   * the loop is unrolled by four (two pairs of tiles): the two score register sets swap
//     roles without copies, and every LDS ring stage the operand reads use is a constant
//     (an immediate offset, no address arithmetic per tile); a ragged last tile is handled
//     (masked) only in the epilogue;
//   * the wave's issue priority is raised from its first MFMA of an iteration to its
//     last, so that of the two waves on a SIMD the one with MFMAs still to issue gets the
//     vector ALU first (3-5 % faster than equal priority);
//   * the row maximum is a tree of v_max3 (depth 4 over a lane's 32 scores) written as
//     the instruction itself (fmaxf would make the compiler quiet every score first;
//     scores are never NaN);
//   * K and V8t tiles go global -> LDS with buffer loads that write LDS directly (no VGPR
//     staging, no ds_write), in four-stage rings; tiles move in pairs, with one vmcnt wait
//     and one barrier per pair of tiles, each pair's loads issued one pair ahead of use;
//     16-byte LDS chunks are XOR-swizzled so operand reads are conflict-free;
//   * 448 * 2^(s log2 e - M) is computed as exp2(s * c - (M - log2 448)), c = scales *
//     log2(e): one FMA and one v_exp_f32 per score;
//   * block -> work mapping is XCD-aware: consecutive work units (the q-tiles of one head,
//     sequence after sequence) go to the same XCD so its L2 keeps that head's K/V; units
//     are enumerated over virtual tiles (vtile_start), so a batch of very unequal
//     sequences launches about one block per real q-tile.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace fp8attn {

namespace {

constexpr int kBM = 128;                 // queries per block
constexpr int kBN = 64;                  // keys per tile
constexpr int kThreads = 256;
constexpr int kKTileBytes = kBN * kHeadDim;   // K tile: 64 rows x 128 B
constexpr int kVTileBytes = kHeadDim * kBN;   // V8t tile: 128 rows x 64 B
constexpr int kStages = 4;                    // ring depth of each of K and V8t
constexpr uint32_t kOnesE4M3 = 0x38383838u;   // four E4M3 1.0
constexpr int kBufferFlags = 0x00020000;      // raw buffer resource, dword 3 (gfx9)
// largest exponent shift applied through the MFMA B scale before the accumulators are
// rescaled: 2^64 x (448 x 448 x 2^20 keys) stays far below the fp32 range
constexpr float kMaxShift = 64.0f;

// LDS row of key kappa (0..63) in the K tile: the MFMA A row m of key block kb that
// yields, in the accumulator layout, key g*32 + kb*16 + i in register i of lane half g.
__device__ __forceinline__ int k_lds_row(int kappa) {
  const int g = kappa >> 5, kb = (kappa >> 4) & 1, i = kappa & 15;
  return kb * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
}
// 16-byte chunk swizzles. K rows are 128 B (8 chunks), V8t rows 64 B (4 chunks). An MFMA
// operand read has 8 (or 16) consecutive lanes on 8 (16) consecutive rows at the same
// logical chunk; these XOR patterns spread them over distinct bank groups whether the LDS
// serves 8 lanes over 128 B or 16 lanes over 256 B per pass.
__device__ __forceinline__ int k_swz(int R) { return ((R >> 1) ^ (R << 2)) & 7; }
__device__ __forceinline__ int v_swz(int R) { return ((R >> 1) ^ (R >> 2)) & 3; }

__device__ __forceinline__ v8i load32(const uint8_t* p0, const uint8_t* p1) {
  const v4i a = *reinterpret_cast<const v4i*>(p0);
  const v4i b = *reinterpret_cast<const v4i*>(p1);
  v8i r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Per-lane constants of one wave (query n = lane % 32, k-half g = lane / 32).
struct Lane {
  int n, g;
  int ks00, ks01, ks10, ks11;   // K operand chunk offsets (step s, half h) within a row
  int vs0, vs1;                 // V8t operand chunk offsets (half h) within a row
};

// S^T = K Q^T for the 64 keys of one LDS K stage: two 32x32 blocks of fp32 scores.
__device__ __forceinline__ void scores(const uint8_t* __restrict__ kt, const Lane& ln,
                                       const v8i& qb0, const v8i& qb1, v16f& s0, v16f& s1) {
  const v16f zero16 = {};
  const uint8_t* r0 = kt + ln.n * kHeadDim;            // K block 0 row of this lane
  const uint8_t* r1 = r0 + 32 * kHeadDim;              // K block 1 row
  s0 = mfma_e4m3_32x32x64(load32(r0 + ln.ks00, r0 + ln.ks01), qb0, zero16);
  s1 = mfma_e4m3_32x32x64(load32(r1 + ln.ks00, r1 + ln.ks01), qb0, zero16);
  s0 = mfma_e4m3_32x32x64(load32(r0 + ln.ks10, r0 + ln.ks11), qb1, s0);
  s1 = mfma_e4m3_32x32x64(load32(r1 + ln.ks10, r1 + ln.ks11), qb1, s1);
}

// O^T += V^T P^T over 4 blocks of 32 channels; the row sum of P accumulates in rs.
// D = A B 2^(sb - 127) + C: the B operand (P^T, one query per lane) scaled by the E8M0
// exponent in byte 0 of sb; the A scale sa holds 127 (x1) in a register.
__device__ __forceinline__ v16f mfma_pv(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ void pv(const uint8_t* __restrict__ vt, const Lane& ln, const v8i& p,
                                   const v8i& ones, int sa, int sb, v16f& rs, v16f& o0,
                                   v16f& o1, v16f& o2, v16f& o3) {
  const uint8_t* vr = vt + ln.n * kBN;
  rs = mfma_pv(ones, p, rs, sa, sb);
  o0 = mfma_pv(load32(vr + ln.vs0, vr + ln.vs1), p, o0, sa, sb);
  o1 = mfma_pv(load32(vr + 32 * kBN + ln.vs0, vr + 32 * kBN + ln.vs1), p, o1, sa, sb);
  o2 = mfma_pv(load32(vr + 64 * kBN + ln.vs0, vr + 64 * kBN + ln.vs1), p, o2, sa, sb);
  o3 = mfma_pv(load32(vr + 96 * kBN + ln.vs0, vr + 96 * kBN + ln.vs1), p, o3, sa, sb);
}

// Maxima of scores written as the instructions themselves: the scores are never NaN, and
// fmaxf would make the compiler quiet every input first (one v_max_f32 x, x, x each).
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Maximum over the two lane halves (lanes l and l ^ 32 hold the two key halves of one
// query): one v_permlane32_swap exchanges the halves.
__device__ __forceinline__ float half_swap_max(float mx) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                   false, false);
  return vmax(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// Scores i0 .. i0+3 of one 16-score block -> 4 packed E4M3 weights exp2(s*c - mc). The
// low-half convert keeps the high half of its "old" operand, which the high-half convert
// then overwrites; passing the first exp's own bits there lets the result take that
// register in place (no zeroing move).
__device__ __forceinline__ int quant4(const v16f& s, int i0, float c, float mc) {
  const float e0 = fast_exp2(__builtin_fmaf(s[i0], c, -mc));
  const int w = cvt_pk_e4m3<false>(e0, fast_exp2(__builtin_fmaf(s[i0 + 1], c, -mc)),
                                   __float_as_int(e0));
  return cvt_pk_e4m3<true>(fast_exp2(__builtin_fmaf(s[i0 + 2], c, -mc)),
                           fast_exp2(__builtin_fmaf(s[i0 + 3], c, -mc)), w);
}

// Row maximum of this lane's query over one tile of scores (both lane halves). Masked
// keys (g*32 + i, g*32 + 16 + i at or past key_lim) are left out.
template <bool MASK>
__device__ __forceinline__ float tile_max(const v16f& s0, const v16f& s1, int g, int key_lim) {
  auto val = [&](const v16f& s, int i, int key) __attribute__((always_inline)) {
    return (MASK && key >= key_lim) ? -__builtin_inff() : s[i];
  };
  // one running chain (the compiler folds it into v_max3 without re-quieting every input)
  float mx = __builtin_fmaxf(val(s0, 0, g * 32), val(s0, 1, g * 32 + 1));
#pragma unroll
  for (int i = 2; i < 16; ++i) mx = __builtin_fmaxf(mx, val(s0, i, g * 32 + i));
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, val(s1, i, g * 32 + 16 + i));
  return half_swap_max(mx);
}

// p = 448 * 2^(s*c - M) = exp2(s*c - mc), mc = M - log2 448; packed E4M3 with byte j of
// the 32 = key g*32 + j of the tile. Masked keys get exp2(-inf) = 0 (the exponent
// argument, not the score, is replaced, so a zero c cannot make -inf * 0).
template <bool MASK>
__device__ __forceinline__ v8i quantise_p(const v16f& s0, const v16f& s1, float c, float mc,
                                          int g, int key_lim) {
  auto arg = [&](float s, int key) __attribute__((always_inline)) {
    const float x = __builtin_fmaf(s, c, -mc);
    return (MASK && key >= key_lim) ? -__builtin_inff() : x;
  };
  v8i p;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i0 = r * 4;
    const int k0 = g * 32 + i0, k1 = g * 32 + 16 + i0;
    // the low-half convert leaves the high half of its destination as it finds it; the
    // high-half convert then overwrites it, so the starting value does not matter
    const int any = __builtin_nondeterministic_value(0);
    const int w = cvt_pk_e4m3<false>(fast_exp2(arg(s0[i0], k0)), fast_exp2(arg(s0[i0 + 1], k0 + 1)),
                                     any);
    p[r] = cvt_pk_e4m3<true>(fast_exp2(arg(s0[i0 + 2], k0 + 2)),
                             fast_exp2(arg(s0[i0 + 3], k0 + 3)), w);
    const int w2 = cvt_pk_e4m3<false>(fast_exp2(arg(s1[i0], k1)),
                                      fast_exp2(arg(s1[i0 + 1], k1 + 1)), any);
    p[4 + r] = cvt_pk_e4m3<true>(fast_exp2(arg(s1[i0 + 2], k1 + 2)),
                                 fast_exp2(arg(s1[i0 + 3], k1 + 3)), w2);
  }
  return p;
}

// Wait for this thread's older LDS-bound tile loads (all but the newest N vector-memory
// operations), then a workgroup barrier that publishes them. The barrier is an asm
// statement with a memory clobber, so no LDS access moves across it; __syncthreads()
// would add its release fence, i.e. a wait for ALL outstanding loads (no lookahead left).
template <int N>
__device__ __forceinline__ void loads_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Keeps p's computation above this point (an empty asm that reads it).
__device__ __forceinline__ void pin(const v8i& p) {
  asm volatile("" ::"v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]),
               "v"(p[6]), "v"(p[7]));
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fp8_kernel(const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8,
                     const uint8_t* __restrict__ v8t, const int32_t* __restrict__ cu,
                     int num_seqs, int H, int64_t Tp, int vtiles, int units_per_xcd,
                     const fp8attn_state* __restrict__ st, float sm_scale,
                     uint16_t* __restrict__ out) {
  // kStages K tiles, then kStages V8t tiles
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * (kKTileBytes + kVTileBytes)];

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
  Lane ln;
  ln.n = lane & 31;
  ln.g = lane >> 5;
  const int row_stride = H * kHeadDim;   // bytes per token row of Q8/K8

  // ---- tile loaders: buffer loads straight into LDS. A wave's load instruction fills
  // 1 KB of LDS with lane L at byte 16 L, so each lane fetches the global chunk that
  // belongs at its LDS position: K block b (8 rows of 128 B) row R = 8b + L/8, physical
  // chunk L % 8 = logical chunk ^ k_swz(R), key = the key stored at row R; V8t block b
  // (16 rows of 64 B) row R = 16b + L/4, chunk L % 4 = logical ^ v_swz(R). Each of the
  // 4 waves loads blocks 2w and 2w + 1 of each tile.
  const uint8_t* kbase = k8 + (int64_t)seq_begin * row_stride + head * kHeadDim;
  const uint8_t* vbase = v8t + (int64_t)head * kHeadDim * Tp + pad_start(seq_begin, seq);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  int kvo[2], vvo[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int b = 2 * wv + j;
    const int R = 8 * b + (lane >> 3);
    const int kb = R >> 5, m = R & 31;
    const int key = ((m >> 2) & 1) * 32 + kb * 16 + (m >> 3) * 4 + (m & 3);   // inverse of k_lds_row
    kvo[j] = key * row_stride + (((lane & 7) ^ k_swz(R)) << 4);
    const int RV = 16 * b + (lane >> 2);
    vvo[j] = RV * (int)Tp + (((lane & 3) ^ v_swz(RV)) << 4);
  }
  const int kvo0 = kvo[0], kvo1 = kvo[1], vvo0 = vvo[0], vvo1 = vvo[1];
  typedef __attribute__((address_space(3))) void lds_void;
  uint8_t* const kst = smem;                                // K stage i at kst + i * kKTileBytes
  uint8_t* const vst = smem + kStages * kKTileBytes;        // V stage i at vst + i * kVTileBytes
  const int ntiles = (S + kBN - 1) / kBN;
  // K tile j into stage j % 4 (clamped to the last tile, so the loads past the end stay in
  // bounds; they fill stages that are never read again); rows at or past the end of the
  // sequence read as 0
  auto load_k = [&](int j) __attribute__((always_inline)) {
    const int stage = j & (kStages - 1);
    const int k0 = (j < ntiles ? j : ntiles - 1) * kBN;
    // uniform by construction; readfirstlane keeps it in SGPRs (a vector value would make
    // the compiler wrap the load in a waterfall loop)
    const int rows = __builtin_amdgcn_readfirstlane(S - k0);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (int64_t)k0 * row_stride), (short)0, rows * row_stride, kBufferFlags);
    uint8_t* dst = kst + stage * kKTileBytes + wv * 2048;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)dst, 16, kvo0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(dst + 1024), 16, kvo1, 0, 0, 0);
  };
  // V8t tile j into stage j % 4 (clamped like K): columns up to the sequence's 128-aligned
  // padded length, which the quantise kernel zero-fills
  auto load_v = [&](int j) __attribute__((always_inline)) {
    const int stage = j & (kStages - 1);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (j < ntiles ? j : ntiles - 1) * kBN), (short)0, 0x7fffffff,
        kBufferFlags);
    uint8_t* dst = vst + stage * kVTileBytes + wv * 2048;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)dst, 16, vvo0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dst + 1024), 16, vvo1, 0, 0, 0);
  };

  // ---- prologue loads: everything iteration 0 and the first pair (tiles 1, 2) read:
  // K(0) .. K(3), V(0), V(1). Tile j always lives in stage j % 4 of its ring.
  load_k(0);
  load_k(1);
  load_k(2);
  load_k(3);
  load_v(0);
  load_v(1);

  // ---- Q^T operand (B of S^T = K Q^T): lane = query n, 32 channel bytes of half g
  const int q_local = qt * kBM + wave * 32 + ln.n;
  const int q_row = seq_begin + (q_local < S ? q_local : S - 1);
  const uint8_t* qp = q8 + (int64_t)q_row * row_stride + head * kHeadDim;
  const v8i qb0 = load32(qp + ln.g * 32, qp + ln.g * 32 + 16);       // channels 0..63
  const v8i qb1 = load32(qp + 64 + ln.g * 32, qp + 64 + ln.g * 32 + 16);

  const float scale_q = st->scale[0], scale_k = st->scale[1], scale_v = st->scale[2];
  const float c = scale_q * scale_k * sm_scale * kLog2e;  // score -> log2 domain

  // ---- lane constants of the operand reads
  {
    const int sk = k_swz(ln.n), sv = v_swz(ln.n);   // the same for every 32-row block
    ln.ks00 = ((0 + ln.g * 2) ^ sk) << 4;
    ln.ks01 = ((1 + ln.g * 2) ^ sk) << 4;
    ln.ks10 = ((4 + ln.g * 2) ^ sk) << 4;
    ln.ks11 = ((5 + ln.g * 2) ^ sk) << 4;
    ln.vs0 = ((ln.g * 2) ^ sv) << 4;
    ln.vs1 = ((ln.g * 2 + 1) ^ sv) << 4;
  }

  // ---- per-lane state for query n
  // ref_prev: reference exponent (the running row maximum in log2 units, rounded up to an
  // integer) after the last tile whose softmax ran; ref_acc: the exponent that the O and
  // row-sum accumulators are relative to (set at the first PV product, moved only when the
  // shift to ref_prev would pass kMaxShift). Both hold integers (as floats) or -inf before
  // the first tile.
  float ref_prev = -__builtin_inff();
  float ref_acc = -__builtin_inff();
  v16f o0 = {}, o1 = {}, o2 = {}, o3 = {};
  v16f rs = {};                                         // row sum of P (entry 0 is used)
  v8i ones;
#pragma unroll
  for (int r = 0; r < 8; ++r) ones[r] = (int)kOnesE4M3;
  asm volatile("" : "+v"(ones));   // opaque: kept in registers, not rebuilt every tile
  int s127 = 127;                  // E8M0 1.0 for the A operand, from a register
  asm volatile("" : "+v"(s127));
  const int last_lim = S - (ntiles - 1) * kBN;          // valid keys of the last tile
  v16f sa0, sa1, sb0, sb1;                              // two score register sets
  v8i p_prev;                                           // quantised P of the previous tile

  // ---- scores of tile 0. The Q loads are younger than the prologue's tile loads and are
  // counted by vmcnt too: wait for everything once here.
  loads_barrier<0>();
  scores(kst, ln, qb0, qb1, sa0, sa1);

  // The accumulators stay relative to ref_acc; the pending P is relative to ref_prev, so
  // its PV and row-sum products are scaled by 2^(ref_prev - ref_acc) through the B scale of
  // the MFMA (returned as the E8M0 byte). Only when that shift would pass kMaxShift (and on
  // the first tile, ref_acc = -inf) are the accumulators rescaled to ref_prev.
  auto catch_up = [&]() __attribute__((always_inline)) -> int {
    if (wave_any(ref_prev - ref_acc > kMaxShift)) {
      // an exact power of two, 2^(ref_acc - ref_prev); 0 while ref_acc = -inf (the clamp
      // keeps the conversion to int defined)
      const float alpha = __builtin_ldexpf(1.0f, (int)__builtin_fmaxf(ref_acc - ref_prev, -200.0f));
      rs[0] *= alpha;
      o0 *= alpha;
      o1 *= alpha;
      o2 *= alpha;
      o3 *= alpha;
      ref_acc = ref_prev;
    }
    return 127 + (int)(ref_prev - ref_acc);
  };

  // Synchronisation of a pair of iterations t, t+1 (t odd). They read K(t+1), K(t+2),
  // V(t-1), V(t), all loaded by the previous pair (or the prologue): wait for this
  // thread's loads, then the barrier publishes everyone's. After it, the stages of K(t-1),
  // K(t) and V(t-3), V(t-2) -- read only by the previous pair -- take the next pair's
  // tiles K(t+3), K(t+4), V(t+1), V(t+2).
  auto pair_sync = [&](int t) __attribute__((always_inline)) {
    loads_barrier<0>();
    load_k(t + 3);
    load_k(t + 4);
    load_v(t + 1);
    load_v(t + 2);
  };


  // Iteration t < ntiles - 1: softmax of tile t (scores in cur), scores of tile t+1 into
  // nxt, PV of tile t-1 (when t > 0).
  auto iteration = [&](int t, v16f& cur0, v16f& cur1, v16f& nxt0, v16f& nxt1,
                       auto do_pv, int sk, int sv) __attribute__((always_inline)) {
    constexpr bool PV = decltype(do_pv)::value;
    // sk: stage of K(t+1), sv: stage of V(t-1) (constants where the caller knows t mod 4)
    int sb = 127;
    if (PV) sb = catch_up();
    // ---- one region, written in issue order: each MFMA is followed by one chunk of the
    // softmax (a part of the row maximum, or the exp/convert of 4 scores), and
    // sched_barrier(0) keeps every pair where it is, so the matrix core always has the
    // next MFMA queued while the vector ALU works through the chunk.
    const uint8_t* vr = vst + sv * kVTileBytes + ln.n * kBN;        // V(t-1) row of lane
    const uint8_t* kr0 = kst + sk * kKTileBytes + ln.n * kHeadDim;  // K(t+1) rows of lane
    const uint8_t* kr1 = kr0 + 32 * kHeadDim;
    const v16f zero16 = {};
    v8i va0, va1, va2, va3;
    if (PV) {
      va0 = load32(vr + ln.vs0, vr + ln.vs1);
      va1 = load32(vr + 32 * kBN + ln.vs0, vr + 32 * kBN + ln.vs1);
      va2 = load32(vr + 64 * kBN + ln.vs0, vr + 64 * kBN + ln.vs1);
      va3 = load32(vr + 96 * kBN + ln.vs0, vr + 96 * kBN + ln.vs1);
    }
    __builtin_amdgcn_sched_barrier(0);
    // raised issue priority from the first MFMA to the last: of the two waves on a SIMD,
    // the one with MFMAs left to issue gets the vector ALU for the chunks between them,
    // and the one in its MFMA-free tail (two chunks, the loop's bookkeeping) yields
    __builtin_amdgcn_s_setprio(1);
    if (PV) rs = mfma_pv(ones, p_prev, rs, s127, sb);
    const float mx0 = vmax(vmax3(vmax3(cur0[0], cur0[1], cur0[2]), vmax3(cur0[3], cur0[4], cur0[5]),
                                 vmax3(cur0[6], cur0[7], cur0[8])),
                           vmax3(vmax3(cur0[9], cur0[10], cur0[11]),
                                 vmax3(cur0[12], cur0[13], cur0[14]), cur0[15]));
    __builtin_amdgcn_sched_barrier(0);
    if (PV) o0 = mfma_pv(va0, p_prev, o0, s127, sb);
    const v8i ka0 = load32(kr0 + ln.ks00, kr0 + ln.ks01);
    const v8i kb0 = load32(kr1 + ln.ks00, kr1 + ln.ks01);
    const v8i ka1 = load32(kr0 + ln.ks10, kr0 + ln.ks11);
    const v8i kb1 = load32(kr1 + ln.ks10, kr1 + ln.ks11);
    const float mx1 = vmax(vmax3(vmax3(cur1[0], cur1[1], cur1[2]), vmax3(cur1[3], cur1[4], cur1[5]),
                                 vmax3(cur1[6], cur1[7], cur1[8])),
                           vmax3(vmax3(cur1[9], cur1[10], cur1[11]),
                                 vmax3(cur1[12], cur1[13], cur1[14]), cur1[15]));
    const float mx = vmax(mx0, mx1);
    // c > 0, so the maximum of the raw dot products gives the maximum score
    const float ref_cur = vmax(ref_prev, __builtin_ceilf(half_swap_max(mx) * c));
    const float mc = ref_cur - kLog2E4M3Max;
    __builtin_amdgcn_sched_barrier(0);
    v8i p;
    if (PV) o1 = mfma_pv(va1, p_prev, o1, s127, sb);
    p[0] = quant4(cur0, 0, c, mc);
    __builtin_amdgcn_sched_barrier(0);
    if (PV) o2 = mfma_pv(va2, p_prev, o2, s127, sb);
    p[1] = quant4(cur0, 4, c, mc);
    __builtin_amdgcn_sched_barrier(0);
    if (PV) o3 = mfma_pv(va3, p_prev, o3, s127, sb);
    p[2] = quant4(cur0, 8, c, mc);
    __builtin_amdgcn_sched_barrier(0);
    nxt0 = mfma_e4m3_32x32x64(ka0, qb0, zero16);
    p[3] = quant4(cur0, 12, c, mc);
    __builtin_amdgcn_sched_barrier(0);
    nxt1 = mfma_e4m3_32x32x64(kb0, qb0, zero16);
    p[4] = quant4(cur1, 0, c, mc);
    __builtin_amdgcn_sched_barrier(0);
    nxt0 = mfma_e4m3_32x32x64(ka1, qb1, nxt0);
    p[5] = quant4(cur1, 4, c, mc);
    __builtin_amdgcn_sched_barrier(0);
    nxt1 = mfma_e4m3_32x32x64(kb1, qb1, nxt1);
    __builtin_amdgcn_s_setprio(0);
    p[6] = quant4(cur1, 8, c, mc);
    __builtin_amdgcn_sched_barrier(0);
    p[7] = quant4(cur1, 12, c, mc);
    pin(p);
    p_prev = p;
    ref_prev = ref_cur;
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  // ---- main loop over t = 0 .. ntiles-2 in pairs (scores alternate a <-> b). Iteration
  // 0 reads only prologue tiles, which the barrier above published.
  int t = 0;
  if (ntiles > 1) {
    iteration(0, sa0, sa1, sb0, sb1, F_{}, 1, 3);
    t = 1;
    // two pairs per trip, t = 1 (mod 4): every ring stage is a constant
    for (; t + 4 < ntiles; t += 4) {
      pair_sync(t);
      iteration(t, sb0, sb1, sa0, sa1, T_{}, 2, 0);
      iteration(t + 1, sa0, sa1, sb0, sb1, T_{}, 3, 1);
      pair_sync(t + 2);
      iteration(t + 2, sb0, sb1, sa0, sa1, T_{}, 0, 2);
      iteration(t + 3, sa0, sa1, sb0, sb1, T_{}, 1, 3);
    }
    if (t + 2 < ntiles) {
      pair_sync(t);
      iteration(t, sb0, sb1, sa0, sa1, T_{}, 2, 0);
      iteration(t + 1, sa0, sa1, sb0, sb1, T_{}, 3, 1);
      t += 2;
    }
    if (t + 1 < ntiles) {
      // a last single iteration t = ntiles - 2: K(t+1), V(t-1) came with the previous
      // pair; V(t+1) = V(ntiles-1) is still to load (for the epilogue)
      loads_barrier<0>();
      load_v(t + 1);
      iteration(t, sb0, sb1, sa0, sa1, T_{}, (t + 1) & 3, (t - 1) & 3);
      ++t;
    } else {
      sa0 = sb0;   // the last tile's scores are in set b: move them (once)
      sa1 = sb1;
    }
  }
  // ---- epilogue: t = ntiles - 1, scores in set a; V(ntiles-2), V(ntiles-1) loaded
  loads_barrier<0>();
  if (ntiles > 1) {
    const int sb = catch_up();
    pv(vst + ((ntiles - 2) & (kStages - 1)) * kVTileBytes, ln, p_prev, ones, s127, sb, rs, o0, o1, o2,
       o3);   // PV(ntiles-2)
  }
  {
    const bool ragged = last_lim != kBN;
    const float ref_cur = __builtin_fmaxf(
        ref_prev, __builtin_ceilf(c * (ragged ? tile_max<true>(sa0, sa1, ln.g, last_lim)
                                              : tile_max<false>(sa0, sa1, ln.g, kBN))));
    const float mc = ref_cur - kLog2E4M3Max;
    p_prev = ragged ? quantise_p<true>(sa0, sa1, c, mc, ln.g, last_lim)
                    : quantise_p<false>(sa0, sa1, c, mc, ln.g, kBN);
    ref_prev = ref_cur;
  }
  const int sb_last = catch_up();
  pv(vst + ((ntiles - 1) & (kStages - 1)) * kVTileBytes, ln, p_prev, ones, s127, sb_last, rs, o0, o1, o2,
     o3);   // PV(ntiles-1)

  // ---- O = O * scale_v / l, bf16, one query row per lane
  if (q_local < S) {
    const float f = scale_v / rs[0];
    uint16_t* op = out + (int64_t)(seq_begin + q_local) * row_stride + head * kHeadDim;
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    auto put = [&](const v16f& o, int cb) __attribute__((always_inline)) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f2 x0 = {o[i4 * 4 + 0] * f, o[i4 * 4 + 1] * f};
        const f2 x1 = {o[i4 * 4 + 2] * f, o[i4 * 4 + 3] * f};
        const b2 y0 = __builtin_convertvector(x0, b2);
        const b2 y1 = __builtin_convertvector(x1, b2);
        uint2 w;
        w.x = *reinterpret_cast<const uint32_t*>(&y0);
        w.y = *reinterpret_cast<const uint32_t*>(&y1);
        *reinterpret_cast<uint2*>(op + cb * 32 + i4 * 8 + ln.g * 4) = w;
      }
    };
    put(o0, 0);
    put(o1, 1);
    put(o2, 2);
    put(o3, 3);
  }
}

}  // namespace

hipError_t launch_attn_fp8(const AttnLaunch& a, const fp8attn_state* st, const uint8_t* q8,
                           const uint8_t* k8, const uint8_t* v8t, hipStream_t s) {
  if (a.max_seqlen <= 0) return hipSuccess;
  const int64_t vtiles = (a.T + 127) / 128 + a.num_seqs;
  const int64_t units = vtiles * a.H;
  const int64_t per_xcd = (units + 7) / 8;
  if (per_xcd * 8 > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_fp8_kernel, dim3((unsigned)(per_xcd * 8)), dim3(kThreads), 0, s, q8,
                     k8, v8t, a.cu, a.num_seqs, a.H, a.Tp, (int)vtiles, (int)per_xcd, st,
                     a.softmax_scale, a.out);
  return hipGetLastError();
}

}  // namespace fp8attn
