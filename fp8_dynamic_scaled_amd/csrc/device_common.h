// Device-side helpers shared by the gfx950 kernels of libfp8attn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8attn.h"

namespace fp8attn {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr float kE4M3Max = 448.0f;
// log2(448): folds the fixed P scale into the exponent of exp2.
constexpr float kLog2E4M3Max = 8.807354922057604f;
constexpr float kLog2e = 1.4426950408889634f;

// bf16 halves of a packed dword as fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> two E4M3 bytes (a in the lower byte) in the low half (HI = false) or the
// high half of `old`. gfx950's converter rounds to nearest even and is OCP E4M3FN; it
// only saturates up to 464, so callers that can exceed 448 clamp first.
template <bool HI>
__device__ __forceinline__ int cvt_pk_e4m3(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// Per-tensor scale pair from the window (or static) amax A: scale = A/448, inv = 448/A,
// both by IEEE division, with A floored at 2^-64 so that an all-zero tensor still gets a
// finite inverse. Every kernel that turns an A into a scale uses these.
constexpr float kAmaxFloor = 0x1p-64f;
__device__ __forceinline__ float scale_from_amax(float A) {
  return __builtin_fmaxf(A, kAmaxFloor) / kE4M3Max;
}
__device__ __forceinline__ float inv_scale_from_amax(float A) {
  return kE4M3Max / __builtin_fmaxf(A, kAmaxFloor);
}

// Largest ring entry of tensor t other than slot `skip`: the window maximum that the
// observation going into slot `skip` can only raise. Every slot is loaded and the skipped
// one counts as 0 (entries are >= 0): a conditional load per slot would become a chain of
// dependent scalar loads.
__device__ __forceinline__ float ring_max_except(const fp8attn_state* st, int t, uint32_t skip) {
  float r[FP8ATTN_RING_SLOTS];
#pragma unroll
  for (int s = 0; s < FP8ATTN_RING_SLOTS; ++s) r[s] = st->ring[t][s];
  float a = 0.0f;
#pragma unroll
  for (int s = 0; s < FP8ATTN_RING_SLOTS; ++s) a = __builtin_fmaxf(a, (uint32_t)s == skip ? 0.0f : r[s]);
  return a;
}

// One tensor's dynamic scale update: observation obs replaces ring slot `slot`, whose
// other slots' maximum is rest. Writes the window maximum A = max(rest, obs) with its scale
// pair and returns whether A moved (A != rest).
__device__ __forceinline__ bool dynamic_update(fp8attn_state* st, int t, uint32_t slot,
                                               float rest, float obs) {
  st->ring[t][slot] = obs;
  const float A = __builtin_fmaxf(rest, obs);
  st->amax[t] = A;
  st->scale[t] = scale_from_amax(A);
  st->inv_scale[t] = inv_scale_from_amax(A);
  return A != rest;
}

// The pending observation of tensor t: the maximum over its stripes (fp32 bit images),
// which are cleared.
__device__ __forceinline__ float take_observation(fp8attn_state* st, int t) {
  uint32_t m = 0;
#pragma unroll
  for (int s = 0; s < FP8ATTN_CUR_STRIPES; ++s) {
    const uint32_t v = st->cur[s][t];
    m = v > m ? v : m;
  }
#pragma unroll
  for (int s = 0; s < FP8ATTN_CUR_STRIPES; ++s) st->cur[s][t] = 0u;
  return __uint_as_float(m);
}

// Folds a block's maximum (fp32 bit image of a non-negative value, which orders like the
// value) into *word with one device atomic, skipped when the word already holds at least
// as much. Atomics on one 64-byte line serialise (about 13 ns each), hence the stripes of
// the state's cur and this filter; its read bypasses the XCD's L2 (system scope): an L2
// copy of a word that other XCDs' atomics keep raising can stay stale for the whole launch.
__device__ __forceinline__ void fold_max(uint32_t* word, uint32_t img) {
  if (img != 0 && img > __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM))
    atomicMax(word, img);
}

// The same fold with no filter read: an atomic whose result is unused is posted, so the
// wave does not wait for it, whereas the filter's L2-bypassing read makes it wait a
// memory round trip. Where blocks are short and their tails count (the quantise pass that
// observes the amax while it quantises), this is the cheaper form: 31 instead of 36 us for
// the one-pass dynamic quantisation of 8192 tokens x 16 heads. The amax kernel keeps the
// filter (1 % faster there).
__device__ __forceinline__ void post_max(uint32_t* word, uint32_t img) {
  if (img != 0) atomicMax(word, img);
}

__device__ __forceinline__ float clamp_e4m3(float y) {
  return __builtin_fminf(__builtin_fmaxf(y, -kE4M3Max), kE4M3Max);
}

// D = A * B + C on FP8 E4M3 operands (32x32x64, fp32 accumulate). Both operands hold,
// per lane, 32 bytes of the k dimension: lane l owns row/column l % 32 and k-half l / 32.
__device__ __forceinline__ v16f mfma_e4m3_32x32x64(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D = A * B + C on bf16 operands (32x32x16, fp32 accumulate); 8 k-values per lane.
__device__ __forceinline__ v16f mfma_bf16_32x32x16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

// Work units of the attention kernels: the 128-query tiles of every (sequence, head). For
// each head they are enumerated over "virtual tiles", the 128-column tiles of the padded
// key range of V8t: sequence i owns virtual tiles [vtile_start(i), vtile_start(i+1)) with
// vtile_start(i) = ceil(cu_i / 128) + i, its q-tiles are the first ceil(S_i / 128) of them
// and the rest (at most two per sequence) are empty. A head has ceil(T / 128) + num_seqs
// virtual tiles, so a batch of very unequal sequences launches about one block per real
// q-tile, not num_seqs times the longest sequence's count.
__device__ __forceinline__ int vtile_start(const int32_t* cu, int i) {
  return ((cu[i] + 127) >> 7) + i;
}
// The sequence owning virtual tile vt: the largest i with vtile_start(i) <= vt (starts
// strictly increase; vtile_start(0) = 0). A binary search on block-uniform loads.
__device__ __forceinline__ int vtile_seq(const int32_t* cu, int num_seqs, int vt) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (vtile_start(cu, mid) <= vt)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Start column of sequence i in the key-contiguous V8t layout (see fp8attn.h).
__device__ __host__ __forceinline__ int64_t pad_start(int64_t cu_i, int i) {
  return ((cu_i + 127) / 128) * 128 + 128 * (int64_t)i;
}

}  // namespace fp8attn
