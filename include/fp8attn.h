/*
 * fp8attn.h — C-ABI of the online per-tensor FP8 attention library (libfp8attn.so).
 *
 * What the library computes, per attention call:
 *   1. the absolute maximum of each of Q, K and V (one value per tensor),
 *   2. a per-tensor E4M3 scale, from a 16-slot ring of observed maxima or from a
 *      calibrated static maximum times a margin,
 *   3. Q, K, V quantised to E4M3 with that scale, then a non-causal, variable-length
 *      (cu_seqlens, no padding) flash-attention forward on FP8 matrix cores, or — when the
 *      caller asks to skip FP8 for this call — the same attention in BF16.
 *
 * Sources for the behaviour (web pages):
 *   - vLLM-Omni user guide "Quantized KV Cache", sections "Overview" (Q/K/V quantised on
 *     the fly right before the attention operator, weights untouched; native dtype when
 *     FP8 is not requested) and "Parameters" (step/layer selectors that keep listed
 *     forwards in the native dtype).
 *   - vLLM docs "FP8 ViT Encoder Attention", sections "Usage" (dynamic scaling driven by a
 *     circular buffer of the last 16 observed Q/K/V amax values; static scales calibrated
 *     once; saved scales multiplied by a margin that defaults to 1.5) and "Scale file format"
 *     (one q/k/v triple per attention layer).
 *   - the Korean wiki rewrite of that page, "FP8 ViT 인코더 어텐션", section "Requirements"
 *     (the AMD backend is a varlen, per-tensor-scale FP8 flash attention).
 * The E4M3 format is the OCP 8-bit floating point E4M3 ("FN") encoding: bias 7, no
 * infinities, 0x7F/0xFF are NaN, largest finite magnitude 448.
 *
 * Conventions common to every call:
 *   - Pointers are DEVICE pointers unless the name ends in _host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every call
 *     only enqueues work on that stream and never waits for the device.
 *   - The caller owns every buffer (state, workspace, inputs, outputs). The library
 *     allocates no device memory and keeps no global state apart from the thread-local
 *     error message and the fixed scratch array of fp8attn_forward_noalloc.
 *   - Argument checks happen on the host before anything is enqueued. A failed check
 *     returns a negative status, enqueues nothing, and sets fp8attn_last_error().
 *     A failed kernel launch returns FP8ATTN_EHIP.
 *   - Tensors Q, K, V, O are packed "THD": [total_tokens][num_heads][head_dim], row major,
 *     bf16, contiguous, sequences concatenated along tokens as described by cu_seqlens.
 *   - cu_seqlens is int32[num_seqs + 1]: cu[0] = 0, non-decreasing, cu[num_seqs] = total
 *     tokens. Empty sequences are allowed and produce no rows.
 *   - Non-finite input values are outside the contract.
 */
#ifndef FP8ATTN_H
#define FP8ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8attn_status {
  FP8ATTN_OK = 0,
  FP8ATTN_EINVAL = -1,      /* a null pointer, a size out of range, inconsistent cu_seqlens */
  FP8ATTN_EUNSUPPORTED = -2, /* a valid request the library does not implement (head_dim != 128) */
  FP8ATTN_EHIP = -3          /* the HIP runtime reported an error while enqueuing */
} fp8attn_status;

/* Scale modes of fp8attn_scales. */
#define FP8ATTN_DYNAMIC 0 /* scale from the 16-slot ring of observed amax values */
#define FP8ATTN_STATIC 1  /* scale from a calibrated amax times a margin */

/* Flags of fp8attn_forward. */
#define FP8ATTN_SKIP 1u    /* run the BF16 kernel on the unquantised inputs; state is not read */
#define FP8ATTN_OBSERVE 2u /* dynamic scaling inside the call: the FP8 path quantises with
                              fp8attn_quantize_dynamic (observe + ring + scales + quantise)
                              instead of the state's current scales; excludes SKIP */

#define FP8ATTN_RING_SLOTS 16
#define FP8ATTN_E4M3_MAX 448.0f
#define FP8ATTN_DEFAULT_MARGIN 1.5f

/*
 * Per-attention-layer scale state, in DEVICE memory, owned by the caller.
 * The layout is part of the ABI so that callers can inspect, snapshot and restore it
 * by copying bytes. Tensor index t: 0 = Q, 1 = K, 2 = V.
 *   ring[t][s]   amax observed by dynamic forward number f is stored in slot f mod 16
 *                (vLLM docs "FP8 ViT Encoder Attention", "Usage": 16 observed values).
 *   count        number of dynamic scale updates so far (the next slot is count mod 16).
 *   scale[t]     dequantisation scale A/448 of the current forward.
 *   inv_scale[t] quantisation multiplier 448/A of the current forward.
 *   amax[t]      the A behind scale[t] (window maximum, or static amax times margin).
 *   moved        bit t set when the last dynamic scale update changed tensor t's window
 *                maximum, i.e. its new observation exceeded the other 15 slots (0 after a
 *                static update); fp8attn_quantize_dynamic re-quantises exactly those.
 *   cur[s][t]    (t < 3) the amax being gathered by fp8attn_observe_amax, striped: the
 *                observation of tensor t is the maximum over the FP8ATTN_CUR_STRIPES
 *                stripes s of these fp32 bit images (a non-negative float compares like
 *                its bit pattern). Each block of an observing kernel folds its maximum
 *                into the stripe of its block index, and each stripe is a 64-byte line
 *                of its own (words 3..15 are unused), because device atomics on one line
 *                serialise. Gathered and cleared by fp8attn_scales.
 */
#define FP8ATTN_CUR_STRIPES 16

typedef struct fp8attn_state {
  float ring[3][FP8ATTN_RING_SLOTS];
  uint32_t count;
  float scale[3];
  float inv_scale[3];
  float amax[3];
  uint32_t moved;
  uint32_t reserved[5];
  uint32_t cur[FP8ATTN_CUR_STRIPES][16];
} fp8attn_state;

/* Size in bytes of fp8attn_state (1280). */
size_t fp8attn_state_bytes(void);

/*
 * Zero a state (empty ring, count 0, no pending observation). Call once per attention
 * layer before its first forward. Implemented with a kernel, not a memset node.
 * Errors: EINVAL if state is NULL.
 */
int fp8attn_state_reset(void* state, void* stream);

/*
 * Observe the per-tensor absolute maximum of Q, K and V for this forward
 * (vLLM docs "FP8 ViT Encoder Attention", "Usage": the amax of Q, K and V is observed on
 * every dynamic forward). One launch reads all three bf16 tensors of n elements each
 * (n = total_tokens * num_heads * head_dim; 16-byte aligned pointers) and folds
 * max|x| into the striped state->cur[.][t] with at most one atomic per block and tensor.
 * The result is exact (a bf16 magnitude). n = 0 observes 0. Must be followed by exactly one fp8attn_scales.
 * Errors: EINVAL for a NULL state, NULL tensor with n > 0, n < 0, or a misaligned pointer.
 */
int fp8attn_observe_amax(void* state, const void* q, const void* k, const void* v, int64_t n,
                         void* stream);

/*
 * Compute this forward's scales (vLLM docs "FP8 ViT Encoder Attention", "Usage" and
 * "Scale file format").
 *   mode FP8ATTN_DYNAMIC: ring[t][count mod 16] = the observation (the maximum of
 *     cur[.][t]); A_t = max over the 16 slots (empty slots hold 0); count += 1.
 *     static_amax_host and margin are ignored.
 *   mode FP8ATTN_STATIC: A_t = fp32(static_amax_host[t] * margin); the ring and count are
 *     left unchanged. static_amax_host is a HOST array of 3 floats (q, k, v calibrated
 *     amax); margin > 0 (the pages' default is 1.5, FP8ATTN_DEFAULT_MARGIN).
 *   Both modes: A' = max(A_t, 2^-64); scale[t] = fp32(A'/448) and inv_scale[t] =
 *     fp32(448/A'), each a correctly rounded division; cur is cleared.
 * One single-wave launch; no host synchronisation.
 * Errors: EINVAL for a NULL state, an unknown mode, a NULL static_amax_host in static
 * mode, a static amax that is negative or not finite, a margin that is not > 0 and finite,
 * or a product fp32(static amax * margin) that overflows to infinity.
 */
int fp8attn_scales(void* state, int mode, const float* static_amax_host, float margin,
                   void* stream);

/*
 * Workspace needed by fp8attn_forward on the FP8 path, in bytes:
 *   Q8 e4m3 [T][H][D] at offset 0,
 *   K8 e4m3 [T][H][D] at offset T*H*D,
 *   V8t e4m3 [H][D][Tp] at offset 2*T*H*D: V transposed so that keys are contiguous,
 *     where sequence i occupies columns [pad_start(i), pad_start(i) + S_i) with
 *     pad_start(i) = roundup(cu[i], 128) + 128*i, and every other column is 0;
 *     Tp = roundup(T, 128) + 128*num_seqs. (Every start is 128-aligned and lies past the
 *     previous sequence's last column, so whole 64-key tiles read past a sequence's end
 *     see zeros, and each 128-column tile belongs to one sequence.)
 * Returns 0 for negative or overflowing arguments.
 */
size_t fp8attn_workspace_bytes(int64_t total_tokens, int num_seqs, int num_heads,
                               int head_dim);

/*
 * Quantise Q, K, V into the workspace layout above with the state's inv_scale
 * (q8 = E4M3(fp32(x * inv_scale[t])), round to nearest even, saturating to +-448; the
 * sign of zero is kept). This is the first half of the FP8 path of fp8attn_forward,
 * exposed so that the bytes can be checked. cu_seqlens and cu_seqlens_host describe the
 * same int32[num_seqs + 1] array (device and host copies).
 * Errors: as fp8attn_forward.
 */
int fp8attn_quantize(const void* state, const void* q, const void* k, const void* v,
                     const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int num_seqs,
                     int num_heads, int head_dim, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * One dynamic forward's scaling and quantisation in one call (vLLM docs "FP8 ViT Encoder
 * Attention", "Usage": every dynamic forward observes the Q/K/V amax and the 16-slot ring
 * drives its scale). The result -- state (ring, count, amax, scales) and workspace bytes --
 * is exactly that of fp8attn_observe_amax, fp8attn_scales(FP8ATTN_DYNAMIC) and
 * fp8attn_quantize in sequence. The work differs: the window maximum of this forward is
 * max(A_pred, amax) with A_pred the maximum of the 15 ring slots that stay, so Q, K and V
 * are quantised with A_pred's scale while their amax is observed in the same pass; after
 * the scales update, only a tensor whose window maximum moved (its amax is a new maximum,
 * e.g. on the first forward) is quantised again. In steady state Q, K and V are read once.
 * The state's pending observation (cur) must be clear, as every fp8attn_scales call and
 * fp8attn_state_reset leave it. Arguments as fp8attn_quantize; the state is written.
 * Errors: as fp8attn_quantize.
 */
int fp8attn_quantize_dynamic(void* state, const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                             int num_seqs, int num_heads, int head_dim, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * FP8 attention on a workspace already filled by fp8attn_quantize with this state's
 * scales (the second half of the FP8 path of fp8attn_forward, which is exactly
 * fp8attn_quantize followed by fp8attn_attend). Arguments and the computation are those of
 * fp8attn_forward's FP8 path; q, k and v are not read. Lets a caller reuse one quantised
 * workspace, or time the attention kernel on its own.
 * Errors: as fp8attn_forward (q, k, v are not needed and may be NULL).
 */
int fp8attn_attend(const void* state, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                   int num_seqs, int num_heads, int head_dim, float softmax_scale,
                   const void* workspace, size_t workspace_bytes, void* out, void* stream);

/*
 * Variable-length, non-causal attention forward over packed sequences (vLLM-Omni
 * "Quantized KV Cache", "Overview" and "Parameters"; vLLM docs "FP8 ViT Encoder
 * Attention", "Usage"). For every sequence i, head h and query row r of that sequence:
 *   O[r,h,:] = sum_j w_j V[j,h,:] over the keys j of sequence i only.
 * FP8 path (flags without FP8ATTN_SKIP): quantises Q, K, V with the state's scales into
 *   `workspace` (see fp8attn_workspace_bytes), then s_j = (q8.k8_j) * scale_q * scale_k *
 *   softmax_scale; with m = max_j s_j, the row maximum over all keys of the sequence, and
 *   M = ceil(m * log2 e), p8_j = E4M3(448 * 2^(s_j * log2 e - M)) (448 times a power of
 *   two, so the largest p8_j is in [224, 448]); O = scale_v * sum_j p8_j v8_j / sum_j p8_j.
 *   The PV product uses the E4M3 V; accumulation and softmax are fp32 (the scores and
 *   products on FP8 matrix cores); O is bf16. The kernel finds M in the same pass as the
 *   weights (rescaling by powers of two as it grows), which gives this result whatever
 *   the key tiling, except that a weight below 2^-6 of a key visited before the row's
 *   final M keeps the finer rounding of its provisional reference (at most 2^-9 apart on
 *   the weights' scale, where the largest weight is 224 to 448).
 *   Requires a preceding fp8attn_scales on this state (same stream), unless
 *   FP8ATTN_OBSERVE is set: then the call itself performs the dynamic observe + ring +
 *   scales update (fp8attn_quantize_dynamic) before the attention, writing the state.
 * BF16 path (FP8ATTN_SKIP): w_j = softmax(q.k_j * softmax_scale) in fp32 with P rounded
 *   to bf16 for the PV product; workspace and state are not used (may be NULL).
 * softmax_scale <= 0 selects 1/sqrt(head_dim).
 * cu_seqlens (device) and cu_seqlens_host (host) must hold the same values; the host
 * copy is used for checks and launch sizes so that no device read-back is needed.
 * An empty batch (cu_seqlens_host[num_seqs] == 0) reads and writes no tensor element; q, k,
 * v and out may then be NULL (with FP8ATTN_OBSERVE the ring still records a 0 observation).
 * Errors: EINVAL for NULL pointers (other than those just named), num_seqs < 1, num_heads < 1, total tokens beyond
 * 2^31-1 elements per head row, a host cu_seqlens that does not start at 0 or decreases,
 * a workspace smaller than fp8attn_workspace_bytes, unknown flag bits, SKIP together with
 * OBSERVE, or a NULL state on the FP8 path; EUNSUPPORTED for head_dim != 128, or when the longest sequence times
 * num_heads * head_dim, or head_dim times the padded key count, reaches 2^31 (on the BF16
 * path, when twice the former does).
 */
int fp8attn_forward(void* state, const void* q, const void* k, const void* v,
                    const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int num_seqs,
                    int num_heads, int head_dim, float softmax_scale, unsigned flags,
                    void* workspace, size_t workspace_bytes, void* out, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture, serving
 * loops and harnesses that forbid hipMalloc. The same call as fp8attn_forward, without the
 * workspace argument: the FP8 path's workspace is a fixed device array inside the library,
 * FP8ATTN_NOALLOC_SCRATCH_BYTES long (64 MiB: up to 10 880 tokens at 16 heads), one
 * per GPU, held from the library's first use on that GPU until the process ends. The call
 * allocates nothing; on its first use on a device it looks up that device's array address
 * (hipGetSymbolAddress) with that device current. The device that is current during the
 * call must be the stream's device.
 * Concurrency: all calls on one GPU share its array, so calls that overlap in time on one
 * GPU (two streams, two host threads) race on it and must be serialised by the caller.
 * Nothing in the array needs to start at zero; a call's results do not depend on what an
 * earlier call left there.
 * Errors: as fp8attn_forward; EINVAL (before anything is enqueued) when the FP8 path would
 * need more than FP8ATTN_NOALLOC_SCRATCH_BYTES, i.e. when fp8attn_workspace_bytes(total
 * tokens, num_seqs, num_heads, head_dim) exceeds it; EHIP when the array's address cannot
 * be obtained. The BF16 path (FP8ATTN_SKIP) does not touch the array.
 */
#define FP8ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fp8attn_forward_noalloc(void* state, const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                            int num_seqs, int num_heads, int head_dim, float softmax_scale,
                            unsigned flags, void* out, void* stream);

/* Message describing the last non-OK return on the calling thread ("" if none). */
const char* fp8attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8ATTN_H */
