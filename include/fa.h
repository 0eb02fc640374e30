/*
 * fa.h -- C ABI of the fused exact-attention forward pass for AMD Instinct MI355X (gfx950).
 *
 * The operation is exact attention for every (batch b, head h):
 *
 *     O = softmax(Q K^T * scale + mask) V,    LSE_i = ln sum_{j visible to i} exp(scale * q_i . k_j)
 *
 * as defined in "FlashAttention Interview Questions: IO Complexity, Tiling, and Numerical
 * Stability" (cswork.org), section "What is FlashAttention exact about?" (scores = Q K^T /
 * sqrt(d); weights = row_softmax(scores + mask); output = weights V, one head of length N and
 * width d).  It is computed tile by tile with running row statistics -- the update of the same
 * page's section "How can softmax be computed across tiles?" -- inside one kernel, so the
 * N x N score matrix never exists in device memory ("FlashAttention 1, 2 & 3: Memory Tiling &
 * Eliminating the O(N^2) HBM Bottleneck", section 2, "Kernel Fusion").  The log-sum-exp is the
 * compact per-row normalisation information that a backward pass needs (cswork.org page,
 * section "Why can recomputation help training?").
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The library allocates,
 *     frees and synchronises nothing and keeps no state between calls except a thread-local
 *     copy of the last HIP error and, for fa_fwd_varlen_noalloc only, one fixed device array
 *     per device (see there).  Work is enqueued on `stream` (a hipStream_t; NULL means the
 *     default stream) and the call returns without waiting for it.
 *   - Layout: Q, K, V and O are [B, H, N, d] contiguous row-major (d fastest); LSE is [B, H, N].
 *   - Masks (bit flags, FA_MASK_*): under FA_MASK_CAUSAL key j is visible to query i only when
 *     j <= i (square, aligned positions).  Under FA_MASK_KEY_PADDING key j of batch element b is
 *     visible only when j < seqlens[b] (values are clamped to [0, N]); query rows are never
 *     masked.  Masked scores are replaced (not offset) so they carry exactly zero weight, and
 *     extreme finite values stored at masked K/V positions do not change any visible output.
 *   - A row with no visible key (only possible when seqlens[b] == 0) gets O = 0 and LSE = -inf,
 *     never NaN (the cswork.org page asks that this case be defined: section "Does subtracting
 *     the maximum solve every numerical issue?").
 *   - Arguments are validated on the host before any HIP call; nothing is launched when a check
 *     fails.  B, H or N equal to 0 is a no-op that returns FA_OK.
 *   - NaN or infinite values in Q, K or V are outside the contract.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_VERSION 10500 /* major*10000 + minor*100 + patch */

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,  /* null pointer, negative size, unknown mask bit, padding without
                                seqlens, scale negative or not finite, misaligned pointer,
                                O aliasing an input, size overflow */
    FA_ERR_UNSUPPORTED = 2,  /* valid arguments the library has no kernel for (d, dtype pair) */
    FA_ERR_HIP = 3,          /* the launch failed; fa_last_hip_error() gives the hipError_t */
    FA_ERR_SCRATCH_LIMIT = 4 /* fa_fwd_varlen_noalloc only: the call needs more workspace than the
                                library's fixed scratch array holds (fa_scratch_bytes()) */
} fa_status;

enum { FA_MASK_NONE = 0, FA_MASK_CAUSAL = 1, FA_MASK_KEY_PADDING = 2 };
enum { FA_DTYPE_F32 = 0, FA_DTYPE_BF16 = 1, FA_DTYPE_FP8_E4M3 = 2 };
/* Causal alignment of fa_fwd_varlen (see there). */
enum { FA_ALIGN_BOTTOM_RIGHT = 0, FA_ALIGN_TOP_LEFT = 1 };

/*
 * fa_fwd -- the fused forward pass.
 *
 *   q, k, v   [B, H, N, d] device tensors of `in_dtype`, 16-byte aligned.
 *   o         [B, H, N, d] device tensor of `out_dtype`, 16-byte aligned; written.  Must not
 *             overlap q, k or v.
 *   lse       [B, H, N] float32 device tensor, 4-byte aligned, natural-log log-sum-exp of the
 *             visible scaled scores; written.  NULL: not stored.
 *   B, H, N   batch, heads, sequence length (>= 0).  d: head width.
 *   scale     multiplier of every dot product (finite, >= 0; normally 1/sqrt(d)).
 *   mask_kind FA_MASK_* bits (0..3).
 *   seqlens   device int32[B], valid key length per batch element; required iff
 *             FA_MASK_KEY_PADDING is set, ignored otherwise.
 *   in_dtype, out_dtype   supported pairs: (BF16, BF16) and (BF16, F32) with d in {64, 128};
 *             (F32, F32) with d in {64, 128}.  Products take bf16 operands with float32
 *             accumulation; with a float32 output the probabilities enter the value product
 *             as a two-term bf16 split, so their rounding stays below 2^-16 relative.
 *             float32 inputs are multiplied in float32 throughout.  FP8_E4M3 inputs (BF16 or
 *             F32 output): as fa_fwd_fp8 with every descale 1.
 *   stream    hipStream_t to enqueue on (NULL = default stream).
 *
 * Returns an fa_status.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int mask_kind, const int32_t* seqlens,
           int in_dtype, int out_dtype, void* stream);

/*
 * fa_fwd_dropout -- fa_fwd with dropout on the attention probabilities:
 *
 *     O = (P * Z) V,   Z_ij = keep_ij * 256 / (256 - t),   t = round(256 * p_drop),
 *
 * with P the probabilities of fa_fwd; the LSE output is that of P, before dropout.  The
 * cswork.org page asks that dropout be tested against the implementation's random-number and
 * reproducibility contract (section "Does subtracting the maximum solve every numerical
 * issue?"); this is the contract:
 *   keep_ij for query row i and key j of head bh = b * H + h is
 *       byte (4 * (i % 4) + (j % 4)) of Philox4x32-10(counter = (j / 4, i / 4, bh, offset),
 *                                                     key = (seed & 0xffffffff, seed >> 32)) >= t,
 *   the 16 output bytes taken from the four 32-bit words in order, each little-endian
 *   (Philox4x32-10: Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
 *   3", SC '11).  The same (seed, offset) gives the same mask on every run and every device;
 *   the drop probability is quantised to 1/256.
 *
 *   p_drop    drop probability, finite, 0 <= p_drop < 255.5/256 (else FA_ERR_INVALID_ARG).
 *   seed, offset   Philox key and fourth counter word.
 *   Other arguments as for fa_fwd; in_dtype must be BF16 (F32 inputs: FA_ERR_UNSUPPORTED).
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int mask_kind, const int32_t* seqlens,
                   float p_drop, uint64_t seed, uint32_t offset,
                   int in_dtype, int out_dtype, void* stream);

/*
 * fa_fwd_fp8 -- fa_fwd for 8-bit floating-point inputs with per-tensor descales:
 *
 *     O = softmax(scale * (dq Q)(dk K)^T + mask) (dv V),   LSE as for fa_fwd on those inputs,
 *
 * where Q, K and V hold OCP FP8 E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; subnormals; 0x7F and 0xFF are NaN, no infinities; largest finite 448).  The page
 * "FlashAttention 1, 2 & 3: Memory Tiling & Eliminating the O(N^2) HBM Bottleneck", section 3,
 * names FP8 support among the third kernel generation's hardware features and fixes nothing
 * more; the result defined here is exact attention on the real values descale * code.
 *
 *   q, k, v   [B, H, N, d] device byte tensors of E4M3 codes, 16-byte aligned.
 *   descale_q, descale_k, descale_v   finite, >= 0; scale * descale_q * descale_k must be a
 *             finite float32 (else FA_ERR_INVALID_ARG).
 *   out_dtype BF16 or F32.  d in {64, 128}.
 *   Other arguments, layouts, masks and validation as for fa_fwd.
 *
 * Q K^T runs on the 8-bit matrix cores with float32 accumulation (exact products); V is
 * widened to bf16 without rounding, so the value product, the probability precision and the
 * tolerances are those of fa_fwd with bf16 inputs.  Codes 0x7F / 0xFF (NaN) are outside the
 * contract, like NaN inputs of fa_fwd.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, float descale_q, float descale_k, float descale_v,
               int mask_kind, const int32_t* seqlens, int out_dtype, void* stream);

/*
 * fa_fwd_variant -- fa_fwd with an explicit kernel variant, for tests and tuning only.
 * variant 0 is what fa_fwd runs.  Other values select alternative, equally exact
 * implementations of the same operation (see fa_variant_count); every variant must pass the
 * same parity tests.  An unknown variant returns FA_ERR_UNSUPPORTED.
 */
int fa_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int mask_kind, const int32_t* seqlens,
                   int in_dtype, int out_dtype, void* stream, int variant);

/*
 * fa_bwd -- gradients of the forward pass with respect to Q, K and V.
 *
 * With P the attention probabilities of the forward pass (masked keys have P = 0) and dO the
 * gradient arriving at O:
 *     dV = P^T dO,   dP = dO V^T,   D_i = dO_i . O_i,   dS = P * (dP - D),
 *     dQ = scale * dS K,   dK = scale * dS^T Q.
 * Only O receives a gradient; the LSE output is not differentiated.  P is recomputed tile by
 * tile from Q, K and the LSE saved by fa_fwd instead of being stored ("FlashAttention Interview
 * Questions: IO Complexity, Tiling, and Numerical Stability" (cswork.org), section "Why can
 * recomputation help training?"), so no N x N buffer exists.
 *
 *   q, k, v, o, dout  [B, H, N, d] device tensors of `in_dtype`, 16-byte aligned: the forward
 *             inputs, its output O and the upstream gradient dO.
 *   lse       [B, H, N] float32, 4-byte aligned: the natural-log LSE fa_fwd wrote for these
 *             inputs (rows with no visible key hold -inf and receive no gradient).
 *   delta     [B, H, N] float32 workspace owned by the caller, 4-byte aligned; receives
 *             D_i = dO_i . O_i.
 *   dq, dk, dv  [B, H, N, d] device tensors of `grad_dtype`, 16-byte aligned; written.  Keys no
 *             row may see (masked, or past seqlens[b]) get zero gradient.
 *   B, H, N, d, scale, mask_kind, seqlens, stream   as for fa_fwd.
 *   in_dtype, grad_dtype   supported: (BF16, F32) with d in {64, 128}.  P and dS enter the
 *             value and key products as bf16 values with float32 accumulation.
 * dq, dk, dv and delta must not overlap each other or any input.  Three kernels are enqueued on
 * `stream`; there are no atomics, so results are identical from run to run.
 * Returns an fa_status (validation as for fa_fwd, before any HIP call).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, float* delta, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int mask_kind, const int32_t* seqlens,
           int in_dtype, int grad_dtype, void* stream);

/*
 * fa_fwd_varlen -- the forward pass over a packed batch of sequences with their own query and
 * key lengths: unequal query and key counts, variable-length (packed) batches and decoding
 * (one or a few new query rows against a long key range).  The cswork.org page warns that
 * these cases change which keys a query may see (section "Does subtracting the maximum solve
 * every numerical issue?") and separates prefill from single-token decoding (closing benchmark
 * section); the visibility rule is therefore explicit here:
 *
 *   Sequence b owns query tokens cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (Lq of them) and key /
 *   value tokens cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 (Lk of them).  Sequences never see each
 *   other's keys.  Without a mask every key of the sequence is visible.  Under FA_MASK_CAUSAL,
 *   query row i (0-based within its sequence) sees key j iff j <= i + delta, with
 *     causal_align == FA_ALIGN_BOTTOM_RIGHT: delta = Lk - Lq (the queries are the last Lq of
 *                     the Lk positions: decoding, chunked prefill);
 *     causal_align == FA_ALIGN_TOP_LEFT:     delta = 0 (query i and key i share a position).
 *   The two agree when Lq == Lk.  A row that sees no key (bottom-right with Lq > Lk, or Lk == 0)
 *   gets O = 0 and LSE = -inf.
 *
 *   q, o      [total_q, H, d] token-major (d fastest, then heads), 16-byte aligned; q of
 *             `in_dtype`, o of `out_dtype`, written.  o must not overlap any input.
 *   k, v      [total_k, H, d] of `in_dtype`, 16-byte aligned (may be NULL when total_k == 0).
 *   lse       [H, total_q] float32, 4-byte aligned, natural-log log-sum-exp; NULL: not stored.
 *   cu_seqlens_q, cu_seqlens_k   device int32[B + 1] prefix sums of the lengths: first entry 0,
 *             non-decreasing, last entry <= total.  Each length must be <= max_seqlen_q /
 *             max_seqlen_k.  (Memory safety does not depend on this: entries are clamped into
 *             the tensors and lengths to the maxima, rows past max_seqlen_q are then not
 *             written and keys past max_seqlen_k are ignored.)
 *   B, H      sequences and heads.  max_seqlen_q, max_seqlen_k: the longest query and key
 *             sequence (>= 0); they size the launch.  max_seqlen_k * H * d * 2 must be < 2^32.
 *   d, scale  as for fa_fwd.  mask_kind: FA_MASK_NONE or FA_MASK_CAUSAL (key lengths come
 *             from cu_seqlens_k, so FA_MASK_KEY_PADDING is invalid here).
 *   causal_align   FA_ALIGN_BOTTOM_RIGHT or FA_ALIGN_TOP_LEFT; required (validated) even
 *             without the causal mask, which ignores it.
 *   workspace, workspace_bytes   device scratch owned by the caller, 16-byte aligned, of at
 *             least fa_fwd_varlen_workspace_size(B, H, max_seqlen_q, max_seqlen_k, d) bytes
 *             (NULL / 0 when that size is 0).  It must not overlap any other argument; its
 *             contents on entry do not matter and on return are unspecified.
 *   in_dtype, out_dtype   (BF16, BF16) or (BF16, F32), d in {64, 128}.
 *   stream    hipStream_t to enqueue on (NULL = default stream).
 *
 * Kernels: when max_seqlen_q <= 4 (decoding shapes) the keys of every (sequence, head) are cut
 * into ranges processed by separate workgroups with fp32 vector arithmetic (the work is bound
 * by the K/V stream), and a second kernel merges the ranges' running statistics; otherwise the
 * tiled MFMA kernel of fa_fwd runs on the packed layout.  When those tiles would number at most
 * 128 (e.g. one long sequence) and max_seqlen_k >= 1024, each (sequence, head)'s keys are cut
 * into ranges there too: every range runs the tiled kernel into the workspace (float32 rows and
 * log-sum-exps), and a second kernel merges the ranges, with the same rescaling, into o and
 * lse.  No atomics, and the ranges merge in a fixed order: results are identical from run to
 * run.  Validation is done on the host before any HIP call; B, H, total_q or
 * max_seqlen_q equal to 0 is a no-op.  Returns an fa_status.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                  int B, int H, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                  int d, float scale, int mask_kind, int causal_align,
                  void* workspace, size_t workspace_bytes,
                  int in_dtype, int out_dtype, void* stream);

/*
 * Bytes of workspace fa_fwd_varlen needs for these sizes (0: none).  A pure function of its
 * arguments; 0 for sizes fa_fwd_varlen would reject.  Decoding shapes with their keys split:
 * B*H*ranges*rows*(d+2)*4 bytes (rows 1 or 4).  Prefill shapes with their keys split:
 * ranges*B*H*max_seqlen_q*(d+1)*4 bytes.
 */
size_t fa_fwd_varlen_workspace_size(int B, int H, int max_seqlen_q, int max_seqlen_k, int d);

/*
 * fa_fwd_varlen_noalloc -- fa_fwd_varlen for callers that cannot allocate device memory: code
 * recorded into a HIP graph, tight serving loops, harnesses that forbid hipMalloc.  It takes no
 * workspace argument; the key ranges' partial states go to a fixed array inside the library
 * instead (a `__device__` array of fa_scratch_bytes() = 9 MiB, which holds the workspace of every
 * decoding size fa_fwd_varlen accepts).  Each device keeps its own copy from the library's first
 * call on it until the process ends; the call itself allocates nothing.
 *
 *   Arguments, layouts, visibility rule and results: those of fa_fwd_varlen with the same
 *   arguments.  Kernels: those of fa_fwd_varlen (bitwise equal outputs), except that a prefill
 *   shape whose split keys would need more than the array runs the tiled kernel unsplit (equal
 *   within rounding, not bitwise).  Validation as for fa_fwd_varlen, plus FA_ERR_SCRATCH_LIMIT if
 *   a decoding shape's fa_fwd_varlen_workspace_size() exceeds fa_scratch_bytes().
 *   The first call on a device looks up the array's address there (hipGetSymbolAddress) with that
 *   device current; a failure of that lookup returns FA_ERR_HIP.
 *
 * Every call on one device shares that device's array, and the array keeps the last call's
 * contents (each call writes every entry it later reads, so nothing needs clearing).  Calls that
 * can overlap in time on one device -- on different streams, or from several host threads without
 * ordering -- race on the array and may return wrong results: order them on one stream.
 */
int fa_fwd_varlen_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int B, int H, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                          int d, float scale, int mask_kind, int causal_align,
                          int in_dtype, int out_dtype, void* stream);

/* Bytes of the fixed array fa_fwd_varlen_noalloc uses per device (9 MiB). */
size_t fa_scratch_bytes(void);

/*
 * fa_bwd_dropout -- gradients of fa_fwd_dropout's output with respect to Q, K and V, with the
 * dropout mask of the same (p_drop, seed, offset) regenerated from the contract of
 * fa_fwd_dropout (no mask is stored):
 *     dV = (P * Z)^T dO,   dP = Z * (dO V^T),   D_i = dO_i . O_i,   dS = P * (dP - D),
 *     dQ = scale * dS K,   dK = scale * dS^T Q,   Z = keep * 256 / (256 - round(256 p_drop)).
 * o must be fa_fwd_dropout's output and lse its LSE.  Arguments, layouts and validation as for
 * fa_bwd, plus p_drop, seed and offset as for fa_fwd_dropout.
 */
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, float* delta, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int mask_kind, const int32_t* seqlens,
                   float p_drop, uint64_t seed, uint32_t offset,
                   int in_dtype, int grad_dtype, void* stream);

/* Number of kernel variants fa_fwd_variant accepts (variants are 0 .. count-1). */
int fa_variant_count(void);

/* Static, never-NULL description of a status code (unknown codes get a generic string). */
const char* fa_status_str(int status);

/* hipError_t behind the most recent FA_ERR_HIP returned on this thread (0 if none). */
int fa_last_hip_error(void);

/* FA_VERSION of the built library. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
