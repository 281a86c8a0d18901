/*
 * sattn.h — C ABI of the MI355X (gfx950) quantized video-DiT self-attention library.
 *
 * The numerical program follows the pages "H3 Performance Roadmap"
 * (sections "Measured GB10 Baseline" → "SageAttention 2.2.0 internals", the Sage2 phase
 * decomposition paragraph after "The fresh block kernel-time distribution", and "Phase 4:
 * Dense Sage-Compatible Attention") and "Phase 2B Aligned Numerical Prototype" (sections
 * "Decision" and "Exactness"):
 *
 *   1. K smoothing: subtract the per-(sequence, head, channel) mean of K.
 *   2. Q and smoothed K → symmetric INT8, one FP32 scale per 64-token block.
 *   3. V → OCP FP8 E4M3, one FP32 scale per (sequence, head, channel).
 *   4. Scores: INT8·INT8 → exact INT32 accumulators → FP32 scores.
 *   5. Online softmax over 64-key epochs in increasing key order (running max m and
 *      denominator d per query row), probabilities → E4M3 (×448), FP8 P·V with FP32
 *      accumulation into the running output RO, final reciprocal of d, BF16 output.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library never
 *    allocates device memory and keeps no state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *    entry point only enqueues work on `stream`; nothing synchronises the host.
 *  - Argument validation is synchronous and happens before any HIP call: a call that
 *    returns anything but SATTN_OK has enqueued nothing.  A failed kernel launch is
 *    reported as SATTN_EHIP.  Device-side faults surface at the caller's next
 *    synchronisation.  No C++ exception crosses this interface.
 *  - Head dimension D must be 128.
 *  - BF16 views: element (b, t, h, c) lives at ptr + b*stride_b + t*stride_t + h*stride_h + c
 *    (strides in elements; the channel stride is 1).  The base pointer must be 16-byte
 *    aligned and stride_t, stride_h, stride_b multiples of 8, so every (token, head) row
 *    is 256 contiguous, 16-byte-aligned bytes.  This admits contiguous BLHD/BHLD tensors
 *    and the projection-strided slices of a fused [L, 3, H, D] QKV tensor.
 *  - Sequences ("segments"): in dense mode there are B segments of Lq query tokens and
 *    Lk key tokens each (segment b uses batch index b).  In varlen mode the segments are
 *    given by device int32 prefix sums cu_seqlens_q / cu_seqlens_k of length nseg+1
 *    (cu[0] = 0, non-decreasing); segment s covers packed tokens [cu[s], cu[s+1]) and
 *    stride_b is ignored.  Attention is block-diagonal: each segment's queries attend
 *    to its own keys only, with no causal mask.  Empty segments are legal.
 *
 * Quantized buffers (written by sattn_quantize_qkv, read by sattn_fwd*)
 * ---------------------------------------------------------------------
 *  Each segment's tokens are padded to whole 64-token blocks.  Segment s starts at
 *  block index  s*ceil(Lq/64)  (dense)  or  cu[s]/64 + s  (varlen, integer division).
 *  Capacities in blocks:  qblk_cap >= floor(total_q/64) + nseg  (likewise kblk_cap),
 *  where total_q is B*Lq (dense) or cu_seqlens_q[nseg] (varlen); sattn_quant_query
 *  returns exactly that bound.  Padding rows are written as zeros.
 *
 *  q, k : int8,  [H][blk_cap][8192]: one 8 KiB tile per 64-token block in MFMA operand
 *         order.  Byte ((t*4 + u)*64 + g*32 + i)*16 + s of a tile holds token 32*t + i,
 *         channel 64*g + 16*u + s (t,g in {0,1}; u in 0..3; i in 0..31; s in 0..15).
 *  q_scale : float, [H][qblk_cap][64 / q_scale_rows]: the FP32 scale of each 64-token
 *         block, or of each 32-row half of it (q_scale_rows = 32).
 *  k_scale : float, [H][kblk_cap], the FP32 scale of each 64-token block.
 *  k_mean : float, [nseg][H][128], the per-channel mean subtracted from K.
 *  v    : OCP E4M3 bytes, [H][kblk_cap][8192]: one tile per 64-key block, channel-major.
 *         Byte ((w*2 + f)*64 + g*32 + i)*16 + s holds channel 32*w + i and key
 *         32*f + 8*(s/4) + 4*g + (s%4) of the block (w in 0..3; f,g in {0,1}).
 *  v_scale : float, [nseg][H][128], the per-channel FP32 scale of V.
 */
#ifndef SATTN_H_
#define SATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SATTN_API __attribute__((visibility("default")))
#else
#define SATTN_API
#endif

typedef int32_t sattn_status;
#define SATTN_OK 0
#define SATTN_EINVAL 1       /* bad pointer, size, stride, alignment or segment count   */
#define SATTN_EUNSUPPORTED 2 /* well-formed but outside what the kernels implement (D, grid size) */
#define SATTN_ENOSPACE 3     /* a capacity or workspace is smaller than required       */
#define SATTN_EHIP 4         /* a HIP launch or runtime call failed                    */

/* Strided BF16 input view (see the conventions above). */
typedef struct {
  const void* ptr;
  int64_t stride_b, stride_t, stride_h;
} sattn_bf16_in;

/* Strided BF16 output view: same addressing as the input, token-major. */
typedef struct {
  void* ptr;
  int64_t stride_b, stride_t, stride_h;
} sattn_bf16_out;

/* Caller-owned quantized Q/K/V buffers and their capacities (see the layout above).
 * q_scale_rows selects the Q scale granularity, read by sattn_quantize_qkv and by every
 * forward entry point (the two must agree): 64 (or 0) = one scale per 64-token block,
 * 32 = one scale per 32 query rows, the "per-warp INT8 Q" policy of the roadmap page's
 * "Phase 4: Dense Sage-Compatible Attention" (a 128-query tile split over four QK warps);
 * K keeps one scale per 64 tokens in both.  Any other value gives SATTN_EINVAL. */
typedef struct {
  int8_t* q;
  float* q_scale;
  int8_t* k;
  float* k_scale;
  float* k_mean;
  uint8_t* v;
  float* v_scale;
  int64_t qblk_cap, kblk_cap;
  int32_t q_scale_rows;
} sattn_qkv_quant;

/* Byte sizes of every buffer of sattn_qkv_quant, plus scratch sizes. */
typedef struct {
  int64_t qblk_cap, kblk_cap;
  size_t q_bytes, q_scale_bytes, k_bytes, k_scale_bytes, k_mean_bytes, v_bytes, v_scale_bytes;
                                /* q_scale_bytes holds either Q scale granularity     */
  size_t quant_workspace_bytes; /* workspace of sattn_quantize_qkv                     */
  size_t fwd_workspace_bytes;   /* workspace of sattn_fwd_varlen, and of sattn_fwd's key split */
} sattn_sizes;

/*
 * sattn_quant_query — host-only, pure.  Fills *out for nseg segments holding total_q
 * query tokens and total_k key tokens (dense: nseg = B, total = B*L) with H heads and
 * head dimension D.  Returns SATTN_EINVAL for nseg < 1, negative totals, H < 1 or a null
 * `out`, and SATTN_EUNSUPPORTED for D != 128.
 */
SATTN_API sattn_status sattn_quant_query(int nseg, int64_t total_q, int64_t total_k, int H, int D, sattn_sizes* out);

/*
 * sattn_quantize_qkv — steps 1–3 of the program above ("Q/K INT8 quantization", "V FP8
 * quantization" and "K smoothing" in the SageAttention internals table of the roadmap
 * page; the later decomposition into K smoothing, Q/K quantization and V
 * transpose/quantization phases).
 *
 *   dense  (cu_seqlens_q == cu_seqlens_k == NULL): nseg = B segments; q holds B x Lq
 *          tokens, k and v hold B x Lk tokens.
 *   varlen (both non-NULL): device int32 arrays of nseg+1 entries; Lq and Lk are the
 *          number of packed tokens the q and k/v views hold (cu[nseg] must not exceed
 *          them; tokens beyond are never read, and a segment reaching past them is
 *          clipped on the device).
 *
 * For each segment s, head h, channel c (all sums in FP64, every scale operation a single
 * correctly rounded FP32 operation):
 *   k_mean[s,h,c] = fl32( (sum_t K[t,h,c]) / Lk_s ),  K' = fl32(K - k_mean)
 *   per 64-token block (Q: per 32 rows when out->q_scale_rows = 32): amax = max|x|,
 *     scale = fl32(amax/127), inv = fl32(127/amax),
 *     code = clamp(rne(fl32(x*inv)), -127, 127)   (x = Q, or K'; amax = 0 → scale 0, codes 0)
 *   v_scale[s,h,c] = fl32(amax_V/448), V8 = e4m3_rne(fl32(V * fl32(448/amax_V)))
 *
 * `workspace` must hold quant_workspace_bytes from sattn_quant_query (16-byte aligned);
 * it is scratch: its contents are undefined after the call.  Returns SATTN_ENOSPACE when
 * a capacity in `out` or workspace_bytes is too small, and SATTN_EUNSUPPORTED when a
 * launch would exceed 2^24 - 1 workgroups of 256 threads (one dispatch counts work-items
 * in 32 bits; the statistics and Q blocks share one grid; far beyond what fits in memory).
 *
 * K and V only: with out->q and out->q_scale both NULL, the Q step is skipped and the q
 * view is not read (it may be NULL); this is the preparation sattn_fwd_fused needs.
 */
SATTN_API sattn_status sattn_quantize_qkv(sattn_bf16_in q, sattn_bf16_in k, sattn_bf16_in v, int nseg, int H, int D,
                                int64_t Lq, int64_t Lk, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, const sattn_qkv_quant* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * sattn_fwd — dense attention forward over quantized inputs (steps 4–5; the pages'
 * "Attention forward" / prequantized mainloop, and the checkpoint list of the
 * Phase 2B report's "Exactness" section).  B segments of Lq queries and Lk keys, H heads,
 * D = 128.  sm_scale multiplies q·k (usually 1/sqrt(D)); it must be finite and > 0.
 *
 * `workspace` (optional, 16-byte aligned, fwd_workspace_bytes of sattn_quant_query) lets
 * the 128-query tiles that would run with CUs left idle split their keys between 2 or 4
 * workgroups (pieces): the tiles of the last dispatch round (two workgroups per CU; the
 * whole grid when it is shorter than a round) when the pieces of each get a CU of their own
 * (at most 128 tiles in 2 pieces or 64 in 4 on a 256-CU device) and the keys span at least
 * 16 (32) epochs of 64.  Each later piece starts from the running max over the keys before
 * it (computed from their scores), so every E4M3 probability equals the sequential
 * recurrence's, and the partial results are merged in piece order as
 * O = sum_q O_q 2^(m_q - m), m = max_q m_q (d likewise).  The workspace must
 * hold zeros before its first use and its counters are left zeroed by every call; calls
 * sharing one workspace must not overlap.  NULL (or too small) runs without the split.
 * The split changes the FP32 summation order of O and d only.
 * The score of query i and key j in 64-blocks (bq, bk) is (bq: the 32-row block of i
 * when qkv->q_scale_rows = 32)
 *   S = fl32(acc * sigma),  sigma = fl32(fl32(q_scale[bq] * c) * k_scale[bk]),
 *   c = fl32(sm_scale * log2(e)) computed in double on the host,
 * and the softmax runs in base 2.  o receives BF16 rows for every valid query token
 * (rows of padding are not written).  A segment with Lq > 0 and Lk = 0 writes zeros.
 */
SATTN_API sattn_status sattn_fwd(const sattn_qkv_quant* qkv, int B, int H, int Lq, int Lk, int D, float sm_scale,
                       sattn_bf16_out o, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sattn_fwd_varlen — block-diagonal (per-segment) version of sattn_fwd for packed
 * sequences; cu_seqlens_q/k are the same device arrays given to sattn_quantize_qkv.
 * total_q and total_k are the packed query and key tokens the views held: rows past
 * total_q are never written, and a segment reaching past total_k keys is clipped there,
 * exactly as sattn_quantize_qkv clipped it (its keys past the K/V views were never
 * quantized).  `workspace` (fwd_workspace_bytes, 16-byte aligned) receives the
 * longest-first schedule of the segments and is scratch for the caller.
 */
SATTN_API sattn_status sattn_fwd_varlen(const sattn_qkv_quant* qkv, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int nseg, int64_t total_q, int64_t total_k, int H,
                              int D, float sm_scale, sattn_bf16_out o, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Checkpoint buffers of sattn_debug_scores: caller-owned device memory; any pointer may be
 * NULL to skip that checkpoint.  Row r of each buffer belongs to the r-th sampled query row
 * (see sattn_debug_scores).  Keys and epochs are numbered within the segment. */
typedef struct {
  int32_t* acc;   /* [rows][ld]: the exact INT32 accumulator sum_c q8[i,c] k8[j,c] of key j   */
  float* s;       /* [rows][ld]: the FP32 score fl32(acc * sigma) of key j (base-2 units)    */
  int64_t ld;     /* row stride of acc and s in elements; keys j >= ld are not written        */
  float* m;       /* [rows][nep]: running max m after epoch e                                 */
  float* d;       /* [rows][nep]: running denominator after epoch e, in units of 448 P (the
                     sum of the unquantized 448 * 2^(S - m) values, FP32)                      */
  float* alpha;   /* [rows][nep]: epoch e's rescale factor 2^(m_{e-1} - m_e) (0 for e = 0)     */
  uint8_t* p8;    /* [rows][nep][64]: epoch e's E4M3 probability bytes e4m3(448 P), key
                     64e + k at index k (keys past the segment's end hold 0)                  */
  float* ro;      /* [rows][nep][128]: the running output RO = sum_j e4m3(448 P_j) * v8_j
                     (v8_j the E4M3 code values; the FP32 accumulators) after epoch e          */
  int64_t nep;    /* epochs recorded: e < nep (later epochs are not written)                  */
  float* rcp;     /* [rows]: the epilogue's final reciprocal fl32(1 / (448 d)) of the row's
                     denominator after its last epoch (0 for a row without keys)              */
} sattn_checkpoints;

/*
 * sattn_debug_scores — the checkpoints of the Phase 2B report's "Exactness" section
 * (INT32-to-FP32 QK scores, per-epoch m and d, E4M3 probability words, FP32 rescale
 * values, the running output) for sampled query rows of one (segment, head).  It runs the
 * forward kernel's own instantiation (the same tiles, pipeline and K-scale path as
 * sattn_fwd / sattn_fwd_varlen for this problem) with stores of the checkpoint
 * quantities added, for the query tiles that hold sampled rows only.
 *
 *   dense  (cu_seqlens_q == cu_seqlens_k == NULL): nseg segments of Lq queries and Lk keys.
 *   varlen (both non-NULL): the device arrays given to sattn_quantize_qkv; Lq and Lk are
 *          the packed query and key tokens the views held.
 *
 * Sampled rows: segment-relative query rows q_begin + i*q_step (i = 0, 1, ...) below both
 * q_end and the segment's length; buffer row i belongs to the i-th of them, so every
 * buffer needs ceil((q_end - q_begin) / q_step) rows.  `o` receives the forward output of
 * the sampled rows of head `head` (bit-identical to sattn_fwd's), and no other element.
 * Returns SATTN_EINVAL for seg/head out of range, q_begin < 0, q_end <= q_begin,
 * q_step < 1, a NULL `ck`, ld < 1 with acc or s given, or nep < 1 with a per-epoch buffer.
 */
SATTN_API sattn_status sattn_debug_scores(const sattn_qkv_quant* qkv, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, int nseg, int64_t Lq, int64_t Lk, int H, int D,
                                float sm_scale, int seg, int head, int64_t q_begin, int64_t q_end,
                                int64_t q_step, const sattn_checkpoints* ck, sattn_bf16_out o, void* stream);

/*
 * sattn_fwd_fused — the forward with the Q preparation fused into the attention launch
 * (the roadmap page's "Phase 4" items on fusing preparation and consuming the projection-
 * strided input): each workgroup reads its query rows straight from the BF16 view `q`
 * (same strides and alignment rules as sattn_quantize_qkv's views) and quantizes them in
 * registers with exactly the arithmetic of sattn_quantize_qkv's Q step (amax per 64-token
 * block, or per 32 rows when kv->q_scale_rows = 32; fl32 scale and reciprocal; RNE codes
 * in [-127, 127]), so the output equals sattn_quantize_qkv + sattn_fwd(_varlen) bit for
 * bit.  No INT8 Q is written.  kv holds K and V as written by sattn_quantize_qkv (its q
 * and q_scale are not read and may be NULL).
 *
 *   dense  (cu_seqlens_q == cu_seqlens_k == NULL): nseg segments of Lq queries and Lk
 *          keys; q and o are [nseg, Lq, H, D] views; workspace may be NULL, or (16-byte
 *          aligned, fwd_workspace_bytes) enables the key split of small grids exactly as
 *          in sattn_fwd (same rule, same results, same zero-counter contract).
 *   varlen (both non-NULL): the cu_seqlens arrays given to sattn_quantize_qkv; Lq is the
 *          number of packed query tokens the q and o views hold, Lk the packed key
 *          tokens; workspace: fwd_workspace_bytes (16-byte aligned), scratch.
 *
 * Errors as sattn_fwd / sattn_fwd_varlen; SATTN_ENOSPACE if kv->kblk_cap cannot hold the
 * key blocks or workspace_bytes is too small.
 */
SATTN_API sattn_status sattn_fwd_fused(const sattn_qkv_quant* kv, sattn_bf16_in q, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k, int nseg, int H, int64_t Lq, int64_t Lk, int D,
                             float sm_scale, sattn_bf16_out o, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * sattn_quantize_qkv_noalloc — sattn_quantize_qkv for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops that allocate nothing, harnesses
 * that forbid hipMalloc): the same arguments minus the workspace, the same results bit for
 * bit.  Its workspace is a device array inside the library of sattn_noalloc_scratch_bytes()
 * bytes (16 MiB), one per GPU, held until the process ends; the call makes no allocation.
 * It uses the array of the device current on the calling thread, which must be the device
 * of `stream` and of every buffer.  Returns SATTN_ENOSPACE when the problem's workspace
 * (quant_workspace_bytes of sattn_quant_query) exceeds the array (beyond about 8,000
 * segment-heads), SATTN_EUNSUPPORTED for a device index of 64 or more, and otherwise what
 * sattn_quantize_qkv returns.  Every call on one GPU uses that GPU's one array: calls that
 * overlap in time on one GPU (on different streams, or from different threads without
 * ordering) race and give undefined results.  The array holds only intermediate sums that
 * each call writes before it reads them, so no clearing is needed between calls.
 */
SATTN_API sattn_status sattn_quantize_qkv_noalloc(sattn_bf16_in q, sattn_bf16_in k, sattn_bf16_in v, int nseg, int H,
                                        int D, int64_t Lq, int64_t Lk, const int32_t* cu_seqlens_q,
                                        const int32_t* cu_seqlens_k, const sattn_qkv_quant* out, void* stream);

/* Size in bytes of the per-device workspace array of sattn_quantize_qkv_noalloc. */
SATTN_API size_t sattn_noalloc_scratch_bytes(void);

/* Static, human-readable name of a status code. */
SATTN_API const char* sattn_status_string(sattn_status s);

#ifdef __cplusplus
}
#endif

#endif /* SATTN_H_ */
