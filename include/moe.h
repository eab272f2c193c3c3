/*
 * grouped_expert_amd: single-GPU MoE routed-expert layer for AMD Instinct
 * MI355X (gfx950).  C ABI.
 *
 * The layer (pages cited by title and section):
 *   route    "M6.6 - MoE Runtime Systems", 0x03A router-side tensors;
 *            "M6.2 - Expert Parallelism and DeepSeek MoE", 0x06L1 family
 *            table, Mixtral row (FP32 softmax, top-k, renormalise to one).
 *   permute  M6.2 0x03B count / exclusive prefix / stable permutation and
 *            inverse; M6.2 0x01C capacity; M6.6 0x0CD route assertions.
 *   experts  M6.6 0x04A bias-free SwiGLU expert; 0x04C variable grouped GEMM
 *            over ragged expert segments.
 *   combine  M6.6 0x03C3 inverse permutation and weighted scatter-add over
 *            the semantic key; 0x0AE FP32 gate and FP32 token accumulation.
 *   pack     "Fixed pooled-wave all-to-all for the 8-of-384 MoE", 02-04:
 *            destination pools per wave, stripe rule, header row of local
 *            expert ids, sender capacity.
 *   compact  pooled wave 02-04 and 07: receiver groups rows into static
 *            per-expert arrays in fixed source order, drops above capacity.
 *
 * Conventions for every call
 *   - Pointers named as device buffers are device pointers (HBM).  Sizes and
 *     flags are host values.  Index arrays are int32.  bf16 data is raw
 *     16-bit storage (the upper half of the binary32 pattern), i.e. the
 *     layout of torch.bfloat16.  All tensors are dense row-major.
 *   - Ownership: the caller allocates and owns every buffer, including the
 *     workspaces sized by the *_workspace queries.  The library never
 *     allocates or frees memory and keeps no pointer after a call returns
 *     (apart from the kernels it has enqueued).  It holds no mutable global
 *     state.
 *   - Synchrony: a call only enqueues kernels on `stream` and returns; no
 *     call synchronises with the host.  Counts, offsets and drop totals are
 *     written to device memory.  Buffers may be read once the stream has
 *     reached the call's work.
 *   - Errors: argument violations the host can see (null pointer, bad size,
 *     unsupported shape, misalignment, workspace too small) return a
 *     negative moe_status before anything is enqueued, and nothing is
 *     written.  A failed kernel launch returns MOE_EHIP.  Violations that
 *     live in device data never abort: the offending route or row is treated
 *     as dropped and a bit is OR-ed into *dev_flags (when dev_flags is not
 *     NULL).  The library never clears dev_flags; the caller zeroes it.
 *   - Device-pointer arguments must be 16-byte aligned unless stated.
 */
#ifndef GROUPED_EXPERT_AMD_MOE_H
#define GROUPED_EXPERT_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* bad argument */
  MOE_EUNSUPPORTED = -2,  /* valid but not supported by this build (shape / dtype) */
  MOE_EWORKSPACE = -3,    /* workspace missing or smaller than the query returns */
  MOE_EHIP = -4,          /* a HIP runtime call or kernel launch failed */
  MOE_ESCRATCH = -5       /* larger than the static scratch of moe_permute_noalloc */
} moe_status;

/* Row storage.  MOE_FP8_ROW / MOE_FP8_B128 are fp8 dispatch records
 * ("M6.2 - Expert Parallelism and DeepSeek MoE", 0x0AB-0x0AC: fp8 data plus
 * fp32 scales that travel with their row): d OCP E4M3 codes (bias 7, 3
 * mantissa bits, max 448, 0x7F NaN, no infinity), then G fp32 scales (G = 1,
 * or ceil(d / 128) for one scale per 128 values), then zero bytes up to a
 * multiple of 128, whole cache lines (moe_row_bytes).  Value i of a record is
 * decode(code_i) * scale[i / group width]. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_ROW = 2, MOE_FP8_B128 = 3 } moe_dtype;

/* Gating families ("M6.2 - Expert Parallelism and DeepSeek MoE").
 *   SOFTMAX_TOPK_RENORM   0x06L1, Mixtral row: FP32 softmax over all experts,
 *                         keep the top k, renormalise the kept probabilities.
 *   SOFTMAX_TOPK          0x04D, 0x06L3 (V1): same selection, the selected
 *                         full-softmax probabilities are kept as they are.
 *   SOFTMAX_GROUP_LIMITED 0x05A-0x05B (V2): group-limited greedy on the
 *                         softmax, no renormalisation, times a route scale.
 *   SIGMOID_BIAS_GROUP_TOP2  0x06A-0x06D, 0x06I (V3): sigmoid affinity plus a
 *                         selection bias picks groups by their two largest
 *                         corrected scores, then experts; gates are the
 *                         selected original affinities renormalised, times a
 *                         route scale.
 * The first two are served by moe_route_topk, the last two by
 * moe_route_topk_grouped. */
typedef enum {
  MOE_GATING_SOFTMAX_TOPK_RENORM = 0,
  MOE_GATING_SOFTMAX_TOPK = 1,
  MOE_GATING_SOFTMAX_GROUP_LIMITED = 2,
  MOE_GATING_SIGMOID_BIAS_GROUP_TOP2 = 3
} moe_gating;

/* Bits OR-ed into *dev_flags. */
#define MOE_FLAG_BAD_EXPERT      1u  /* expert id < -1 or >= E (route dropped) */
#define MOE_FLAG_NONFINITE_LOGIT 2u  /* token with a NaN/Inf logit (all slots id -1) */
#define MOE_FLAG_BAD_HEADER      4u  /* header id neither < n_local nor 0xFFFF (row ignored) */
#define MOE_FLAG_BAD_INDEX       8u  /* combine index < -1 or expand slot out of range (ignored) */
#define MOE_FLAG_BAD_SEGMENT    16u  /* expert segment outside [0, rows) (expert skipped) */
#define MOE_FLAG_NONFINITE_INPUT 32u  /* NaN/Inf in a quantized group (group stored as zeros) */

/* Limits of this build. */
#define MOE_MAX_EXPERTS 1024   /* E, n_dest, n_local */
#define MOE_MAX_TOPK    16

/* Bytes of one row of d values stored as dtype (fp8 records: d code bytes,
 * the fp32 scales, zero bytes up to a multiple of 128, a whole number of
 * cache lines); 0 for an unknown dtype or d < 1. */
size_t moe_row_bytes(int32_t dtype, int32_t d);

/* Pool geometry of the pooled-wave pack and the receiver's compaction
 * ("Fixed pooled-wave all-to-all for the 8-of-384 MoE", 02-05: a pool is one
 * packed full-width header row of local expert ids followed by its data
 * rows).  With RB = moe_row_bytes(row_dtype, d), a pool of pool_rows data
 * rows has H = max(1, ceil(2 * pool_rows / RB)) header rows (one 16-bit id
 * per data row) and is PH = pool_rows + H rows tall.
 *   moe_pool_geometry        writes H and PH for pool_rows >= 0.
 *   moe_pool_rows_of_height  writes the data-row count of a pool PH rows tall
 *                            (the inverse); MOE_EINVAL if no count fits.
 * row_dtype MOE_BF16 or an fp8 record dtype, d >= 8 and d % 8 == 0; output
 * pointers are host pointers.  Host-only: nothing is launched.  Returns
 * MOE_OK or MOE_EINVAL. */
int moe_pool_geometry(int32_t row_dtype, int32_t d, int64_t pool_rows, int64_t* header_rows, int64_t* pool_height);
int moe_pool_rows_of_height(int32_t row_dtype, int32_t d, int64_t pool_height, int64_t* pool_rows);

/* ---------------------------------------------------------------------------
 * moe_quantize_fp8 -- rows to fp8 dispatch records.
 *
 * "M6.2 - Expert Parallelism and DeepSeek MoE", 0x0AB-0x0AC: quantization
 * yields fp8 data and its fp32 scales, owned by the same row.  For every
 * scale group of row t (the row, or 128 consecutive values; the pages fix no
 * scale rule, this is the library's): a = largest |x| of the group,
 *   scale = a / 448, inv = 448 / a   (each one correctly rounded fp32 op)
 *   code_i = E4M3(x_i * inv)         (fp32 product; nearest, ties to even,
 *                                     saturating at +-448, sign kept)
 * A group with a = 0 stores scale 0 and zero codes; a group holding NaN or
 * Inf stores the same and sets MOE_FLAG_NONFINITE_INPUT.
 *
 *   x          device [n, d] of x_dtype (MOE_BF16 or MOE_F32); d % 8 == 0
 *   rec_dtype  MOE_FP8_ROW or MOE_FP8_B128
 *   rec        device [n, moe_row_bytes(rec_dtype, d)] bytes, 16-byte aligned
 * ------------------------------------------------------------------------- */
int moe_quantize_fp8(const void* x, int32_t x_dtype, int64_t n, int32_t d, int32_t rec_dtype, void* rec,
                     uint32_t* dev_flags, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_dequantize_fp8 -- fp8 dispatch records back to rows.
 *
 * out[t][i] = decode(code_i) * scale[group of i] (fp32 product), stored as
 * out_dtype (bf16: nearest even) -- the scale read from the same record
 * (M6.2 0x0AC).
 *
 *   rec        device records [n, moe_row_bytes(rec_dtype, d)]; d % 8 == 0
 *   out        device [n, d] of out_dtype (MOE_BF16 or MOE_F32)
 * ------------------------------------------------------------------------- */
int moe_dequantize_fp8(const void* rec, int32_t rec_dtype, int64_t n, int32_t d, void* out, int32_t out_dtype,
                       uint32_t* dev_flags, hipStream_t stream);

/* Human-readable name of a moe_status value.  Never NULL. */
const char* moe_strerror(int status);

/* ABI version of this library (major * 100 + minor). */
int moe_version(void);

/* ---------------------------------------------------------------------------
 * moe_route_topk -- router top-k with renormalised softmax gates.
 *
 * For every token t (M6.6 0x03A; M6.2 0x06L1 Mixtral row):
 *   topk_ids[t, j]  j-th largest logit's expert, j = 0..k-1, ordered by
 *                   descending fp32 logit; equal logits (-0 == +0) place the
 *                   lower expert index first.
 *   topk_w[t, j]    MOE_GATING_SOFTMAX_TOPK_RENORM: exp(z_j - z_0) /
 *                   sum over the k kept experts of exp(z_i - z_0) (= softmax
 *                   over all E, keep k, renormalise);
 *                   MOE_GATING_SOFTMAX_TOPK (V1): exp(z_j - z_0) / sum over
 *                   all E experts of exp(z_i - z_0) (the kept softmax mass).
 * A token whose logits contain NaN or +-Inf gets ids -1 and weights 0 in all
 * k slots and sets MOE_FLAG_NONFINITE_LOGIT.
 *
 *   logits    device, fp32 [T, E]
 *   T >= 0; 1 <= k <= min(E, MOE_MAX_TOPK); 1 <= E <= MOE_MAX_EXPERTS
 *   gating    MOE_GATING_SOFTMAX_TOPK_RENORM or MOE_GATING_SOFTMAX_TOPK
 *             (others: MOE_EUNSUPPORTED)
 *   topk_ids  device, int32 [T, k]       (4-byte alignment suffices)
 *   topk_w    device, fp32  [T, k]       (4-byte alignment suffices)
 *   dev_flags device uint32 or NULL
 * ------------------------------------------------------------------------- */
int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t gating,
                   int32_t* topk_ids, float* topk_w, uint32_t* dev_flags, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_route_topk_grouped -- group-restricted router top-k (V2, V3).
 *
 * "M6.2 - Expert Parallelism and DeepSeek MoE", 0x05A-0x05B (V2) and
 * 0x06A-0x06D, 0x06I (V3).  Experts form n_group contiguous groups of
 * G = E / n_group ids.  For every token t:
 *   MOE_GATING_SOFTMAX_GROUP_LIMITED (V2): group score = largest logit in
 *     the group (softmax is monotone, so this ranks groups as their best
 *     probability does); keep topk_group groups; the k largest logits among
 *     the kept groups' experts, descending; topk_w = softmax probability over
 *     all E experts times route_scale (no renormalisation).  bias must be NULL.
 *   MOE_GATING_SIGMOID_BIAS_GROUP_TOP2 (V3): s_e = 1 / (1 + exp(-z_e))
 *     evaluated in fp64 and rounded once to fp32 (nearest even), and
 *     c_e = s_e + bias[e] in fp32 (bias NULL = 0); group score = sum of the
 *     group's two largest c; keep topk_group groups; the k largest c among the
 *     kept groups' experts, descending; topk_w = route_scale * s_j / sum over
 *     the k selected of s.
 * Groups and experts of equal score rank the lower index first.  A token
 * with a non-finite logit (or corrected score) gets ids -1, weights 0 and
 * sets MOE_FLAG_NONFINITE_LOGIT.
 *
 *   logits      device, fp32 [T, E]
 *   T >= 0; 1 <= E <= MOE_MAX_EXPERTS; 1 <= k <= MOE_MAX_TOPK
 *   n_group     1..64 dividing E; 1 <= topk_group <= n_group;
 *               k <= topk_group * E / n_group; V3 also needs E / n_group >= 2
 *   route_scale finite (V2: 16 in the released V2 checkpoint; V3: 2.5)
 *   bias        device, fp32 [E] or NULL (V3 only)
 *   topk_ids, topk_w, dev_flags as for moe_route_topk
 * Returns MOE_EINVAL for any violated bound, MOE_EUNSUPPORTED for another
 * gating value; nothing is launched then.
 * ------------------------------------------------------------------------- */
int moe_route_topk_grouped(const float* logits, int64_t T, int32_t E, int32_t k, int32_t gating,
                           int32_t n_group, int32_t topk_group, float route_scale, const float* bias,
                           int32_t* topk_ids, float* topk_w, uint32_t* dev_flags, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_permute -- group routes by expert, stable, with capacity and inverse.
 *
 * Routes are r = t*k + j (token-major, then slot).  With e_r = topk_ids[r]
 * (M6.2 0x03B, 0x01C; M6.6 0x0CD):
 *   sel[e]     = #{r : e_r = e}
 *   pos_r      = #{r' < r : e_r' = e_r}            (rank in route order)
 *   accepted   iff capacity < 0 (dropless) or pos_r < capacity
 *   counts[e]  = accepted routes of e = min(sel[e], capacity)
 *   offsets    exclusive prefix of counts, offsets[E] = A (accepted total)
 *   inv[r]     = offsets[e_r] + pos_r, or -1 if dropped
 *   src[p]     = r with inv[r] = p for p < A; -1 for A <= p < T*k
 *   x_perm[p]  = x[src[p] / k] for p < A (rows p >= A are not written); fp8
 *                records move whole, codes and scales together (M6.2 0x0AC)
 *   n_dropped  = T*k - A
 * Expert id -1 means "no route" (dropped, not flagged); ids < -1 or >= E
 * are dropped and set MOE_FLAG_BAD_EXPERT.
 *
 *   x          device, [T, d] of x_dtype; may be NULL when x_perm is NULL
 *   x_dtype    MOE_F32 (d % 4 == 0), MOE_BF16 (d % 8 == 0) or an fp8 record
 *              dtype (d % 8 == 0; rows of moe_row_bytes(x_dtype, d) bytes)
 *   topk_ids   device int32 [T*k]
 *   capacity   -1 (dropless) or >= 0
 *   x_perm     device [T*k, d] of x_dtype, or NULL (metadata only)
 *   src, inv   device int32 [T*k]
 *   sel_counts device int32 [E] or NULL; counts int32 [E]; offsets int32 [E+1]
 *   n_dropped  device int32 [1]
 *   ws         device workspace of at least moe_permute_workspace(T, k, E) bytes
 * ------------------------------------------------------------------------- */
size_t moe_permute_workspace(int64_t T, int32_t k, int32_t E);
int moe_permute(const void* x, int32_t x_dtype, int64_t T, int32_t d,
                const int32_t* topk_ids, int32_t k, int32_t E, int64_t capacity,
                void* x_perm, int32_t* src, int32_t* inv,
                int32_t* sel_counts, int32_t* counts, int32_t* offsets, int32_t* n_dropped,
                void* ws, size_t ws_bytes, uint32_t* dev_flags, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_permute_noalloc -- moe_permute that allocates nothing and takes no
 * workspace.
 *
 * For callers that cannot allocate device memory around the call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, semantics, outputs and errors as moe_permute, without ws /
 * ws_bytes.  The bucket-rank table lives in a static device array of
 * MOE_PERMUTE_NOALLOC_SCRATCH_BYTES bytes that each GPU the library runs on
 * holds until the process ends; a problem whose moe_permute_workspace(T, k,
 * E) exceeds it returns MOE_ESCRATCH before anything is enqueued.  The call
 * never calls hipMalloc / hipFree.  The array's device address is looked up
 * once per device (hipGetSymbolAddress, with the stream's device current)
 * on the first call there; MOE_EHIP if that fails.
 * Every call on one GPU uses that GPU's single array: calls whose work
 * overlaps in time on one GPU (different streams, or host threads without
 * ordering) race and give wrong results; calls ordered on one stream are
 * safe.  Nothing in the array needs to start at zero (every entry a call
 * reads was written earlier in the same call).
 * ------------------------------------------------------------------------- */
#define MOE_PERMUTE_NOALLOC_SCRATCH_BYTES (4u << 20)
int moe_permute_noalloc(const void* x, int32_t x_dtype, int64_t T, int32_t d,
                        const int32_t* topk_ids, int32_t k, int32_t E, int64_t capacity,
                        void* x_perm, int32_t* src, int32_t* inv, int32_t* sel_counts, int32_t* counts,
                        int32_t* offsets, int32_t* n_dropped, uint32_t* dev_flags, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_grouped_swiglu -- bias-free SwiGLU experts over ragged row segments.
 *
 * For every expert e with seg_count[e] > 0, rows
 * X_e = x[seg_start[e] .. seg_start[e] + seg_count[e]) (M6.6 0x04A, 0x04C):
 *   G = X_e W_gate[e]^T,  U = X_e W_up[e]^T            (fp32 accumulate)
 *   H = SiLU(G) * U,      SiLU(v) = v / (1 + exp(-v))  (fp32)
 *   z rows of the segment = H W_down[e]^T              (fp32 accumulate)
 * bf16 path: operands bf16 on MFMA, H rounded to bf16 (nearest-even) between
 * the two products, z stored as z_dtype (bf16 or fp32).  fp32 path: every
 * value fp32 (z_dtype must be MOE_F32).  Rows not covered by a segment are
 * not written.  A segment with start < 0, count < 0 or start + count > rows
 * sets MOE_FLAG_BAD_SEGMENT and is skipped; zero-row experts are skipped
 * without shifting later experts' weights.
 *
 *   x          device [rows, d] of dtype
 *   d % 64 == 0, d_ff % 64 == 0, 1 <= E
 *   seg_start, seg_count   device int32 [E] (e.g. offsets and counts of
 *              moe_permute, or e*cap and counts of moe_recv_compact)
 *   rows       rows of x (upper bound of every segment end): T*k for a
 *              permuted batch, n_local*cap for static arrays
 *   w_gate, w_up  device [E, d_ff, d] of dtype; w_down device [E, d, d_ff]
 *   z          device of z_dtype: [rows, d] without a row map, where row i of
 *              the result is z row i; [z_n_rows, d] with one
 *   z_rows     NULL, or device int32 [rows]: row i of the result is stored
 *              as z row z_rows[i], and not at all when z_rows[i] is outside
 *              [0, z_n_rows) (the values are not otherwise checked; two rows
 *              mapped to one z row race).  With moe_recv_compact's slot_row
 *              this writes the experts' outputs straight into pool-row order
 *              ("Fixed pooled-wave all-to-all for the 8-of-384 MoE", 03:
 *              the receiver returns results in the pools' layout), the rows
 *              that compaction rejected being zeroed by that call.
 *   z_n_rows   rows of z when z_rows is given (<= INT32_MAX; ignored otherwise)
 *   act        NULL, or (bf16 path only, 16-byte aligned) device bf16
 *              [3 * rows * d_ff] that receives, for every row of a segment,
 *              the activations the expert backward needs ("M6.2 - Expert
 *              Parallelism and DeepSeek MoE", 0x03D: saved forward state):
 *              plane 1, [rows, 2 d_ff]: G (columns [0, d_ff)) and U
 *              ([d_ff, 2 d_ff)) rounded to bf16; plane 2, [rows, d_ff] at
 *              element offset 2 * rows * d_ff: H as the down product reads
 *              it.  Rows outside every segment are not written.  Results and
 *              z are the same with or without act.
 *   ws         device workspace of moe_grouped_swiglu_workspace(rows, E, d_ff, dtype)
 * ------------------------------------------------------------------------- */
size_t moe_grouped_swiglu_workspace(int64_t rows, int32_t E, int32_t d_ff, int32_t dtype);
int moe_grouped_swiglu(const void* x, int32_t dtype, int32_t d, int32_t d_ff, int32_t E,
                       const int32_t* seg_start, const int32_t* seg_count, int64_t rows,
                       const void* w_gate, const void* w_up, const void* w_down,
                       void* z, int32_t z_dtype, const int32_t* z_rows, int64_t z_n_rows, void* act,
                       void* ws, size_t ws_bytes, uint32_t* dev_flags, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_unpermute_combine -- inverse permutation + gate-weighted FP32 combine.
 *
 * For every token t (M6.6 0x03C3, 0x0CD; 0x0AE FP32 accumulation):
 *   y[t] (=, or += when accumulate) sum over j = 0..k-1 in ascending order of
 *        g[t*k+j] * z[idx[t*k+j] - lo]   for every j with lo <= idx < hi
 * Other routes add nothing: idx == -1 (dropped) or idx outside the window
 * [lo, hi) (held by another window, e.g. another wave).  idx < -1 sets
 * MOE_FLAG_BAD_INDEX.  No renormalisation is applied.  With k = 1 and
 * gates = NULL this is the row expansion of a static-array result back to
 * pool-row order (zero rows where idx is -1).
 *
 *   z          device [hi - lo, d] of z_dtype (MOE_F32 or MOE_BF16)
 *   d % 4 == 0 (fp32) or d % 8 == 0 (bf16)
 *   idx        device int32 [T*k]
 *   0 <= lo <= hi
 *   gates      device fp32 [T*k], or NULL for weight 1 (4-byte alignment suffices)
 *   y          device fp32 [T, d]
 * ------------------------------------------------------------------------- */
int moe_unpermute_combine(const void* z, int32_t z_dtype, int32_t d,
                          const int32_t* idx, int64_t lo, int64_t hi,
                          const float* gates, int64_t T, int32_t k,
                          float* y, int32_t accumulate, uint32_t* dev_flags, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_combine_backward -- reverse of the combine (route and gate gradients).
 *
 * "M6.2 - Expert Parallelism and DeepSeek MoE", 0x03D: with upstream
 * gradient dy, route r = t*k + j with row p = idx[r] (0 <= p < rows) gets
 *   dz[p]     = gates[r] * dy[t]            (converted to dz_dtype, nearest even)
 *   dgates[r] = sum_i dy[t, i] * z[p, i]    (fp32 accumulation)
 * Routes with idx = -1 get dgates = 0 and write nothing; idx < -1 or >= rows
 * also sets MOE_FLAG_BAD_INDEX.  Rows of dz that no route points to are not
 * written.
 *
 *   dy         device fp32 [T, d]; d % 8 == 0
 *   z          device [rows, d] of z_dtype: the forward's expert outputs
 *   idx        device int32 [T*k] (moe_permute's inv); gates fp32 [T*k]
 *   dz         device [rows, d] of dz_dtype (MOE_F32 or MOE_BF16)
 *   dgates     device fp32 [T*k]
 * ------------------------------------------------------------------------- */
int moe_combine_backward(const float* dy, int64_t T, int32_t d, const void* z, int32_t z_dtype,
                         int64_t rows, const int32_t* idx, const float* gates, int32_t k,
                         void* dz, int32_t dz_dtype, float* dgates, uint32_t* dev_flags, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_grouped_swiglu_backward -- expert backward over ragged row segments.
 *
 * "M6.2 - Expert Parallelism and DeepSeek MoE", 0x03D (expert backward gives
 * route-input and parameter gradients; the segments are backward state),
 * through the SwiGLU of "M6.6 - MoE Runtime Systems", 0x04A.  For every
 * expert e with rows X_e = x[seg_start[e] .. + seg_count[e]) and route
 * gradients dZ_e (same rows of dz), with G, U, H recomputed from X_e, or
 * taken from the activations the forward saved (act):
 *   dH = dZ_e W_d[e],  dG = dH * U * SiLU'(G),  dU = dH * SiLU(G)
 *   dx rows   = dG W_g[e] + dU W_u[e]                 (dx_dtype)
 *   dw_down[e] = dZ_e^T H,  dw_gate[e] = dG^T X_e,  dw_up[e] = dU^T X_e   (fp32)
 * with SiLU'(v) = s (1 + v (1 - s)), s = 1 / (1 + exp(-v)).  bf16 operands
 * on MFMA with fp32 accumulation; dH, dG, dU and H are rounded to bf16
 * between the products.  Every expert's weight gradients are written (zero
 * for an expert without rows).  Segments as in moe_grouped_swiglu.
 *
 *   x, dz      device bf16 [rows, d]; d % 64 == 0, d_ff % 64 == 0
 *   w_gate, w_up  device bf16 [E, d_ff, d]; w_down device bf16 [E, d, d_ff]
 *   act        NULL (recompute G, U and H: W_gate and W_up are read twice),
 *              or moe_grouped_swiglu's saved activations of the same x and
 *              segments (bf16, 16-byte aligned; layout in moe_grouped_swiglu):
 *              dG, dU come from dH and the saved G, U (bf16), H from its
 *              plane, and each weight is read once
 *   dx         device [rows, d] of dx_dtype (rows outside every segment not written)
 *   dw_gate, dw_up  device fp32 [E, d_ff, d]; dw_down device fp32 [E, d, d_ff]
 *   ws         device workspace of moe_grouped_swiglu_backward_workspace(rows, E, d, d_ff)
 * ------------------------------------------------------------------------- */
size_t moe_grouped_swiglu_backward_workspace(int64_t rows, int32_t E, int32_t d, int32_t d_ff);
int moe_grouped_swiglu_backward(const void* x, int32_t d, int32_t d_ff, int32_t E,
                                const int32_t* seg_start, const int32_t* seg_count, int64_t rows,
                                const void* w_gate, const void* w_up, const void* w_down,
                                const void* dz, const void* act, void* dx, int32_t dx_dtype,
                                float* dw_gate, float* dw_up, float* dw_down,
                                void* ws, size_t ws_bytes, uint32_t* dev_flags, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expand_rows -- receiver expansion of static-array results to pool rows.
 *
 * "Fixed pooled-wave all-to-all for the 8-of-384 MoE", 03 (the receiver
 * expands its expert rows back to the pool layout for the reverse exchange);
 * "M6.6 - MoE Runtime Systems", 0x04B (padding and dropped rows never reach
 * the combine) and 0x0AE (the returned row is BF16).  For i in [0, n_rows):
 *   ret[i] = z[row_slot[i]]   converted to ret_dtype, if 0 <= row_slot[i] < n_slots
 *   ret[i] = 0                otherwise (header, empty, receiver-dropped rows)
 * f32 -> bf16 rounds to nearest even; bf16 -> f32 is exact; same dtype is a
 * copy.  row_slot < -1 or >= n_slots sets MOE_FLAG_BAD_INDEX (row zeroed).
 *
 *   z          device [n_slots, d] of z_dtype (MOE_F32 or MOE_BF16)
 *   d % 8 == 0
 *   row_slot   device int32 [n_rows] (e.g. moe_recv_compact's row_slot)
 *   ret        device [n_rows, d] of ret_dtype, every row written
 * ------------------------------------------------------------------------- */
int moe_expand_rows(const void* z, int32_t z_dtype, int32_t d, const int32_t* row_slot,
                    int64_t n_rows, int64_t n_slots, void* ret, int32_t ret_dtype,
                    uint32_t* dev_flags, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_pool_pack -- pooled-wave sender pack into fixed destination pools.
 *
 * Pool rows are RB = moe_row_bytes(pool_dtype, d) bytes: bf16 rows, or fp8
 * records (M6.2 0x0AB-0x0AC: the scales travel inside the row).  Rows are
 * moved as they are (pool_dtype == x_dtype) or bf16 rows are quantized into
 * records on the way (x_dtype bf16, pool_dtype fp8: every token row is
 * quantized once, exactly as moe_quantize_fp8 does, and its record written to
 * each placed slot).  A pool has
 * H = max(1, ceil(2 * pool_rows / RB)) full-width header rows (one for bf16
 * rows at the pages' sizes) followed by pool_rows data rows;
 * PH = pool_rows + H.  The header rows hold little-endian uint16 ids: id i
 * (bytes 2i, 2i+1 of the flattened header) is data row i's local id.
 *
 * For route r = t*k + j with valid expert e = topk_ids[r] (pooled wave 02-05):
 *   dest = e / experts_per_dest,  local = e % experts_per_dest
 *   o_r  = #{r' < r : dest_r' = dest_r}     (the route's destination rank)
 *   wave = o_r % n_waves,  row = o_r / n_waves,  accepted iff row < pool_rows
 *   pools[wave][dest][H + row][:] = x[t]
 *   header element row of pools[wave][dest] = local   (uint16)
 *   route_loc[r] = (wave*n_dest + dest)*PH + H + row, else -1
 * Every other header element is 0xFFFF and every data row without a route
 * is zero.  dest_counts[dest] = routes to dest before the cap;
 * sender_dropped = T*k - accepted (routes above the cap plus routes whose id
 * is -1 or invalid; invalid ids set MOE_FLAG_BAD_EXPERT).
 *
 *   x          device [T] rows of x_dtype (MOE_BF16, MOE_FP8_ROW, MOE_FP8_B128), d % 8 == 0
 *   pool_dtype x_dtype, or an fp8 record dtype when x_dtype is MOE_BF16
 *   E <= n_dest * experts_per_dest, n_dest <= MOE_MAX_EXPERTS, 1 <= n_waves
 *   wave       -1: pools is [n_waves][n_dest][PH] rows of RB bytes (all waves);
 *              w >= 0: pools is [n_dest][PH] rows, only wave w's rows and
 *              headers are written (route_loc keeps the all-wave index)
 *   route_loc  device int32 [T*k]; dest_counts int32 [n_dest]; sender_dropped int32 [1]
 *   ws         device workspace of moe_pool_pack_workspace(T, k, n_dest)
 * ------------------------------------------------------------------------- */
size_t moe_pool_pack_workspace(int64_t T, int32_t k, int32_t n_dest);
int moe_pool_pack(const void* x, int32_t x_dtype, int32_t pool_dtype, int64_t T, int32_t d,
                  const int32_t* topk_ids, int32_t k,
                  int32_t E, int32_t experts_per_dest, int32_t n_dest, int32_t n_waves,
                  int32_t pool_rows, int32_t wave, void* pools, int32_t* route_loc,
                  int32_t* dest_counts, int32_t* sender_dropped, void* ws, size_t ws_bytes,
                  uint32_t* dev_flags, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_recv_compact -- receiver compaction into static per-expert arrays.
 *
 * Pools have the layout of moe_pool_pack for rows of pool_dtype: H header
 * rows, then pool_rows data rows; PH = pool_rows + H.  Over one
 * wave's incoming pools, visiting sources s = (src_rotation + v) % n_src for
 * v = 0..n_src-1 (src_rotation = 0: the fixed source order of pooled wave
 * 07; another value is the per-receiver rotation proposed there), then
 * i = 0..pool_rows-1 (pooled wave 02-04, 07):
 *   h = header element i of source s (uint16); 0xFFFF = empty row
 *   q = number of earlier visited rows with the same h
 *   accepted iff q < cap:  compact[h][q][:] = pools_in[s][H + i][:]
 *                          (fp8 records: dequantized to bf16 as in
 *                          moe_dequantize_fp8, with the record's own scales)
 *   row_slot[s*PH + H + i] = h*cap + q, else -1
 *   row_slot of header rows and empty rows = -1
 *   arrived[h] = rows with id h, counts[h] = min(arrived[h], cap),
 *   recv_dropped = sum_h arrived[h] - counts[h]
 * Header ids >= n_local other than 0xFFFF set MOE_FLAG_BAD_HEADER and the
 * row is ignored.  compact rows at or past counts[h] are not written.
 * Optional outputs for a receiver that writes its results in pool-row order
 * (moe_grouped_swiglu with z_rows = slot_row) instead of expanding them:
 *   slot_row[j] = n  for every accepted row n = s*PH + H + i with
 *                    row_slot[n] = j (the inverse of row_slot; entries of
 *                    slots at or past counts[h] are not written)
 *   ret[n][:] = 0    for every row n with row_slot[n] == -1 (header, empty
 *                    and receiver-dropped rows); accepted rows not written
 *
 *   pools_in   device [n_src][PH] rows of pool_dtype (MOE_BF16, MOE_FP8_ROW,
 *              MOE_FP8_B128), d % 8 == 0
 *   1 <= n_local <= MOE_MAX_EXPERTS, cap >= 0, 0 <= src_rotation < max(n_src, 1)
 *   compact    device bf16 [n_local][cap][d]
 *   counts int32 [n_local]; arrived int32 [n_local] or NULL;
 *   row_slot int32 [n_src*PH]; recv_dropped int32 [1]
 *   slot_row   device int32 [n_local*cap], or NULL
 *   ret        device [n_src*PH][d] of ret_dtype (MOE_F32 or MOE_BF16), or NULL
 *              (ret_dtype then ignored)
 *   ws         device workspace of moe_recv_compact_workspace(n_src, pool_rows, n_local)
 * ------------------------------------------------------------------------- */
size_t moe_recv_compact_workspace(int32_t n_src, int32_t pool_rows, int32_t n_local);
int moe_recv_compact(const void* pools_in, int32_t pool_dtype, int32_t n_src, int32_t pool_rows, int32_t d,
                     int32_t n_local, int32_t cap, int32_t src_rotation, void* compact, int32_t* counts,
                     int32_t* arrived, int32_t* row_slot, int32_t* recv_dropped,
                     int32_t* slot_row, void* ret, int32_t ret_dtype,
                     void* ws, size_t ws_bytes, uint32_t* dev_flags, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GROUPED_EXPERT_AMD_MOE_H */
