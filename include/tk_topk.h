/*
 * tk_topk.h -- exact row-wise top-k over wide bf16 rows on AMD Instinct MI355X.
 *
 * The operation (TensorFold PR #713 "the drafter's attention and top-k use
 * more of the GPU", change 3 and its Exactness table): for every row of a
 * rows x cols matrix of bf16 logits, return the k best entries -- score
 * descending, and among equal scores the lower column (token) index first --
 * together with the row's entry count and a non-finite mask.  Results must be
 * identical byte for byte across every way the work is split (the page
 * compares its span path with a single-group control) and to a CPU oracle,
 * over ties, both zeros, NaN, infinities and padded strides.
 *
 * Value policy (plain readings where the page is silent):
 *   NaN   -- any sign or payload; never an entry; sets TK_NONFINITE_NAN.
 *   +inf  -- ranked as the largest value; sets TK_NONFINITE_POSINF.
 *   -inf  -- ranked as the smallest value; sets TK_NONFINITE_NEGINF.
 *   +0/-0 -- compare equal (the lower column wins); each entry keeps its own
 *            bit pattern, so a -0 entry is 0x8000.
 *   subnormals are ordered by exact value (nothing is flushed).
 *
 * Layouts (all device memory, owned by the caller):
 *   in             rows x row_stride bf16 bit patterns, row-major, row_stride
 *                  in ELEMENTS; only columns [0, cols) of each row are read,
 *                  the padding [cols, row_stride) is never touched.
 *   out_idx        int32  [rows][k]  column of entry j (0 <= j < count), else -1
 *   out_val        uint16 [rows][k]  bf16 bits of in[r][out_idx], else 0x7FC0
 *   out_count      int32  [rows]     min(k, number of non-NaN columns of the row)
 *   out_nonfinite  uint32 [rows]     OR of TK_NONFINITE_* over the row's columns
 *
 * Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream): outputs are valid once the stream passes the call.  The library
 * keeps no pointer after the call returns; the caller keeps the buffers alive
 * until the stream has passed the call.  Calls on different streams may run
 * concurrently.  Temporary span lists are stream-ordered allocations of the
 * library (hipMallocAsync / hipFreeAsync on `stream`), kept per stream between
 * calls; calls that overlap on one stream cannot happen (the stream orders
 * them), and the buffer's per-row merge counters return to zero at the end of
 * every call.
 *
 * k up to 64 keeps one wavefront lane per entry; 64 < k <= TK_MAX_K (256)
 * runs a scan whose per-wave kept list spans two or four registers (every
 * input format; the pages give the library a compile-time max_k, and this is
 * its extension).  The shard merge, sampling and the fused head take k <=
 * TK_MAX_K_LANE (64).
 *
 * Errors: the guards below run on the host before any device work; on a
 * guard error nothing is launched and nothing is written.  TK_ERR_DEVICE
 * reports a failed allocation or launch; an asynchronous fault surfaces at the
 * caller's next synchronisation (HIP convention).
 */
#ifndef TK_TOPK_H
#define TK_TOPK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TK_MAX_K 256u     /* largest k of the row top-k (bf16, fp16, fp32; _ex and _shard forms) */
#define TK_MAX_K_LANE 64u /* largest k of the shard merge, sampling and the fused head: one lane per entry */

#define TK_NONFINITE_NAN 1u    /* the row has at least one NaN (none is an entry)  */
#define TK_NONFINITE_POSINF 2u /* the row has at least one +inf                    */
#define TK_NONFINITE_NEGINF 4u /* the row has at least one -inf                    */

#define TK_FILL_IDX (-1)      /* out_idx of an unused entry slot */
#define TK_FILL_VAL 0x7FC0u   /* out_val of an unused entry slot (a quiet NaN) */

typedef enum tk_status {
  TK_OK = 0,
  TK_ERR_NULL = 1,   /* a required pointer is NULL: with rows > 0 every output, and `in` when cols > 0 */
  TK_ERR_SHAPE = 2,  /* rows < 0, cols < 0, cols > INT32_MAX, row_stride < cols, or sizes overflow */
  TK_ERR_K = 3,      /* k < 1 or k above the entry point's limit (TK_MAX_K or TK_MAX_K_LANE) */
  TK_ERR_ALIGN = 4,  /* in/out_val not 2-byte aligned, or out_idx/out_count/out_nonfinite not 4-byte aligned */
  TK_ERR_ALIAS = 5,  /* two of the five buffers overlap (outputs must not alias the input or each other) */
  TK_ERR_DEVICE = 6, /* HIP reported an error while allocating or launching */
  TK_ERR_OPTION = 7, /* tk_options out of range */
  TK_ERR_SCRATCH = 8 /* tk_topk_bf16_noalloc: one row needs more scratch than its fixed array holds */
} tk_status;

/*
 * Row-wise exact top-k (see the file comment for the contract): the wide-row
 * top-k of TensorFold PR #713, change 3 (entries in score-then-lower-token
 * order), with the outputs its Exactness table compares (entries, counts,
 * non-finite masks).
 *   rows        >= 0; rows == 0 returns TK_OK without touching the device.
 *   cols        0 <= cols <= INT32_MAX; cols == 0 gives count 0 and all fills.
 *   row_stride  >= cols, in elements.
 *   k           1 <= k <= TK_MAX_K; k may exceed cols.
 *   stream      hipStream_t the work is queued on.
 */
tk_status tk_topk_bf16(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                       int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                       void *stream);

/*
 * tk_topk_bf16 without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc.  Same arguments, results, guards and errors as
 * tk_topk_bf16; the scratch it needs (the span lists and arrival counters of
 * split rows) lives in one fixed device array per GPU of
 * TK_NOALLOC_SCRATCH_BYTES, set up on the first call on that GPU (with it
 * current) and held until the process ends.  No hipMalloc, hipFree or
 * allocating library call is made, ever.  Split rows are processed in row
 * batches small enough for the array; a call whose single row needs more
 * scratch than the array holds (only rows of over a billion columns) returns
 * TK_ERR_SCRATCH before any launch.  Every call on a GPU shares that GPU's
 * array: calls that overlap in time on one GPU (on different streams, or
 * from different threads) race and must be ordered by the caller; calls on
 * one stream are ordered by the stream.  The array's arrival counters are
 * zero before and after every call.
 */
#define TK_NOALLOC_SCRATCH_BYTES (2u << 20)

tk_status tk_topk_bf16_noalloc(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                               int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                               void *stream);

/*
 * Planning overrides, for tests and benchmarks.  The result never depends on
 * them: every plan computes the same bytes.  TensorFold PR #713, change 3:
 * its benchmark dispatches the single-group kernel directly as the control
 * of the span path (spans = 1 here), and its Exactness table requires the
 * span path's entries, counts and masks to equal that control's byte for
 * byte (any spans here).
 *   spans  0 = automatic; 1 = one workgroup scans each whole row (the
 *          single-group control); n > 1 = split each row into n spans whose
 *          candidate lists are merged in the same order: by the row's last
 *          scan workgroup for n <= 64, by merge dispatches above.  Rejected with
 *          TK_ERR_OPTION when a span would exceed the library's span limit
 *          (tk_max_span_cols()) or n > cols (for cols > 0), and for k > 64
 *          when n > 64 (k > 64 splits a row into at most 64 spans, so rows
 *          wider than 64 x tk_max_span_cols() give TK_ERR_SHAPE there).
 *          The automatic plan splits k > 64 rows into at most 12 spans.
 *   exact  0 = automatic; 1 = never take the speculative floor (wide spans
 *          otherwise skip elements below a floor estimated from a sample and
 *          verify it afterwards, scanning again when it does not hold).
 *   general  0 = automatic; 1 = k == 1 runs the general top-k scan instead of
 *          the argmax scan (the control of that fast path), for every input
 *          format.  Automatically k == 1 takes the argmax scan when rows are
 *          fewer than the GPU's CUs or spans is forced, else the general scan.  With k == 1 the argmax scan takes spans (forced or
 *          planned) up to 64; above that (bf16 / fp16 only) the general scan
 *          runs.
 *   Values other than 0 and 1 for exact and general give TK_ERR_OPTION.
 */
typedef struct tk_options {
  int32_t spans;
  int32_t exact;
  int32_t general;
  int32_t reserved[5]; /* must be zero */
} tk_options;

tk_status tk_topk_bf16_ex(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                          int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                          void *stream, const tk_options *opt);

/*
 * IEEE binary16 (fp16) rows: the same operation, layouts, outputs, guards
 * and options as tk_topk_bf16 / tk_topk_bf16_ex, with `in` holding fp16 bit
 * patterns (+inf 0x7C00, -inf 0xFC00, NaN any magnitude above 0x7C00).  The
 * pages' rows are bf16; fp16 logits are an extension on the same row ABI.
 * out_val holds the fp16 bits of the entries; empty slots hold 0x7FC0 (an
 * fp16 NaN pattern too).  tk_validate_bf16 gives the guards of both.
 */
tk_status tk_topk_f16(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                      int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite, void *stream);
tk_status tk_topk_f16_ex(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                         int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                         void *stream, const tk_options *opt);

/*
 * IEEE binary32 (fp32) rows: the same operation, outputs and rules with
 * 32-bit inputs and entry values.  in: uint32 fp32 bit patterns, 4-byte
 * aligned, row_stride in elements; out_val: uint32 [rows][k], the entries'
 * own bits, empty slots 0x7FC00000.  Keys are 32 bits wide and composites 64,
 * so one span may be any width; tk_options.spans accepts 0..64
 * (TK_ERR_OPTION above).  1 <= k <= TK_MAX_K (TK_ERR_K above).
 * tk_validate_f32 gives the guards alone.
 */
tk_status tk_topk_f32(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint32_t *in,
                      int32_t *out_idx, uint32_t *out_val, int32_t *out_count, uint32_t *out_nonfinite, void *stream);
tk_status tk_topk_f32_ex(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint32_t *in,
                         int32_t *out_idx, uint32_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                         void *stream, const tk_options *opt);
tk_status tk_validate_f32(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint32_t *in,
                          const int32_t *out_idx, const uint32_t *out_val, const int32_t *out_count,
                          const uint32_t *out_nonfinite);

/*
 * The host-side guards alone (no HIP call is made): returns the status
 * tk_topk_bf16 would return before launching anything.  TensorFold PR #713,
 * Exactness table, the row of the GPU top-k bench: the row ABI and its guards
 * are checked beside the exact cases; this entry point lets a host test run
 * every guard without a device.  Arguments as tk_topk_bf16 (no stream); the
 * pointers are only compared, never dereferenced.
 */
tk_status tk_validate_bf16(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                           const int32_t *out_idx, const uint16_t *out_val, const int32_t *out_count,
                           const uint32_t *out_nonfinite);

/*
 * The span count the automatic plan picks for a shape on a GPU with
 * `compute_units` CUs (host-only arithmetic; no HIP call).  For k == 1 that
 * is the plan of the argmax scan, for k > 64 that of the multi-register scan,
 * for 2 <= k <= 32 on few rows one of 8 to 12 spans by the row's width (bf16
 * and fp16 rows).
 */
int32_t tk_plan_spans(int64_t rows, int64_t cols, int32_t k, int32_t compute_units);

/*
 * Vocabulary-sharded top-k.  The split of a wide row into spans whose
 * candidate lists are merged in the same (score desc, lower index first) order
 * (TensorFold PR #713, change 3) carried across devices: each device holds a
 * column shard of every row, finds the shard's top k, and one merge over the
 * gathered shard results gives the row's top k.  (The pages run one rank; the
 * cross-device use is this library's plain reading of the span split.)
 *
 * tk_topk_bf16_shard: tk_topk_bf16 on a shard whose column 0 is the row's
 * global column col_base; out_idx holds global indices (col_base + local).
 * Requires col_base >= 0 and col_base + cols - 1 <= INT32_MAX
 * (TK_ERR_SHAPE otherwise); all else as tk_topk_bf16.
 */
tk_status tk_topk_bf16_shard(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, int64_t col_base,
                             const uint16_t *in, int32_t *out_idx, uint16_t *out_val, int32_t *out_count,
                             uint32_t *out_nonfinite, void *stream);

#define TK_MAX_SHARDS 4096

/*
 * tk_merge_topk_bf16: the top k of each row over `shards` shard results, in
 * the same order.  Inputs are the shards' outputs stacked shard-major, the
 * layout an all-gather of dense per-shard blocks produces (all device
 * memory):
 *   idx_in, val_in     [shards][rows][k]   entries as tk_topk_bf16_shard wrote
 *                                          them (global indices, bf16 bits)
 *   count_in, mask_in  [shards][rows]      per-shard counts and non-finite masks
 * Outputs as tk_topk_bf16: count = min(k, sum of the shard counts), mask = OR
 * of the shard masks, entries in order, fill after count.  Every shard must
 * have used this k, 1 <= k <= TK_MAX_K_LANE (else TK_ERR_K).
 * 1 <= shards <= TK_MAX_SHARDS (else TK_ERR_SHAPE).
 * Guards as tk_topk_bf16 (NULL, alignment, outputs overlapping each other or
 * an input -> TK_ERR_ALIAS); entries are trusted as written by
 * tk_topk_bf16_shard (no memory is addressed through them).  Asynchronous on
 * `stream`; no scratch memory.
 */
tk_status tk_merge_topk_bf16(int64_t rows, int32_t shards, int32_t k, const int32_t *idx_in, const uint16_t *val_in,
                             const int32_t *count_in, const uint32_t *mask_in, int32_t *out_idx, uint16_t *out_val,
                             int32_t *out_count, uint32_t *out_nonfinite, void *stream);

/* The host-side guards of tk_merge_topk_bf16 alone (no HIP call). */
tk_status tk_validate_merge_bf16(int64_t rows, int32_t shards, int32_t k, const int32_t *idx_in,
                                 const uint16_t *val_in, const int32_t *count_in, const uint32_t *mask_in,
                                 const int32_t *out_idx, const uint16_t *out_val, const int32_t *out_count,
                                 const uint32_t *out_nonfinite);

/*
 * Seeded top-p sampling over the top-k entries of each row: the step a
 * sampled drafted decode takes after top-k (the pages name its parameters,
 * temperature, top-k, top-p and seed, in the receipt of TensorFold PR #3069
 * "qwen27 metal: restore the long-copy driver for a lone greedy stream on
 * M5", and require seeded sampled decodes to repeat token for token, in the
 * seeded sampled exactness cases of the review of PR #713).  The pages give
 * no algorithm; this is the library's reading, in float32 throughout, with
 * every operation a single IEEE float32 operation in the order given:
 *   inputs per row: idx/val/count as tk_topk_bf16 writes them ([rows][k],
 *   [rows], device memory), entries in order.
 *   - count <= 0: token -1, kept 0.  temperature == 0: greedy, token = idx[0].
 *   - x_j = the bf16 value val[j] as float32 (exact).  If x_0 is +inf, the
 *     weight w_j is 1 for x_j == +inf and 0 otherwise; else w_j = 0 for
 *     x_j == -inf and w_j = exp2(float32(float32(x_j - x_0) * s)) with
 *     s = float32(log2(e) / temperature) formed in double, and exp2 =
 *     n = rint(t), f = t - n, 2^f by the degree-7 Taylor polynomial
 *     (coefficients (ln 2)^i / i! as float32, Horner), times 2^n; 0 when
 *     n < -125.
 *   - c_0 = 0, c_{j+1} = c_j + w_j (float32, in entry order); Z = c_count.
 *   - kept = the smallest n >= 1 with c_n >= float32(top_p * Z).
 *   - u = (r >> 8) * 2^-24 with r the first word of Philox4x32-10 (Salmon,
 *     Moraes, Dror and Shaw, SC 2011), key (seed low word, seed high word),
 *     counter (row, 0, offset low word, offset high word); h =
 *     float32(u * c_kept).
 *   - token = idx[j] for the smallest j < kept with c_{j+1} > h, else
 *     idx[kept - 1].
 * Outputs: out_token, out_kept int32 [rows].  `offset` is the decode step:
 * the same (seed, offset, row) always draws the same u.  Guards: 1 <= k <=
 * TK_MAX_K_LANE (TK_ERR_K), 0 <= temperature finite and 0 < top_p <= 1
 * (TK_ERR_OPTION), NULL, alignment, outputs overlapping each other or an
 * input (TK_ERR_ALIAS).  Asynchronous on `stream`; no scratch memory.
 */
tk_status tk_sample_topk_bf16(int64_t rows, int32_t k, const int32_t *idx, const uint16_t *val, const int32_t *count,
                              float temperature, float top_p, uint64_t seed, uint64_t offset, int32_t *out_token,
                              int32_t *out_kept, void *stream);

/* The host-side guards of tk_sample_topk_bf16 alone (no HIP call). */
tk_status tk_validate_sample_bf16(int64_t rows, int32_t k, const int32_t *idx, const uint16_t *val,
                                  const int32_t *count, float temperature, float top_p, const int32_t *out_token,
                                  const int32_t *out_kept);

/*
 * Draft-head logits fused with the row top-k.  The drafter of TensorFold PR
 * #713 computes its draft head and takes the top k of each of its rows (15
 * rows of 98592 columns in change 3); this call does both in one pass over
 * the head's weights, so the logits are never written to memory.  The pages
 * give no kernel for the head; the library's reading:
 *   logits[r][n] = bf16_rne( sum_i h[r][i] * w[n][i] )
 * with the products and their sum in float32 on the matrix cores (the
 * summation order is the hardware's; the result is within float32
 * accumulation error of the exact sum before the bf16 rounding to nearest,
 * ties to even; NaN inputs give NaN logits), and then exactly the top-k of
 * tk_topk_bf16 over those logits (order, NaN, infinities, flags, fills).
 *   h      bf16 [rows][h_stride], 16-byte aligned, h_stride % 8 == 0
 *   w      bf16 [vocab][w_stride] (vocabulary-major, as a linear layer's
 *          weight), 16-byte aligned, w_stride % 8 == 0
 *   out_*  as tk_topk_bf16 ([rows][k] entries with vocabulary indices,
 *          [rows] counts and masks)
 *   logits NULL, or bf16 [rows][logits_stride] (logits_stride >= vocab,
 *          2-byte aligned) that also receives the logits -- for tests; the
 *          top-k does not depend on it.
 * Guards: 0 <= rows <= TK_HEAD_MAX_ROWS, 32 <= hidden <= 65536 with hidden %
 * 32 == 0, 1 <= vocab <= INT32_MAX, hidden <= h_stride, w_stride <= 2^21
 * (TK_ERR_SHAPE); 1 <= k <= TK_MAX_K_LANE (TK_ERR_K); NULL (logits may be
 * NULL), alignment, and outputs overlapping each other or an input
 * (TK_ERR_ALIAS).  Asynchronous on `stream`; scratch as tk_topk_bf16.
 */
#define TK_HEAD_MAX_ROWS 64

tk_status tk_head_topk_bf16(int64_t rows, int64_t hidden, int64_t vocab, int32_t k, const uint16_t *h,
                            int64_t h_stride, const uint16_t *w, int64_t w_stride, int32_t *out_idx,
                            uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite, uint16_t *logits,
                            int64_t logits_stride, void *stream);

/* The host-side guards of tk_head_topk_bf16 alone (no HIP call). */
tk_status tk_validate_head_bf16(int64_t rows, int64_t hidden, int64_t vocab, int32_t k, const uint16_t *h,
                                int64_t h_stride, const uint16_t *w, int64_t w_stride, const int32_t *out_idx,
                                const uint16_t *out_val, const int32_t *out_count, const uint32_t *out_nonfinite,
                                const uint16_t *logits, int64_t logits_stride);

/*
 * Releases the scratch the library keeps for `stream` on the current device
 * (the span lists of split rows, cached per stream between calls) with a
 * stream-ordered free that follows the work already queued on `stream`, and
 * forgets the stream.  Call it before destroying a stream that ran top-k
 * calls with split rows: a stream created later may reuse the handle value,
 * and would otherwise share the cached buffer (and its arrival counters)
 * with work still pending from the destroyed one.  A stream the library has
 * no scratch for returns TK_OK at once; a later call on the stream simply
 * allocates again.  TK_ERR_DEVICE if HIP fails.  (The library's own: the
 * pages keep one draft stream per drafter and say nothing of stream
 * lifetimes.)
 */
tk_status tk_release_stream(void *stream);

/*
 * Measurement probe, beside the top-k rather than part of it.  TensorFold PR
 * #713, change 3 measures its span path against a control dispatch in a
 * bench of its own; here the control of a scan's time is the bare read of
 * the same bytes: `bytes` (a multiple of 16) of device memory at `in`
 * (16-byte aligned) are streamed by `workgroups` workgroups of four waves
 * with exactly the loads of the top-k scan (four nontemporal 16-byte vectors
 * per lane per chunk, two chunks in flight) and nothing is computed from
 * them.  `sink` (device, uint32 [8192], 4-byte aligned) is written only if
 * the bytes' XOR fold hits a fixed sentinel (it keeps the loads from being
 * dropped).  bytes == 0 launches an empty kernel of `workgroups` workgroups
 * (in may be NULL): the launch floor of that grid.
 * Errors: TK_ERR_SHAPE (bytes < 0 or not a multiple of 16, workgroups < 1
 * or > 2^24, a wave's share of 2^26 vectors or more), TK_ERR_NULL,
 * TK_ERR_ALIGN, TK_ERR_ALIAS (sink inside the read range), TK_ERR_DEVICE.
 * Asynchronous on `stream`; no scratch memory.
 */
tk_status tk_probe_read(const void *in, int64_t bytes, int32_t workgroups, uint32_t *sink, void *stream);

/*
 * tk_max_k: TK_MAX_K, the largest k of the row top-k as built.  TensorFold PR
 * #713, change 3 ties the kernel's lane, span and max_k constants to the
 * calling side at compile time, so that a mismatch breaks the build; here the
 * kernels' constants are static_asserted against this header's and the
 * calling side reads the built value from the library (tk_max_span_cols
 * likewise gives the widest span one workgroup scans).
 */
int32_t tk_max_k(void);
int64_t tk_max_span_cols(void);     /* widest span one workgroup scans */
const char *tk_status_string(tk_status s);
const char *tk_build_info(void);    /* target and build flags of the library */

#ifdef __cplusplus
}
#endif

#endif /* TK_TOPK_H */
