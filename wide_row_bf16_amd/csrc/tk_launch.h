// Internal launch interface between the C ABI (tk_api.cpp) and the kernels
// (tk_kernels.hip).  Not part of the public header.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace tk {

// One scan workgroup per (row, span).  Rows [row0, row0 + rows_in_launch) of
// the matrix are covered by rows_in_launch * spans workgroups.  With spans == 1
// the scan writes the final outputs; otherwise it writes one sorted candidate
// list per (row, span) into the span arrays, for the merge dispatch or, with
// row_done set, for the row's last workgroup to fold (fused merge: spans <=
// kMergeGroup, rows_in_launch <= kFusedMaxRows).
struct ScanArgs {
  const uint16_t *in;
  int64_t row0;
  int64_t cols;
  int64_t stride;
  int32_t k;
  int32_t spans;
  int32_t exact;        // 1: never use a speculative floor
  int32_t spec_rank;    // rank (1-based) of the speculative floor in the pooled sample; 0: none
  int32_t *out_idx;
  uint16_t *out_val;
  int32_t *out_count;
  uint32_t *out_nonfinite;
  uint64_t *span_list;  // [rows][spans][k] composite (key << 32 | ~col), descending
  int32_t *span_count;  // [rows][spans]
  uint32_t *span_flags; // [rows][spans]
  int32_t *row_done;    // non-NULL: fused merge; per-row arrival counters, zero between calls
  int64_t col_base;     // added to every output column index (a shard's first global column)
  uint32_t inf;         // +inf bit pattern of the input format: 0x7F80 bf16, 0x7C00 fp16
};

// k = 1 (argmax) scan, one workgroup per (row, span) as ScanArgs.  With
// spans == 1 it writes the outputs; with 2 <= spans <= kMergeGroup each
// workgroup writes its span's best composite (key << 32 | ~col, flags in bits
// 48..50) to span_slot and the row's last workgroup (row_done, as ScanArgs)
// writes the outputs.
struct ArgmaxArgs {
  const uint16_t *in;
  int64_t row0;
  int64_t cols;
  int64_t stride;
  int32_t spans;
  uint32_t inf;         // +inf bit pattern of the input format
  int64_t col_base;     // added to the output column index
  uint64_t *span_slot;  // [rows_in_launch][spans]
  int32_t *row_done;    // per-row arrival counters, zero between calls
  int32_t *out_idx;
  uint16_t *out_val;
  int32_t *out_count;
  uint32_t *out_nonfinite;
};

hipError_t launch_argmax(const ArgmaxArgs &a, int64_t rows_in_launch, hipStream_t stream);

// Fused draft head (tk_head.hip): one workgroup per span; span s covers the
// vocabulary's 16-column tiles [ntiles * s / spans, ntiles * (s + 1) / spans)
// with ntiles = ceil(vocab / 16), at most kHeadSpanCols / 16 of them (the
// host's choice of spans guarantees it); each writes, for
// every row, the span's top k as signed composites (key << 32 |
// (0x7FFFFFFF - column) << 1 | sign) into span_list [rows][spans][k] with
// counts and flags [rows][spans], for span_merge_kernel (in == NULL) to fold.
// logits: NULL, or [rows][logits_stride] bf16 to receive the logits as well.
struct HeadArgs {
  int64_t rows;
  int64_t hidden;
  int64_t vocab;
  int32_t k;
  int32_t spans;
  const uint16_t *h;
  int64_t h_stride;
  const uint16_t *w;
  int64_t w_stride;
  uint64_t *span_list;
  int32_t *span_count;
  uint32_t *span_flags;
  uint16_t *logits;
  int64_t logits_stride;
  // NULL, or [rows][k] key slots, zero at the call's start: a workgroup puts
  // its span's best key of row r (an entry of its list) into slot (span mod
  // k) with an atomic max, and one that finds all k slots of a row filled
  // keeps only keys >= their minimum (k listed entries reach it).  Used with
  // one row tile (rows <= 16); the last merge level sets the slots to zero.
  uint32_t *sketch;
};

hipError_t launch_head_scan(const HeadArgs &a, hipStream_t stream);

// One merge workgroup per (row, group of up to kMergeGroup input lists).
// With in == NULL the lists hold signed composites (see HeadArgs) and the
// outputs are decoded from them alone.
// With lists_out == 1 the merge writes the final outputs.
struct MergeArgs {
  const uint16_t *in;  // the input matrix: entry values are read back from it
  int64_t row0;
  int64_t stride;
  int32_t k;
  int32_t lists_in;    // lists per row on input
  int32_t lists_out;   // lists per row on output = ceil(lists_in / group)
  int32_t group;       // input lists folded by one workgroup
  const uint64_t *list_in;
  const int32_t *count_in;
  const uint32_t *flags_in;
  uint64_t *list_out;
  int32_t *count_out;
  uint32_t *flags_out;
  int32_t *out_idx;
  uint16_t *out_val;
  int32_t *out_count;
  uint32_t *out_nonfinite;
  int64_t col_base;    // added to every output column index
  uint32_t *sketch;    // lists_out == 1: [rows][k] words set to zero after the row is written (or NULL)
};

// Merge of per-shard top-k results: shard g's outputs for all rows are the
// dense blocks idx/val [g][rows][k], count/mask [g][rows].
struct ShardMergeArgs {
  int64_t rows;
  int32_t shards;
  int32_t k;
  const int32_t *idx_in;
  const uint16_t *val_in;
  const int32_t *count_in;
  const uint32_t *mask_in;
  int32_t *out_idx;
  uint16_t *out_val;
  int32_t *out_count;
  uint32_t *out_nonfinite;
};

hipError_t launch_shard_merge(const ShardMergeArgs &a, hipStream_t stream);

// Seeded top-p sampling over top-k results [rows][k] (tk_sample.hip).
struct SampleArgs {
  int64_t rows;
  int32_t k;
  const int32_t *idx;
  const uint16_t *val;
  const int32_t *count;
  int32_t greedy;      // temperature == 0
  float scale;         // float32(log2(e) / temperature)
  float top_p;
  float coef[8];       // (ln 2)^i / i! rounded to float32
  uint32_t key0, key1; // seed, low and high words
  uint32_t off0, off1; // offset, low and high words
  int32_t *out_token;
  int32_t *out_kept;
};

hipError_t launch_sample(const SampleArgs &a, hipStream_t stream);

hipError_t launch_span_scan(const ScanArgs &a, int64_t rows_in_launch, hipStream_t stream);

// 64 < k <= 256 (tk_wide.hip): ScanArgs as for launch_span_scan, with every
// split row (2 <= spans <= kMergeGroup) folded by its last workgroup
// (row_done, span_list [rows][spans][k], span_count, span_flags required then).
hipError_t launch_wide_scan(const ScanArgs &a, int64_t rows_in_launch, hipStream_t stream);

// The fp32 scan (tk_f32.hip): as ScanArgs with 32-bit inputs and entry
// values; split rows (2 <= spans <= kMergeGroup) are always folded by their
// last workgroup (row_done required then).
struct ScanArgs32 {
  const uint32_t *in;
  int64_t row0;
  int64_t cols;
  int64_t stride;
  int32_t k;
  int32_t spans;
  int32_t exact;
  int32_t spec_rank;
  int32_t *out_idx;
  uint32_t *out_val;
  int32_t *out_count;
  uint32_t *out_nonfinite;
  uint64_t *span_list;
  int32_t *span_count;
  uint32_t *span_flags;
  int32_t *row_done;
};

hipError_t launch_span_scan32(const ScanArgs32 &a, int64_t rows_in_launch, hipStream_t stream);

// k = 1 on fp32 rows (tk_f32.hip), as ArgmaxArgs with 32-bit inputs and
// values; split rows keep a composite (key << 32 | ~column) and a flags word
// per span.
struct ArgmaxArgs32 {
  const uint32_t *in;
  int64_t row0;
  int64_t cols;
  int64_t stride;
  int32_t spans;
  uint64_t *span_slot;  // [rows_in_launch][spans]
  uint32_t *span_flag;  // [rows_in_launch][spans]
  int32_t *row_done;
  int32_t *out_idx;
  uint32_t *out_val;
  int32_t *out_count;
  uint32_t *out_nonfinite;
};

hipError_t launch_argmax32(const ArgmaxArgs32 &a, int64_t rows_in_launch, hipStream_t stream);

// 64 < k <= 256 on fp32 rows (tk_f32.hip): ScanArgs32 as for
// launch_span_scan32 (split rows folded by their last workgroup).
hipError_t launch_wide_scan32(const ScanArgs32 &a, int64_t rows_in_launch, hipStream_t stream);
hipError_t launch_span_merge(const MergeArgs &a, int64_t rows_in_launch, hipStream_t stream);
hipError_t launch_zero_fill(int32_t *p, int64_t n, hipStream_t stream);
// Device address of the current device's fixed scratch array
// (kFixedScratchBytes, 256-byte aligned; its first kFusedMaxRows int32 are
// zero between calls), set up on the first request for `dev`, which must be
// the current device.
hipError_t fixed_scratch(int dev, hipStream_t stream, void **ptr);
// Measurement probe: nvec 16-byte vectors read with the scan's loads over
// `workgroups` workgroups of four waves (nvec = 0: an empty kernel).
hipError_t launch_read_probe(const void *in, int64_t nvec, int32_t workgroups, uint32_t *sink, hipStream_t stream);

}  // namespace tk
