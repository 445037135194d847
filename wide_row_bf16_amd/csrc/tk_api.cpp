// C ABI of the wide-row bf16 top-k library: host guards, span planning,
// stream-ordered scratch and kernel launches.  Contract: include/tk_topk.h.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <atomic>
#include <cmath>
#include <limits>
#include <mutex>

#include "tk_config.h"
#include "tk_launch.h"

#ifndef TK_BUILD_INFO
#define TK_BUILD_INFO "unknown build"
#endif

namespace {

using tk::kMaxK;
using tk::kMaxKWide;
using tk::kMaxSpanVecs;
using tk::kMergeGroup;
using tk::kFusedMaxRows;
using tk::kVecElems;
using tk::kSampleElems;
using tk::kSpecFailure;

constexpr int64_t kMaxBlocksPerLaunch = int64_t(1) << 24;  // keeps grid work-items below 2^32
constexpr int64_t kMinSpanCols = 4096;                      // a split never makes spans narrower
// Automatic plans use at most 12 spans per row (unless the span width limit
// needs more): the row's last workgroup folds the span lists in a chain of
// about S / 4 + 3 merges, and on few-row inputs 8-12 spans measured fastest
// (15 x 98592: 13.8 us at 8-12 spans, 15.6 us at 18; 16 x 248320: 17.6 us at
// 12, 18.0 us at 16).
constexpr int32_t kMaxAutoSpans = 12;
constexpr int32_t kMaxSpans = 1 << 16;

struct Range {
  uintptr_t lo, hi;  // [lo, hi), empty when lo == hi
};

bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool mul_ok(int64_t a, int64_t b, int64_t limit) { return a == 0 || b <= limit / a; }

tk_status guard(int64_t rows, int64_t cols, int64_t stride, int32_t k, const void *in, const void *out_idx,
                const void *out_val, const void *out_count, const void *out_nonfinite, int eb = 2,
                int32_t kmax = kMaxKWide) {
  if (rows < 0 || cols < 0 || cols > INT32_MAX || stride < cols) return TK_ERR_SHAPE;
  if (k < 1 || k > kmax) return TK_ERR_K;
  // k > 64 splits a row into at most kMergeGroup spans of kMaxSpanVecs vectors
  if (k > kMaxK && (cols / kVecElems + kMaxSpanVecs - 1) / kMaxSpanVecs > kMergeGroup) return TK_ERR_SHAPE;
  if (rows == 0) return TK_OK;
  if ((cols > 0 && !in) || !out_idx || !out_val || !out_count || !out_nonfinite) return TK_ERR_NULL;
  const int64_t big = std::numeric_limits<int64_t>::max() / 8;
  if (!mul_ok(rows - 1, stride, big) || (rows - 1) * stride > big - cols) return TK_ERR_SHAPE;
  if (!mul_ok(rows, k, big)) return TK_ERR_SHAPE;
  if (((uintptr_t)in & (uintptr_t)(eb - 1)) || ((uintptr_t)out_val & (uintptr_t)(eb - 1))) return TK_ERR_ALIGN;
  if (((uintptr_t)out_idx & 3) || ((uintptr_t)out_count & 3) || ((uintptr_t)out_nonfinite & 3)) return TK_ERR_ALIGN;
  const int64_t in_elems = cols > 0 ? (rows - 1) * stride + cols : 0;
  const Range rs[5] = {
      {(uintptr_t)in, (uintptr_t)in + (uintptr_t)(eb * in_elems)},
      {(uintptr_t)out_idx, (uintptr_t)out_idx + (uintptr_t)(4 * rows * k)},
      {(uintptr_t)out_val, (uintptr_t)out_val + (uintptr_t)(eb * rows * k)},
      {(uintptr_t)out_count, (uintptr_t)out_count + (uintptr_t)(4 * rows)},
      {(uintptr_t)out_nonfinite, (uintptr_t)out_nonfinite + (uintptr_t)(4 * rows)},
  };
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (overlap(rs[i], rs[j])) return TK_ERR_ALIAS;
  return TK_OK;
}

// Guards of the shard merge: inputs [shards][rows][k] entries and
// [shards][rows] counts and masks, outputs as tk_topk_bf16.
tk_status guard_merge(int64_t rows, int32_t shards, int32_t k, const void *idx_in, const void *val_in,
                      const void *count_in, const void *mask_in, const void *out_idx, const void *out_val,
                      const void *out_count, const void *out_nonfinite) {
  if (rows < 0 || shards < 1 || shards > TK_MAX_SHARDS) return TK_ERR_SHAPE;
  if (k < 1 || k > kMaxK) return TK_ERR_K;
  if (rows == 0) return TK_OK;
  if (!idx_in || !val_in || !count_in || !mask_in || !out_idx || !out_val || !out_count || !out_nonfinite)
    return TK_ERR_NULL;
  const int64_t big = std::numeric_limits<int64_t>::max() / 8;
  if (!mul_ok(rows, (int64_t)shards * k, big) || rows > (int64_t)UINT32_MAX) return TK_ERR_SHAPE;
  if (((uintptr_t)val_in & 1) || ((uintptr_t)out_val & 1)) return TK_ERR_ALIGN;
  if (((uintptr_t)idx_in & 3) || ((uintptr_t)count_in & 3) || ((uintptr_t)mask_in & 3) || ((uintptr_t)out_idx & 3) ||
      ((uintptr_t)out_count & 3) || ((uintptr_t)out_nonfinite & 3))
    return TK_ERR_ALIGN;
  const int64_t n_in = rows * shards;
  const Range rs[8] = {
      {(uintptr_t)idx_in, (uintptr_t)idx_in + (uintptr_t)(4 * n_in * k)},
      {(uintptr_t)val_in, (uintptr_t)val_in + (uintptr_t)(2 * n_in * k)},
      {(uintptr_t)count_in, (uintptr_t)count_in + (uintptr_t)(4 * n_in)},
      {(uintptr_t)mask_in, (uintptr_t)mask_in + (uintptr_t)(4 * n_in)},
      {(uintptr_t)out_idx, (uintptr_t)out_idx + (uintptr_t)(4 * rows * k)},
      {(uintptr_t)out_val, (uintptr_t)out_val + (uintptr_t)(2 * rows * k)},
      {(uintptr_t)out_count, (uintptr_t)out_count + (uintptr_t)(4 * rows)},
      {(uintptr_t)out_nonfinite, (uintptr_t)out_nonfinite + (uintptr_t)(4 * rows)},
  };
  // outputs must overlap neither each other nor any input (inputs may share memory)
  for (int i = 4; i < 8; ++i)
    for (int j = 0; j < 8; ++j)
      if (j != i && overlap(rs[i], rs[j])) return TK_ERR_ALIAS;
  return TK_OK;
}

// Guards of the fused head: shapes, strides and limits that keep every
// buffer offset of a workgroup within 32 bits, alignment of the 16-byte
// fragment loads, and no output overlapping another or an input.
constexpr int64_t kHeadMaxHidden = 65536;
constexpr int64_t kHeadMaxStride = int64_t(1) << 21;

tk_status guard_head(int64_t rows, int64_t hidden, int64_t vocab, int32_t k, const void *h, int64_t h_stride,
                     const void *w, int64_t w_stride, const void *out_idx, const void *out_val, const void *out_count,
                     const void *out_nonfinite, const void *logits, int64_t logits_stride) {
  if (rows < 0 || rows > TK_HEAD_MAX_ROWS) return TK_ERR_SHAPE;
  if (hidden < 32 || hidden > kHeadMaxHidden || hidden % 32 != 0) return TK_ERR_SHAPE;
  if (vocab < 1 || vocab > INT32_MAX) return TK_ERR_SHAPE;
  if (h_stride < hidden || w_stride < hidden || h_stride % 8 != 0 || w_stride % 8 != 0) return TK_ERR_SHAPE;
  if (h_stride > kHeadMaxStride || w_stride > kHeadMaxStride) return TK_ERR_SHAPE;
  // logits rows are addressed as r * logits_stride + column in 64 bits
  if (logits && (logits_stride < vocab || logits_stride > (std::numeric_limits<int64_t>::max() / 8 - vocab) / 64))
    return TK_ERR_SHAPE;
  if (k < 1 || k > kMaxK) return TK_ERR_K;
  if (rows == 0) return TK_OK;
  if (!h || !w || !out_idx || !out_val || !out_count || !out_nonfinite) return TK_ERR_NULL;
  if (((uintptr_t)h & 15) || ((uintptr_t)w & 15)) return TK_ERR_ALIGN;
  if (((uintptr_t)out_val & 1) || ((uintptr_t)logits & 1)) return TK_ERR_ALIGN;
  if (((uintptr_t)out_idx & 3) || ((uintptr_t)out_count & 3) || ((uintptr_t)out_nonfinite & 3)) return TK_ERR_ALIGN;
  const Range rs[7] = {
      {(uintptr_t)h, (uintptr_t)h + (uintptr_t)(2 * ((rows - 1) * h_stride + hidden))},
      {(uintptr_t)w, (uintptr_t)w + (uintptr_t)(2 * ((vocab - 1) * w_stride + hidden))},
      {(uintptr_t)out_idx, (uintptr_t)out_idx + (uintptr_t)(4 * rows * k)},
      {(uintptr_t)out_val, (uintptr_t)out_val + (uintptr_t)(2 * rows * k)},
      {(uintptr_t)out_count, (uintptr_t)out_count + (uintptr_t)(4 * rows)},
      {(uintptr_t)out_nonfinite, (uintptr_t)out_nonfinite + (uintptr_t)(4 * rows)},
      {(uintptr_t)logits, logits ? (uintptr_t)logits + (uintptr_t)(2 * ((rows - 1) * logits_stride + vocab))
                                 : (uintptr_t)logits},
  };
  for (int i = 2; i < 7; ++i)
    for (int j = 0; j < 7; ++j)
      if (j != i && overlap(rs[i], rs[j])) return TK_ERR_ALIAS;
  return TK_OK;
}

// Guards of the sampling call: inputs [rows][k] entries and [rows] counts.
tk_status guard_sample(int64_t rows, int32_t k, const void *idx, const void *val, const void *count, float temperature,
                       float top_p, const void *out_token, const void *out_kept) {
  if (rows < 0 || rows > (int64_t)UINT32_MAX) return TK_ERR_SHAPE;
  if (k < 1 || k > kMaxK) return TK_ERR_K;
  if (!(temperature >= 0.0f) || temperature > 3.0e38f) return TK_ERR_OPTION;  // also NaN, inf
  if (!(top_p > 0.0f) || top_p > 1.0f) return TK_ERR_OPTION;
  if (rows == 0) return TK_OK;
  if (!idx || !val || !count || !out_token || !out_kept) return TK_ERR_NULL;
  if (!mul_ok(rows, k, std::numeric_limits<int64_t>::max() / 8)) return TK_ERR_SHAPE;
  if (((uintptr_t)val & 1) || ((uintptr_t)idx & 3) || ((uintptr_t)count & 3) || ((uintptr_t)out_token & 3) ||
      ((uintptr_t)out_kept & 3))
    return TK_ERR_ALIGN;
  const Range rs[5] = {
      {(uintptr_t)idx, (uintptr_t)idx + (uintptr_t)(4 * rows * k)},
      {(uintptr_t)val, (uintptr_t)val + (uintptr_t)(2 * rows * k)},
      {(uintptr_t)count, (uintptr_t)count + (uintptr_t)(4 * rows)},
      {(uintptr_t)out_token, (uintptr_t)out_token + (uintptr_t)(4 * rows)},
      {(uintptr_t)out_kept, (uintptr_t)out_kept + (uintptr_t)(4 * rows)},
  };
  for (int i = 3; i < 5; ++i)
    for (int j = 0; j < 5; ++j)
      if (j != i && overlap(rs[i], rs[j])) return TK_ERR_ALIAS;
  return TK_OK;
}

// Smallest span count that keeps every span within one workgroup's limit.
int64_t min_spans(int64_t cols) {
  const int64_t nv = cols / kVecElems;
  const int64_t s = (nv + kMaxSpanVecs - 1) / kMaxSpanVecs;
  return s < 1 ? 1 : s;
}

int32_t plan(int64_t rows, int64_t cols, int32_t compute_units) {
  if (cols <= 0 || rows <= 0) return 1;
  const int64_t need = min_spans(cols);
  int64_t s = 1;
  if (rows < compute_units) {
    // Few rows: split each row so that rows * spans covers every CU once,
    // without making spans narrower than kMinSpanCols.
    s = (compute_units + rows - 1) / rows;
    const int64_t by_width = cols / kMinSpanCols;
    if (s > by_width) s = by_width;
    if (s > kMaxAutoSpans) s = kMaxAutoSpans;
  }
  if (s < need) s = need;
  if (s < 1) s = 1;
  return (int32_t)s;
}

// The 16-bit scan with k <= 32 on few rows: spans aimed at about
// kNarrowSpanCols columns (a wave's share of about one and a half chunks),
// but no fewer than kMinNarrowSpans.  Below 12 spans the row's fold chains
// fewer merges, and at these k the longer shares cost less than that saves;
// at k = 64 a wave's exact path is longer and 12 spans stay faster.  Measured
// per call, forced span counts in alternated rounds on one box: 15 x 98592,
// k = 32: 13.07 us at 8 spans against 13.43 at 12; 15 x 49152 and
// 15 x 65536: 11.1 and 11.2 us at 8 against 11.9 and 12.2 at 12;
// 15 x 151936 and 16 x 248320 keep 12 (14.05 and 17.3 us; 8 spans 14.6 and
// 18.3); 15 x 98592 at k = 64: 13.8 us at 12 against 14.1 at 8.
constexpr int64_t kNarrowSpanCols = 12288;
constexpr int64_t kMinNarrowSpans = 8;
constexpr int32_t kNarrowMaxK = 32;
// Where the CU count asks for at most kDoubleMaxSpans spans (a third of the
// CU count of rows or more, but fewer rows than CUs), the scans take twice
// that many: two or more workgroups per CU, so one workgroup's fixed
// chain (first load, floors, merges, fold) runs while another streams.
// Measured per call, alternated rounds on one box (N(0, 2) rows): 96 x 98592
// 16.6 us at 6 spans against 19.4 at 3; 128 x 98592 17.6 against 21.5;
// 128 x 151936 at k = 64 23.4 against 30.3; 192 x 98592 19.3 against 22.8;
// 224 x 98592 20.9 against 23.1.  At 64 rows (4 spans) doubling gained on
// such rows but lost 0.4 us on rows of mixed ties and non-finite values.
// The k > 64 and fp32 scans gain the same way: 128 x 98592 at k = 128
// 24.6 us at 4 spans against 26.9 at 2 (fp32: 29.0 against 37.3);
// 192 x 151936 at k = 256 36.8 against 42.8.
constexpr int64_t kDoubleMaxSpans = 3;

int32_t doubled(int64_t rows, int64_t cols, int32_t spans, int32_t compute_units) {
  int64_t s = spans;
  if (rows < compute_units && s > 1 && s <= kDoubleMaxSpans) {
    const int64_t by_width = cols / kMinSpanCols;
    s = 2 * s <= by_width ? 2 * s : (by_width > s ? by_width : s);
  }
  return (int32_t)s;
}

// On so few rows that 12 spans fill under a quarter of the CUs (1 to 5 rows
// on 256 CUs), the 16-bit scan takes up to kTinyMaxSpans: the fold's one
// extra merge costs less than the shorter shares save.  Measured per call,
// alternated rounds on one box (N(0, 2) rows), 16 spans against the plan of
// 8 or 12: 1 x 151936 k = 32 12.75 against 13.15 us; 2 x 151936 k = 64 13.71
// against 14.18; 3 x 98592 k = 32 12.11 against 12.31; 4 x 248320 k = 20
// 14.09 against 14.89; 5 x 98592 12.13 against 12.44; 1 x 98592 k = 8 10.99
// against 11.11 (20 spans: faster still on the wider rows, slower on 98592
// columns).
constexpr int64_t kTinyMaxSpans = 16;

int32_t plan_scan16(int64_t rows, int64_t cols, int32_t k, int32_t compute_units) {
  if (rows > 0 && cols > 0 && rows * kMaxAutoSpans * 4 < compute_units) {
    int64_t t = (compute_units + rows - 1) / rows;
    const int64_t by_width = cols / kMinSpanCols;
    if (t > by_width) t = by_width;
    if (t > kTinyMaxSpans) t = kTinyMaxSpans;
    const int64_t need = min_spans(cols);
    if (t < need) t = need;
    return (int32_t)(t < 1 ? 1 : t);
  }
  int64_t s = doubled(rows, cols, plan(rows, cols, compute_units), compute_units);
  if (k <= kNarrowMaxK && s > kMinNarrowSpans) {
    int64_t t = cols / kNarrowSpanCols;
    if (t < kMinNarrowSpans) t = kMinNarrowSpans;
    if (s > t) s = t;
    const int64_t need = min_spans(cols);
    if (s < need) s = need;
  }
  return (int32_t)s;
}

// Rank j of the speculative floor in a workgroup's pooled sample (the first
// chunk of each wave).  The floor T is the sample's j-th largest lane
// maximum, at most its j-th largest element; it fails (fewer than k keys of
// the span reach it) only if j sample elements lie among the span's k - 1
// largest.  That count is about Poisson with mean k * sample / span, so j is
// the smallest rank whose tail probability is at most kSpecFailure.  Returns
// 0 when no rank below k qualifies (the exact floor, rank k, is then as good).
int32_t spec_rank(int32_t k, int64_t span_cols, int64_t sample = kSampleElems) {
  if (span_cols <= 0) return 0;
  const double lambda = (double)k * (double)sample / (double)span_cols;
  double p = std::exp(-lambda), cdf = p;  // P(X = 0), P(X <= 0)
  for (int32_t j = 1; j < k; ++j) {
    if (1.0 - cdf <= kSpecFailure) return j;  // P(X >= j)
    p *= lambda / j;
    cdf += p;
  }
  return 0;
}

std::atomic<int32_t> g_cu_count[64];
std::atomic<bool> g_pool_ready[64];

int32_t device_cus(int dev) {
  if (dev < 0 || dev >= 64) return 256;
  int32_t v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Keep stream-ordered allocations in the device's default pool between calls.
void keep_pool(int dev) {
  if (dev < 0 || dev >= 64 || g_pool_ready[dev].load(std::memory_order_acquire)) return;
  hipMemPool_t pool;
  if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
    uint64_t threshold = std::numeric_limits<uint64_t>::max();
    (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &threshold);
  }
  g_pool_ready[dev].store(true, std::memory_order_release);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Span lists need device scratch.  Each (device, stream) keeps one buffer
// between calls so that a call makes no allocation once warm; a buffer grows
// stream-ordered (hipFreeAsync of the old one, hipMallocAsync of the new one,
// both on that stream, so work already queued there still sees the old one).
// Calls on one stream are ordered by the stream itself; the mutex orders the
// host side from lookup to the last launch.  Requests above kCacheMaxBytes,
// or beyond kCacheStreams distinct streams, allocate and free per call.
constexpr size_t kCacheMaxBytes = size_t(64) << 20;
constexpr int kCacheStreams = 64;

struct ScratchSlot {
  int dev;
  hipStream_t stream;
  void *ptr;
  size_t cap;
};

std::mutex g_scratch_mu;
ScratchSlot g_scratch[kCacheStreams];
int g_scratch_used = 0;

// With g_scratch_mu held: a cached buffer of at least `bytes` for (dev,
// stream), or nullptr when the request is not cached (the caller allocates).
// *fresh tells that the buffer was just allocated (its contents are
// undefined).
void *cached_scratch(int dev, hipStream_t stream, size_t bytes, tk_status *st, bool *fresh) {
  *st = TK_OK;
  *fresh = false;
  if (bytes > kCacheMaxBytes) return nullptr;
  ScratchSlot *slot = nullptr;
  for (int i = 0; i < g_scratch_used; ++i)
    if (g_scratch[i].dev == dev && g_scratch[i].stream == stream) slot = &g_scratch[i];
  if (!slot) {
    if (g_scratch_used == kCacheStreams) return nullptr;
    slot = &g_scratch[g_scratch_used++];
    *slot = ScratchSlot{dev, stream, nullptr, 0};
  }
  if (slot->cap < bytes) {
    size_t cap = slot->cap * 2 > bytes ? slot->cap * 2 : bytes;
    if (cap > kCacheMaxBytes) cap = kCacheMaxBytes < bytes ? bytes : kCacheMaxBytes;
    if (slot->ptr && hipFreeAsync(slot->ptr, stream) != hipSuccess) *st = TK_ERR_DEVICE;
    slot->ptr = nullptr;
    slot->cap = 0;
    if (*st == TK_OK && hipMallocAsync(&slot->ptr, cap, stream) != hipSuccess) {
      slot->ptr = nullptr;
      *st = TK_ERR_DEVICE;
    }
    if (*st != TK_OK) return nullptr;
    slot->cap = cap;
    *fresh = true;
  }
  return slot->ptr;
}

// With g_scratch_mu held: `total` bytes of device scratch for one call, whose
// first kFusedMaxRows int32 are the fused merges' arrival counters (zero
// between calls; zeroed here whenever the buffer is new).  The stream's cached
// buffer, or one owned by the call (*owned: the caller frees it,
// stream-ordered, after its last launch).
// With g_scratch_mu held: forgets the cached buffer of (dev, stream) after a
// stream-ordered free, so the next call allocates (and zeroes) a new one.
void drop_cached(int dev, hipStream_t stream) {
  for (int i = 0; i < g_scratch_used; ++i) {
    if (g_scratch[i].dev != dev || g_scratch[i].stream != stream) continue;
    if (g_scratch[i].ptr) (void)hipFreeAsync(g_scratch[i].ptr, stream);
    g_scratch[i] = g_scratch[--g_scratch_used];
    return;
  }
}

tk_status acquire_scratch(int dev, hipStream_t stream, size_t total, char **base, bool *owned) {
  tk_status sst = TK_OK;
  bool fresh = false;
  void *scratch = cached_scratch(dev, stream, total, &sst, &fresh);
  if (sst != TK_OK) return sst;
  *owned = scratch == nullptr;
  if (*owned && hipMallocAsync(&scratch, total, stream) != hipSuccess) return TK_ERR_DEVICE;
  if ((*owned || fresh) && tk::launch_zero_fill((int32_t *)scratch, kFusedMaxRows, stream) != hipSuccess) {
    // already failing: the first error is the one reported.  A cached buffer
    // whose counters were not zeroed must not be used by a later call.
    if (*owned) (void)hipFreeAsync(scratch, stream);
    else drop_cached(dev, stream);
    return TK_ERR_DEVICE;
  }
  *base = (char *)scratch;
  return TK_OK;
}

// Where a call's scratch comes from.  Cached: the (device, stream) buffer of
// the allocating entry points, grown stream-ordered.  Fixed: the device's
// fixed array (tk_topk_bf16_noalloc), never allocated or freed; row batches
// shrink until their scratch fits it.
struct Place {
  int dev;
  hipStream_t stream;
  bool fixed;
};

// The largest batch of at most `want` rows whose scratch bytes(batch) fits
// the place: `want` itself for the cached scratch; 0 when not even one row
// fits the fixed array.
template <class Bytes>
int64_t fit_batch(const Place &p, int64_t want, Bytes bytes) {
  if (!p.fixed || bytes(want) <= tk::kFixedScratchBytes) return want;
  int64_t lo = 0, hi = want;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (bytes(mid) <= tk::kFixedScratchBytes) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// `total` bytes of scratch for one call at *base, with the arrival counters
// zero at its start (see acquire_scratch).  *owned: the caller frees it,
// stream-ordered, after its last launch (cached place only).  The caller
// holds g_scratch_mu for the cached place.
tk_status take_scratch(const Place &p, size_t total, char **base, bool *owned) {
  *owned = false;
  if (p.fixed) {
    if (total > tk::kFixedScratchBytes) return TK_ERR_SCRATCH;
    void *ptr = nullptr;
    if (tk::fixed_scratch(p.dev, p.stream, &ptr) != hipSuccess) return TK_ERR_DEVICE;
    *base = (char *)ptr;
    return TK_OK;
  }
  keep_pool(p.dev);
  return acquire_scratch(p.dev, p.stream, total, base, owned);
}

// Holds g_scratch_mu for the cached place only: calls through the fixed
// array are documented to race when they overlap on one device.
std::unique_lock<std::mutex> scratch_lock(const Place &p) {
  return p.fixed ? std::unique_lock<std::mutex>() : std::unique_lock<std::mutex>(g_scratch_mu);
}

// k = 1: span plan of the argmax scan.  On few rows a call is latency bound:
// each extra workgroup costs about 9 ns of dispatch, while a workgroup streams
// its span with a fixed number of bytes in flight, so its time grows with the
// span width; a split also adds the fold (~1.2 us: slot store, arrival count,
// slot loads).  Minimising rows * S * beta + gamma * cols / S gives S = sqrt(cols /
// (c * rows)); c = 150 matched the measured best span count on MI355X within
// 0.2 us for 1-32 rows of 98592-248320 columns (15 x 98592: 7 spans, 7.2 us
// device time; 64 x 151936: 4; 1 x 151936: 32).  Rows of fewer than
// kArgmaxSplitCols columns, and calls with a workgroup for every CU, are not
// split.  Spans stay at least kArgmaxMinSpanCols wide (each wave reads at
// least one 16-byte vector per lane) and at most kMergeGroup per row (the
// last workgroup takes the maximum of one slot per lane).  A result above
// kMergeGroup (only from the span width limit, for rows over 16.7 M columns)
// sends the call to the general scan.
constexpr int64_t kArgmaxMinSpanCols = 2048;
constexpr int64_t kArgmaxSplitCols = 32768;
constexpr double kArgmaxSpanScale = 150.0;

int32_t plan_argmax(int64_t rows, int64_t cols, int32_t compute_units) {
  if (cols <= 0 || rows <= 0) return 1;
  int64_t s = 1;
  if (rows < compute_units && cols >= kArgmaxSplitCols) {
    s = (int64_t)(std::sqrt((double)cols / (kArgmaxSpanScale * (double)rows)) + 0.5);
    const int64_t by_width = cols / kArgmaxMinSpanCols;
    if (s > by_width) s = by_width;
    if (s > kMergeGroup) s = kMergeGroup;
  }
  const int64_t need = min_spans(cols);
  if (s < need) s = need;
  if (s < 1) s = 1;
  return (int32_t)s;
}

// k = 1 through argmax_scan_kernel: spans == 1 writes the outputs directly;
// 2 <= spans <= kMergeGroup writes one slot per (row, span) after the arrival
// counters, in batches of at most kFusedMaxRows rows.
tk_status run_argmax(int64_t rows, int64_t cols, int64_t stride, const uint16_t *in, int32_t *out_idx,
                     uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite, const Place &place,
                     int32_t spans, int64_t col_base, uint32_t inf) {
  const hipStream_t stream = place.stream;
  tk::ArgmaxArgs a{};
  a.in = in;
  a.cols = cols;
  a.stride = stride;
  a.spans = spans;
  a.inf = inf;
  a.col_base = col_base;
  a.out_idx = out_idx;
  a.out_val = out_val;
  a.out_count = out_count;
  a.out_nonfinite = out_nonfinite;
  const int64_t rows_per_launch = kMaxBlocksPerLaunch / spans;
  if (spans == 1) {
    for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
      const int64_t nr = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
      a.row0 = r0;
      if (tk::launch_argmax(a, nr, stream) != hipSuccess) return TK_ERR_DEVICE;
    }
    return TK_OK;
  }
  const int64_t batch_cap = rows_per_launch > kFusedMaxRows ? kFusedMaxRows : rows_per_launch;
  const size_t off_slot = align256((size_t)kFusedMaxRows * sizeof(int32_t));
  auto bytes = [&](int64_t b) { return align256(off_slot + (size_t)b * (size_t)spans * sizeof(uint64_t)); };
  const int64_t batch = fit_batch(place, rows < batch_cap ? rows : batch_cap, bytes);
  if (batch < 1) return TK_ERR_SCRATCH;
  const size_t total = bytes(batch);
  auto lock = scratch_lock(place);
  char *base = nullptr;
  bool owned = false;
  const tk_status sst = take_scratch(place, total, &base, &owned);
  if (sst != TK_OK) return sst;
  tk_status result = TK_OK;
  for (int64_t r0 = 0; r0 < rows; r0 += batch) {
    const int64_t nr = rows - r0 < batch ? rows - r0 : batch;
    tk::ArgmaxArgs b = a;
    b.in = in + r0 * stride;
    b.row0 = 0;
    b.span_slot = (uint64_t *)(base + off_slot);
    b.row_done = (int32_t *)base;
    b.out_idx = out_idx + r0;
    b.out_val = out_val + r0;
    b.out_count = out_count + r0;
    b.out_nonfinite = out_nonfinite + r0;
    if (tk::launch_argmax(b, nr, stream) != hipSuccess) {
      result = TK_ERR_DEVICE;
      break;
    }
  }
  if (owned && hipFreeAsync(base, stream) != hipSuccess && result == TK_OK) result = TK_ERR_DEVICE;
  return result;
}

// 64 < k <= 256: the multi-register scan (tk_wide.hip).  Automatic plans
// split as for k <= 64, at most kWideMaxAutoSpans spans (the fold of a split
// row merges lists of up to 256 entries: on 15 x 98592 rows 12 spans measured
// 21.5 us at k = 128 and 42.4 us at k = 256 against 22.9 and 43.4 at 8, and
// 16 x 248320 rows at k = 256 57.7 against 61.6 us); forced plans take up to
// kMergeGroup spans; rows needing more spans (over 16.7 M columns) are
// rejected with TK_ERR_SHAPE.  Split rows are always folded by their last
// workgroup: scratch = the arrival counters, then [batch][S][k] composites,
// [batch][S] counts and flags.
constexpr int32_t kWideMaxAutoSpans = 12;

int32_t plan_wide(int64_t rows, int64_t cols, int32_t compute_units) {
  int32_t spans = doubled(rows, cols, plan(rows, cols, compute_units), compute_units);
  if (spans > kWideMaxAutoSpans) spans = kWideMaxAutoSpans;
  if (spans < (int32_t)min_spans(cols)) spans = (int32_t)min_spans(cols);
  return spans;
}

tk_status run_wide(int64_t rows, int64_t cols, int64_t stride, int32_t k, const uint16_t *in, int32_t *out_idx,
                   uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite, const Place &place,
                   int32_t forced, int32_t exact, int64_t col_base, uint32_t inf) {
  const hipStream_t stream = place.stream;
  const int32_t spans = forced > 0 ? forced : plan_wide(rows, cols, device_cus(place.dev));
  if (spans > kMergeGroup) return TK_ERR_SHAPE;  // excluded by the guards; kept as a bound on the fold
  tk::ScanArgs sa{};
  sa.in = in;
  sa.cols = cols;
  sa.stride = stride;
  sa.k = k;
  sa.spans = spans;
  sa.exact = exact;
  sa.spec_rank = exact ? 0 : spec_rank(k, cols / spans);
  sa.out_idx = out_idx;
  sa.out_val = out_val;
  sa.out_count = out_count;
  sa.out_nonfinite = out_nonfinite;
  sa.col_base = col_base;
  sa.inf = inf;
  const int64_t rows_per_launch = kMaxBlocksPerLaunch / spans;
  if (spans == 1) {
    for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
      const int64_t nr = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
      sa.row0 = r0;
      if (tk::launch_wide_scan(sa, nr, stream) != hipSuccess) return TK_ERR_DEVICE;
    }
    return TK_OK;
  }
  const int64_t batch_cap = rows_per_launch > kFusedMaxRows ? kFusedMaxRows : rows_per_launch;
  size_t off_list = 0, off_count = 0, off_flags = 0;
  auto bytes = [&](int64_t b) {
    const size_t nlists = (size_t)b * (size_t)spans;
    off_list = align256((size_t)kFusedMaxRows * sizeof(int32_t));
    off_count = align256(off_list + nlists * (size_t)k * sizeof(uint64_t));
    off_flags = align256(off_count + nlists * sizeof(int32_t));
    return align256(off_flags + nlists * sizeof(uint32_t));
  };
  const int64_t batch = fit_batch(place, rows < batch_cap ? rows : batch_cap, bytes);
  if (batch < 1) return TK_ERR_SCRATCH;
  const size_t total = bytes(batch);  // also sets the offsets for this batch
  auto lock = scratch_lock(place);
  char *base = nullptr;
  bool owned = false;
  const tk_status sst = take_scratch(place, total, &base, &owned);
  if (sst != TK_OK) return sst;
  tk_status result = TK_OK;
  for (int64_t r0 = 0; r0 < rows; r0 += batch) {
    const int64_t nr = rows - r0 < batch ? rows - r0 : batch;
    tk::ScanArgs b = sa;
    b.in = in + r0 * stride;
    b.row0 = 0;
    b.span_list = (uint64_t *)(base + off_list);
    b.span_count = (int32_t *)(base + off_count);
    b.span_flags = (uint32_t *)(base + off_flags);
    b.row_done = (int32_t *)base;
    b.out_idx = out_idx + r0 * k;
    b.out_val = out_val + r0 * k;
    b.out_count = out_count + r0;
    b.out_nonfinite = out_nonfinite + r0;
    if (tk::launch_wide_scan(b, nr, stream) != hipSuccess) {
      result = TK_ERR_DEVICE;
      break;
    }
  }
  if (owned && hipFreeAsync(base, stream) != hipSuccess && result == TK_OK) result = TK_ERR_DEVICE;
  return result;
}

// Head spans: the vocabulary's 16-column tiles cut into near-equal ranges of
// at most kHeadSpanCols / 16 tiles, one workgroup each.  By default the
// spans are full (16 tiles).  Two cases take a multiple of the CU count
// instead, the smallest whose spans fit, so that every CU holds the same
// number of workgroups: full spans would put a third workgroup on some CUs
// (more than 2 x CUs spans: 15 x 2048 x 151936 went from 140.8 to 128.1 us
// with 768 spans instead of 594), or four row tiles (more than 32 rows,
// at most two workgroups per CU: 64 x 2048 x 98592, 164.5 -> 157.4 us).
// With 15 or 32 rows of 98592 columns the 386 full spans measured faster
// than 512 of 12-13 tiles (82.3 vs 86.3 and 113.5 vs 125.7 us for the head
// kernel): there the time is set by the bytes the whole grid keeps in
// flight, which the cut does not change.
int64_t plan_head(int64_t rows, int64_t vocab, int32_t cus) {
  constexpr int64_t kTiles = tk::kHeadSpanCols / 16;
  const int64_t ntiles = (vocab + 15) / 16;
  const int64_t full = (ntiles + kTiles - 1) / kTiles;
  if (ntiles < 8 * (int64_t)cus || (full <= 2 * (int64_t)cus && rows <= 32)) return full;
  return (int64_t)cus * ((ntiles + kTiles * cus - 1) / (kTiles * cus));
}

// Lists one merge workgroup of the fused head folds at a level of n lists per
// row: all of them when they fit one workgroup, else groups of half of
// kMergeGroup (eight-wave workgroups; the last level then folds the groups).
// On 15 x 2048 x 98592 (386 lists per row -> 13 -> 1) the call took 82.2 us,
// against 82.9 with groups of 16 (386 -> 25 -> 1) and 84.2 with groups of 64
// (386 -> 7 -> 1).
int64_t head_group(int64_t n) { return n <= kMergeGroup ? n : kMergeGroup / 2; }

// Fused head: the head kernel writes one candidate list per (row, span);
// span_merge_kernel levels (groups of up to kMergeGroup lists, at least one
// level) fold them into the outputs.
tk_status run_head(int64_t rows, int64_t hidden, int64_t vocab, int32_t k, const uint16_t *h, int64_t h_stride,
                   const uint16_t *w, int64_t w_stride, int32_t *out_idx, uint16_t *out_val, int32_t *out_count,
                   uint32_t *out_nonfinite, uint16_t *logits, int64_t logits_stride, hipStream_t stream, int dev) {
  const int64_t spans = plan_head(rows, vocab, device_cus(dev));
  // merge levels: lists in per row at each level; the last level has one
  // group per row (lists_out == 1) and writes the outputs, every earlier level
  // writes the next level's lists (span_merge_kernel tells the two apart by
  // lists_out alone)
  int64_t level_lists[8];
  int levels = 0;
  int64_t n = spans;
  do {
    level_lists[levels++] = n;
    n = (n + head_group(n) - 1) / head_group(n);
  } while (n > 1);
  size_t off_list[8], off_count[8], off_flags[8], total = 0;
  for (int i = 0; i < levels; ++i) {
    const size_t nlists = (size_t)rows * (size_t)level_lists[i];
    off_list[i] = total;
    total = align256(total + nlists * (size_t)k * sizeof(uint64_t));
    off_count[i] = total;
    total = align256(total + nlists * sizeof(int32_t));
    off_flags[i] = total;
    total = align256(total + nlists * sizeof(uint32_t));
  }
  const size_t off0 = align256((size_t)kFusedMaxRows * sizeof(int32_t));  // the counters stay untouched
  const Place place{dev, stream, false};
  auto lock = scratch_lock(place);
  char *base = nullptr;
  bool owned = false;
  const tk_status sst = take_scratch(place, off0 + total, &base, &owned);
  if (sst != TK_OK) return sst;
  base += off0;
  tk_status result = TK_OK;
  tk::HeadArgs ha{};
  ha.rows = rows;
  ha.hidden = hidden;
  ha.vocab = vocab;
  ha.k = k;
  ha.spans = (int32_t)spans;
  ha.h = h;
  ha.h_stride = h_stride;
  ha.w = w;
  ha.w_stride = w_stride;
  ha.span_list = (uint64_t *)(base + off_list[0]);
  ha.span_count = (int32_t *)(base + off_count[0]);
  ha.span_flags = (uint32_t *)(base + off_flags[0]);
  ha.logits = logits;
  ha.logits_stride = logits_stride;
  // the row sketch lives in the counter words at the buffer's start, zero
  // between calls (the last merge level zeroes it again); one row tile only
  uint32_t *sketch = rows <= 16 ? (uint32_t *)(base - off0) : nullptr;
  static_assert(16 * kMaxK <= kFusedMaxRows, "the sketch fits the counter words");
  ha.sketch = sketch;
  if (tk::launch_head_scan(ha, stream) != hipSuccess) result = TK_ERR_DEVICE;
  for (int i = 0; i < levels && result == TK_OK; ++i) {
    tk::MergeArgs m{};
    m.in = nullptr;
    m.row0 = 0;
    m.k = k;
    m.lists_in = (int32_t)level_lists[i];
    m.group = (int32_t)head_group(m.lists_in);
    m.lists_out = (m.lists_in + m.group - 1) / m.group;
    m.list_in = (const uint64_t *)(base + off_list[i]);
    m.count_in = (const int32_t *)(base + off_count[i]);
    m.flags_in = (const uint32_t *)(base + off_flags[i]);
    if ((m.lists_out == 1) != (i + 1 == levels)) {  // the level plan and the kernel's test must agree
      result = TK_ERR_DEVICE;
      break;
    }
    if (i + 1 < levels) {
      m.list_out = (uint64_t *)(base + off_list[i + 1]);
      m.count_out = (int32_t *)(base + off_count[i + 1]);
      m.flags_out = (uint32_t *)(base + off_flags[i + 1]);
    } else {
      m.out_idx = out_idx;
      m.out_val = out_val;
      m.out_count = out_count;
      m.out_nonfinite = out_nonfinite;
      m.sketch = sketch;
    }
    if (tk::launch_span_merge(m, rows, stream) != hipSuccess) result = TK_ERR_DEVICE;
  }
  // a head kernel that ran without its last merge level leaves the sketch
  // (the counter words) non-zero: such a cached buffer must not be used again
  if (result != TK_OK && sketch && !owned) drop_cached(dev, stream);
  if (owned && hipFreeAsync(base - off0, stream) != hipSuccess && result == TK_OK) result = TK_ERR_DEVICE;
  return result;
}

tk_status run(int64_t rows, int64_t cols, int64_t stride, int32_t k, const uint16_t *in, int32_t *out_idx,
              uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite, void *stream_handle,
              const tk_options *opt, int64_t col_base = 0, uint32_t inf = 0x7F80u, bool fixed = false) {
  tk_status st = guard(rows, cols, stride, k, in, out_idx, out_val, out_count, out_nonfinite);
  if (st != TK_OK) return st;
  if (col_base < 0 || col_base > (int64_t)INT32_MAX - cols + (cols > 0 ? 1 : 0)) return TK_ERR_SHAPE;
  int32_t forced = 0, exact = 0, general = 0;
  if (opt) {
    for (int i = 0; i < 5; ++i)
      if (opt->reserved[i] != 0) return TK_ERR_OPTION;
    if (opt->exact != 0 && opt->exact != 1) return TK_ERR_OPTION;
    if (opt->general != 0 && opt->general != 1) return TK_ERR_OPTION;
    exact = opt->exact;
    general = opt->general;
    forced = opt->spans;
    if (forced < 0 || forced > kMaxSpans) return TK_ERR_OPTION;
    if (forced > 1 && cols > 0 && forced > cols) return TK_ERR_OPTION;
    if (forced >= 1 && forced < min_spans(cols)) return TK_ERR_OPTION;
    if (k > kMaxK && forced > kMergeGroup) return TK_ERR_OPTION;
  }
  if (rows == 0) return TK_OK;

  hipStream_t stream = (hipStream_t)stream_handle;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TK_ERR_DEVICE;
  const Place place{dev, stream, fixed};
  if (k > kMaxK)
    return run_wide(rows, cols, stride, k, in, out_idx, out_val, out_count, out_nonfinite, place, forced,
                    exact, col_base, inf);
  // k = 1: the argmax scan on few rows (or a forced split); with a row for
  // every CU the general scan measured ~2% faster (49.0 vs 50.2 us on 1024 x
  // 151936: both at the read ceiling, the general scan's progress priority
  // evens out its waves' finish times).
  if (k == 1 && !general && (forced > 0 || rows < device_cus(dev))) {
    const int32_t s1 = forced > 0 ? forced : plan_argmax(rows, cols, device_cus(dev));
    if (s1 <= kMergeGroup)
      return run_argmax(rows, cols, stride, in, out_idx, out_val, out_count, out_nonfinite, place, s1,
                        col_base, inf);
  }
  const int32_t spans = forced > 0 ? forced : plan_scan16(rows, cols, k, device_cus(dev));

  tk::ScanArgs sa{};
  sa.in = in;
  sa.cols = cols;
  sa.stride = stride;
  sa.k = k;
  sa.spans = spans;
  sa.exact = exact;
  sa.spec_rank = exact ? 0 : spec_rank(k, cols / spans);
  sa.out_idx = out_idx;
  sa.out_val = out_val;
  sa.out_count = out_count;
  sa.out_nonfinite = out_nonfinite;
  sa.col_base = col_base;
  sa.inf = inf;

  const int64_t rows_per_launch = kMaxBlocksPerLaunch / spans;
  if (spans == 1) {
    for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
      const int64_t nr = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
      sa.row0 = r0;
      if (tk::launch_span_scan(sa, nr, stream) != hipSuccess) return TK_ERR_DEVICE;
    }
    return TK_OK;
  }

  // Scratch for one batch of rows: the fused merge's arrival counters (always
  // at offset 0, so that they keep their all-zero state between calls whatever
  // the shapes), then the span lists, then each merge level's lists.  With at
  // most kMergeGroup spans and kFusedMaxRows rows per launch the scan folds
  // the span lists itself (one dispatch); otherwise merge dispatches follow.
  const bool fused = spans <= kMergeGroup && rows_per_launch >= 1;
  const int64_t batch_cap = fused && rows_per_launch > kFusedMaxRows ? kFusedMaxRows : rows_per_launch;
  int32_t level_lists[8];
  int levels = 0;
  for (int32_t n = spans; n > 1; n = (n + kMergeGroup - 1) / kMergeGroup) level_lists[levels++] = n;
  if (fused) levels = 1;  // only the span lists
  const size_t counters_bytes = align256((size_t)kFusedMaxRows * sizeof(int32_t));
  size_t off_list[8], off_count[8], off_flags[8];
  auto bytes = [&](int64_t b) {
    size_t total = counters_bytes;
    for (int i = 0; i < levels; ++i) {
      const size_t nlists = (size_t)b * (size_t)level_lists[i];
      off_list[i] = total;
      total = align256(total + nlists * (size_t)k * sizeof(uint64_t));
      off_count[i] = total;
      total = align256(total + nlists * sizeof(int32_t));
      off_flags[i] = total;
      total = align256(total + nlists * sizeof(uint32_t));
    }
    return total;
  };
  const int64_t batch = fit_batch(place, rows < batch_cap ? rows : batch_cap, bytes);
  if (batch < 1) return TK_ERR_SCRATCH;
  const size_t total = bytes(batch);  // also sets the offsets for this batch
  auto lock = scratch_lock(place);
  char *base = nullptr;
  bool owned = false;
  const tk_status sst = take_scratch(place, total, &base, &owned);
  if (sst != TK_OK) return sst;
  int32_t *counters = (int32_t *)base;

  tk_status result = TK_OK;
  for (int64_t r0 = 0; r0 < rows && result == TK_OK; r0 += batch) {
    const int64_t nr = rows - r0 < batch ? rows - r0 : batch;
    // Scratch rows are indexed from the batch start: point the row-indexed
    // outputs at the batch, and offset the input by r0 rows.
    tk::ScanArgs b = sa;
    b.in = in + r0 * stride;
    b.row0 = 0;
    b.span_list = (uint64_t *)(base + off_list[0]);
    b.span_count = (int32_t *)(base + off_count[0]);
    b.span_flags = (uint32_t *)(base + off_flags[0]);
    if (fused) {
      b.row_done = counters;
      b.out_idx = out_idx + r0 * k;
      b.out_val = out_val + r0 * k;
      b.out_count = out_count + r0;
      b.out_nonfinite = out_nonfinite + r0;
    }
    if (tk::launch_span_scan(b, nr, stream) != hipSuccess) {
      result = TK_ERR_DEVICE;
      break;
    }
    for (int i = 0; i < levels && !fused; ++i) {
      tk::MergeArgs m{};
      m.in = in + r0 * stride;
      m.row0 = 0;
      m.stride = stride;
      m.k = k;
      m.lists_in = level_lists[i];
      m.group = level_lists[i] < kMergeGroup ? level_lists[i] : kMergeGroup;
      m.lists_out = (level_lists[i] + m.group - 1) / m.group;
      m.list_in = (const uint64_t *)(base + off_list[i]);
      m.count_in = (const int32_t *)(base + off_count[i]);
      m.flags_in = (const uint32_t *)(base + off_flags[i]);
      m.col_base = col_base;
      if (i + 1 < levels) {
        m.list_out = (uint64_t *)(base + off_list[i + 1]);
        m.count_out = (int32_t *)(base + off_count[i + 1]);
        m.flags_out = (uint32_t *)(base + off_flags[i + 1]);
      } else {
        m.out_idx = out_idx + r0 * k;
        m.out_val = out_val + r0 * k;
        m.out_count = out_count + r0;
        m.out_nonfinite = out_nonfinite + r0;
      }
      if (tk::launch_span_merge(m, nr, stream) != hipSuccess) {
        result = TK_ERR_DEVICE;
        break;
      }
    }
  }
  if (owned && hipFreeAsync(base, stream) != hipSuccess && result == TK_OK) result = TK_ERR_DEVICE;
  return result;
}

// k = 1 on fp32 rows: the plan of the 16-bit argmax scan at equal bytes (a
// 4-byte column weighs two 2-byte ones); composites carry absolute columns,
// so no span width limit applies.
int32_t plan_argmax32(int64_t rows, int64_t cols, int32_t compute_units) {
  if (cols <= 0 || rows <= 0) return 1;
  const int64_t cols2 = 2 * cols;
  int64_t s = 1;
  if (rows < compute_units && cols2 >= kArgmaxSplitCols) {
    s = (int64_t)(std::sqrt((double)cols2 / (kArgmaxSpanScale * (double)rows)) + 0.5);
    const int64_t by_width = cols2 / kArgmaxMinSpanCols;
    if (s > by_width) s = by_width;
    if (s > kMergeGroup) s = kMergeGroup;
  }
  return s < 1 ? 1 : (int32_t)s;
}

tk_status run_argmax32(int64_t rows, int64_t cols, int64_t stride, const uint32_t *in, int32_t *out_idx,
                       uint32_t *out_val, int32_t *out_count, uint32_t *out_nonfinite, hipStream_t stream, int dev,
                       int32_t spans) {
  tk::ArgmaxArgs32 a{};
  a.in = in;
  a.cols = cols;
  a.stride = stride;
  a.spans = spans;
  a.out_idx = out_idx;
  a.out_val = out_val;
  a.out_count = out_count;
  a.out_nonfinite = out_nonfinite;
  const int64_t rows_per_launch = kMaxBlocksPerLaunch / spans;
  if (spans == 1) {
    for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
      const int64_t nr = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
      a.row0 = r0;
      if (tk::launch_argmax32(a, nr, stream) != hipSuccess) return TK_ERR_DEVICE;
    }
    return TK_OK;
  }
  const int64_t batch_cap = rows_per_launch > kFusedMaxRows ? kFusedMaxRows : rows_per_launch;
  const int64_t batch = rows < batch_cap ? rows : batch_cap;
  const size_t nslots = (size_t)batch * (size_t)spans;
  const size_t off_slot = align256((size_t)kFusedMaxRows * sizeof(int32_t));
  const size_t off_flag = align256(off_slot + nslots * sizeof(uint64_t));
  const size_t total = align256(off_flag + nslots * sizeof(uint32_t));
  keep_pool(dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  char *base = nullptr;
  bool owned = false;
  const tk_status sst = acquire_scratch(dev, stream, total, &base, &owned);
  if (sst != TK_OK) return sst;
  tk_status result = TK_OK;
  for (int64_t r0 = 0; r0 < rows; r0 += batch) {
    const int64_t nr = rows - r0 < batch ? rows - r0 : batch;
    tk::ArgmaxArgs32 b = a;
    b.in = in + r0 * stride;
    b.row0 = 0;
    b.span_slot = (uint64_t *)(base + off_slot);
    b.span_flag = (uint32_t *)(base + off_flag);
    b.row_done = (int32_t *)base;
    b.out_idx = out_idx + r0;
    b.out_val = out_val + r0;
    b.out_count = out_count + r0;
    b.out_nonfinite = out_nonfinite + r0;
    if (tk::launch_argmax32(b, nr, stream) != hipSuccess) {
      result = TK_ERR_DEVICE;
      break;
    }
  }
  if (owned && hipFreeAsync(base, stream) != hipSuccess && result == TK_OK) result = TK_ERR_DEVICE;
  return result;
}

// fp32 rows: the same plan, guards and scratch layout as the bf16 split path;
// every split row is folded by its last scan workgroup (at most kMergeGroup
// spans: the fp32 scan has no span width limit, so a plan never needs more).
tk_status run32(int64_t rows, int64_t cols, int64_t stride, int32_t k, const uint32_t *in, int32_t *out_idx,
                uint32_t *out_val, int32_t *out_count, uint32_t *out_nonfinite, void *stream_handle,
                const tk_options *opt) {
  tk_status st = guard(rows, cols, stride, k, in, out_idx, out_val, out_count, out_nonfinite, 4, kMaxKWide);
  if (st != TK_OK) return st;
  int32_t forced = 0, exact = 0, general = 0;
  if (opt) {
    for (int i = 0; i < 5; ++i)
      if (opt->reserved[i] != 0) return TK_ERR_OPTION;
    if (opt->exact != 0 && opt->exact != 1) return TK_ERR_OPTION;
    if (opt->general != 0 && opt->general != 1) return TK_ERR_OPTION;
    exact = opt->exact;
    general = opt->general;
    forced = opt->spans;
    if (forced < 0 || forced > kMergeGroup) return TK_ERR_OPTION;
    if (forced > 1 && cols > 0 && forced > cols) return TK_ERR_OPTION;
  }
  if (rows == 0) return TK_OK;
  hipStream_t stream = (hipStream_t)stream_handle;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TK_ERR_DEVICE;
  if (k == 1 && !general && (forced > 0 || rows < device_cus(dev)))  // as for bf16: few rows or a forced split
    return run_argmax32(rows, cols, stride, in, out_idx, out_val, out_count, out_nonfinite, stream, dev,
                        forced > 0 ? forced : plan_argmax32(rows, cols, device_cus(dev)));
  int32_t spans = forced > 0 ? forced : doubled(rows, cols, plan(rows, cols, device_cus(dev)), device_cus(dev));
  if (spans > kMergeGroup) spans = kMergeGroup;
  if (k > kMaxK && forced == 0 && spans > kWideMaxAutoSpans) spans = kWideMaxAutoSpans;
  // k > 64: the multi-register scan, with the same arguments and scratch
  hipError_t (*const launch)(const tk::ScanArgs32 &, int64_t, hipStream_t) =
      k > kMaxK ? tk::launch_wide_scan32 : tk::launch_span_scan32;

  tk::ScanArgs32 sa{};
  sa.in = in;
  sa.cols = cols;
  sa.stride = stride;
  sa.k = k;
  sa.spans = spans;
  sa.exact = exact;
  // the pooled sample holds half as many fp32 elements as bf16 ones
  sa.spec_rank = exact ? 0 : spec_rank(k, cols / spans, kSampleElems / 2);
  sa.out_idx = out_idx;
  sa.out_val = out_val;
  sa.out_count = out_count;
  sa.out_nonfinite = out_nonfinite;
  const int64_t rows_per_launch = kMaxBlocksPerLaunch / spans;
  if (spans == 1) {
    for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
      const int64_t nr = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
      sa.row0 = r0;
      if (launch(sa, nr, stream) != hipSuccess) return TK_ERR_DEVICE;
    }
    return TK_OK;
  }
  const int64_t batch_cap = rows_per_launch > kFusedMaxRows ? kFusedMaxRows : rows_per_launch;
  const int64_t batch = rows < batch_cap ? rows : batch_cap;
  const size_t counters_bytes = align256((size_t)kFusedMaxRows * sizeof(int32_t));
  const size_t nlists = (size_t)batch * (size_t)spans;
  const size_t off_list = counters_bytes;
  const size_t off_count = align256(off_list + nlists * (size_t)k * sizeof(uint64_t));
  const size_t off_flags = align256(off_count + nlists * sizeof(int32_t));
  const size_t total = align256(off_flags + nlists * sizeof(uint32_t));
  const Place place{dev, stream, false};
  auto lock = scratch_lock(place);
  char *base = nullptr;
  bool owned = false;
  const tk_status sst = take_scratch(place, total, &base, &owned);
  if (sst != TK_OK) return sst;
  int32_t *counters = (int32_t *)base;
  tk_status result = TK_OK;
  for (int64_t r0 = 0; r0 < rows; r0 += batch) {
    const int64_t nr = rows - r0 < batch ? rows - r0 : batch;
    tk::ScanArgs32 b = sa;
    b.in = in + r0 * stride;
    b.row0 = 0;
    b.span_list = (uint64_t *)(base + off_list);
    b.span_count = (int32_t *)(base + off_count);
    b.span_flags = (uint32_t *)(base + off_flags);
    b.row_done = counters;
    b.out_idx = out_idx + r0 * k;
    b.out_val = out_val + r0 * k;
    b.out_count = out_count + r0;
    b.out_nonfinite = out_nonfinite + r0;
    if (launch(b, nr, stream) != hipSuccess) {
      result = TK_ERR_DEVICE;
      break;
    }
  }
  if (owned && hipFreeAsync(base, stream) != hipSuccess && result == TK_OK) result = TK_ERR_DEVICE;
  return result;
}

}  // namespace

extern "C" {

tk_status tk_topk_bf16(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                       int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                       void *stream) {
  return run(rows, cols, row_stride, k, in, out_idx, out_val, out_count, out_nonfinite, stream, nullptr);
}

tk_status tk_topk_bf16_noalloc(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                               int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                               void *stream) {
  return run(rows, cols, row_stride, k, in, out_idx, out_val, out_count, out_nonfinite, stream, nullptr, 0, 0x7F80u,
             true);
}

tk_status tk_topk_bf16_ex(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                          int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                          void *stream, const tk_options *opt) {
  return run(rows, cols, row_stride, k, in, out_idx, out_val, out_count, out_nonfinite, stream, opt);
}

tk_status tk_topk_f16(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                      int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite, void *stream) {
  return run(rows, cols, row_stride, k, in, out_idx, out_val, out_count, out_nonfinite, stream, nullptr, 0, 0x7C00u);
}

tk_status tk_topk_f16_ex(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                         int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                         void *stream, const tk_options *opt) {
  return run(rows, cols, row_stride, k, in, out_idx, out_val, out_count, out_nonfinite, stream, opt, 0, 0x7C00u);
}

tk_status tk_topk_f32(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint32_t *in,
                      int32_t *out_idx, uint32_t *out_val, int32_t *out_count, uint32_t *out_nonfinite, void *stream) {
  return run32(rows, cols, row_stride, k, in, out_idx, out_val, out_count, out_nonfinite, stream, nullptr);
}

tk_status tk_topk_f32_ex(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint32_t *in,
                         int32_t *out_idx, uint32_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                         void *stream, const tk_options *opt) {
  return run32(rows, cols, row_stride, k, in, out_idx, out_val, out_count, out_nonfinite, stream, opt);
}

tk_status tk_validate_f32(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint32_t *in,
                          const int32_t *out_idx, const uint32_t *out_val, const int32_t *out_count,
                          const uint32_t *out_nonfinite) {
  return guard(rows, cols, row_stride, k, in, out_idx, out_val, out_count, out_nonfinite, 4, kMaxKWide);
}

tk_status tk_validate_bf16(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                           const int32_t *out_idx, const uint16_t *out_val, const int32_t *out_count,
                           const uint32_t *out_nonfinite) {
  return guard(rows, cols, row_stride, k, in, out_idx, out_val, out_count, out_nonfinite);
}

tk_status tk_topk_bf16_shard(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, int64_t col_base,
                             const uint16_t *in, int32_t *out_idx, uint16_t *out_val, int32_t *out_count,
                             uint32_t *out_nonfinite, void *stream) {
  return run(rows, cols, row_stride, k, in, out_idx, out_val, out_count, out_nonfinite, stream, nullptr, col_base);
}

tk_status tk_validate_merge_bf16(int64_t rows, int32_t shards, int32_t k, const int32_t *idx_in,
                                 const uint16_t *val_in, const int32_t *count_in, const uint32_t *mask_in,
                                 const int32_t *out_idx, const uint16_t *out_val, const int32_t *out_count,
                                 const uint32_t *out_nonfinite) {
  return guard_merge(rows, shards, k, idx_in, val_in, count_in, mask_in, out_idx, out_val, out_count, out_nonfinite);
}

tk_status tk_merge_topk_bf16(int64_t rows, int32_t shards, int32_t k, const int32_t *idx_in, const uint16_t *val_in,
                             const int32_t *count_in, const uint32_t *mask_in, int32_t *out_idx, uint16_t *out_val,
                             int32_t *out_count, uint32_t *out_nonfinite, void *stream) {
  const tk_status st =
      guard_merge(rows, shards, k, idx_in, val_in, count_in, mask_in, out_idx, out_val, out_count, out_nonfinite);
  if (st != TK_OK || rows == 0) return st;
  tk::ShardMergeArgs m{};
  m.rows = rows;
  m.shards = shards;
  m.k = k;
  m.idx_in = idx_in;
  m.val_in = val_in;
  m.count_in = count_in;
  m.mask_in = mask_in;
  m.out_idx = out_idx;
  m.out_val = out_val;
  m.out_count = out_count;
  m.out_nonfinite = out_nonfinite;
  return tk::launch_shard_merge(m, (hipStream_t)stream) == hipSuccess ? TK_OK : TK_ERR_DEVICE;
}

tk_status tk_validate_sample_bf16(int64_t rows, int32_t k, const int32_t *idx, const uint16_t *val,
                                  const int32_t *count, float temperature, float top_p, const int32_t *out_token,
                                  const int32_t *out_kept) {
  return guard_sample(rows, k, idx, val, count, temperature, top_p, out_token, out_kept);
}

tk_status tk_sample_topk_bf16(int64_t rows, int32_t k, const int32_t *idx, const uint16_t *val, const int32_t *count,
                              float temperature, float top_p, uint64_t seed, uint64_t offset, int32_t *out_token,
                              int32_t *out_kept, void *stream) {
  const tk_status st = guard_sample(rows, k, idx, val, count, temperature, top_p, out_token, out_kept);
  if (st != TK_OK || rows == 0) return st;
  tk::SampleArgs a{};
  a.rows = rows;
  a.k = k;
  a.idx = idx;
  a.val = val;
  a.count = count;
  a.greedy = temperature == 0.0f;
  // log2(e) / T in double, as the float32 T was given; log2(e) from the
  // double nearest e
  a.scale = a.greedy ? 0.0f : (float)(std::log2(2.718281828459045) / (double)temperature);
  a.top_p = top_p;
  double fact = 1.0;
  for (int i = 0; i < 8; ++i) {
    if (i > 0) fact *= i;
    a.coef[i] = (float)(std::pow(std::log(2.0), (double)i) / fact);
  }
  a.key0 = (uint32_t)seed;
  a.key1 = (uint32_t)(seed >> 32);
  a.off0 = (uint32_t)offset;
  a.off1 = (uint32_t)(offset >> 32);
  a.out_token = out_token;
  a.out_kept = out_kept;
  return tk::launch_sample(a, (hipStream_t)stream) == hipSuccess ? TK_OK : TK_ERR_DEVICE;
}

tk_status tk_validate_head_bf16(int64_t rows, int64_t hidden, int64_t vocab, int32_t k, const uint16_t *h,
                                int64_t h_stride, const uint16_t *w, int64_t w_stride, const int32_t *out_idx,
                                const uint16_t *out_val, const int32_t *out_count, const uint32_t *out_nonfinite,
                                const uint16_t *logits, int64_t logits_stride) {
  return guard_head(rows, hidden, vocab, k, h, h_stride, w, w_stride, out_idx, out_val, out_count, out_nonfinite,
                    logits, logits_stride);
}

tk_status tk_head_topk_bf16(int64_t rows, int64_t hidden, int64_t vocab, int32_t k, const uint16_t *h,
                            int64_t h_stride, const uint16_t *w, int64_t w_stride, int32_t *out_idx,
                            uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite, uint16_t *logits,
                            int64_t logits_stride, void *stream) {
  const tk_status st = guard_head(rows, hidden, vocab, k, h, h_stride, w, w_stride, out_idx, out_val, out_count,
                                  out_nonfinite, logits, logits_stride);
  if (st != TK_OK || rows == 0) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TK_ERR_DEVICE;
  return run_head(rows, hidden, vocab, k, h, h_stride, w, w_stride, out_idx, out_val, out_count, out_nonfinite,
                  logits, logits_stride, (hipStream_t)stream, dev);
}

int32_t tk_plan_spans(int64_t rows, int64_t cols, int32_t k, int32_t compute_units) {
  const int32_t cus = compute_units > 0 ? compute_units : 256;
  if (k > kMaxK) return plan_wide(rows, cols, cus);
  if (k == 1) {
    const int32_t s1 = plan_argmax(rows, cols, cus);
    if (s1 <= kMergeGroup) return s1;
  }
  return plan_scan16(rows, cols, k, cus);
}

tk_status tk_probe_read(const void *in, int64_t bytes, int32_t workgroups, uint32_t *sink, void *stream) {
  if (bytes < 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > kMaxBlocksPerLaunch) return TK_ERR_SHAPE;
  // each wave's share must fit the loads' 32-bit descriptor range
  if (bytes / 16 / ((int64_t)workgroups * tk::kWgWaves) + 1 > (int64_t(1) << 26)) return TK_ERR_SHAPE;
  if ((bytes > 0 && !in) || !sink) return TK_ERR_NULL;
  if (((uintptr_t)in & 15) || ((uintptr_t)sink & 3)) return TK_ERR_ALIGN;
  const Range rin{(uintptr_t)in, (uintptr_t)in + (uintptr_t)bytes}, rsink{(uintptr_t)sink, (uintptr_t)sink + 4 * 8192};
  if (overlap(rin, rsink)) return TK_ERR_ALIAS;
  return tk::launch_read_probe(in, bytes / 16, workgroups, sink, (hipStream_t)stream) == hipSuccess ? TK_OK
                                                                                                    : TK_ERR_DEVICE;
}

tk_status tk_release_stream(void *stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TK_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  for (int i = 0; i < g_scratch_used; ++i) {
    if (g_scratch[i].dev != dev || g_scratch[i].stream != (hipStream_t)stream) continue;
    // stream-ordered: the free waits for the work already queued on the stream
    const tk_status st =
        g_scratch[i].ptr && hipFreeAsync(g_scratch[i].ptr, g_scratch[i].stream) != hipSuccess ? TK_ERR_DEVICE : TK_OK;
    g_scratch[i] = g_scratch[--g_scratch_used];  // forgotten either way: the next call allocates afresh
    return st;
  }
  return TK_OK;
}

int32_t tk_max_k(void) { return kMaxKWide; }

int64_t tk_max_span_cols(void) { return tk::kMaxSpanCols; }

const char *tk_status_string(tk_status s) {
  switch (s) {
    case TK_OK: return "ok";
    case TK_ERR_NULL: return "a required pointer is NULL";
    case TK_ERR_SHAPE: return "invalid shape (rows, cols or row_stride)";
    case TK_ERR_K: return "k out of range [1, TK_MAX_K] ([1, TK_MAX_K_LANE] for fp32 rows, shard merge, sampling)";
    case TK_ERR_ALIGN: return "misaligned buffer";
    case TK_ERR_ALIAS: return "buffers overlap";
    case TK_ERR_DEVICE: return "HIP error while allocating or launching";
    case TK_ERR_OPTION: return "invalid tk_options";
    case TK_ERR_SCRATCH: return "one row needs more scratch than the fixed array of tk_topk_bf16_noalloc holds";
  }
  return "unknown status";
}

const char *tk_build_info(void) { return TK_BUILD_INFO; }

}  // extern "C"
