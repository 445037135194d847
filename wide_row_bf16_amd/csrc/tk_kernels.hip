// Exact row-wise bf16 top-k kernels for CDNA4 (gfx950).
//
// What is computed (TensorFold PR #713 "the drafter's attention and top-k use
// more of the GPU", change 3): each row's k best entries, highest score first,
// equal scores ordered by the lower column (token) index.  Wide rows may be
// split into spans whose candidate lists a second dispatch merges under that
// same order; the result must not depend on the split (Exactness table of the
// same page).
//
// Order key.  A bf16 pattern b with magnitude m = b & 0x7FFF maps to the
// 16-bit key 0x8000 + m (sign clear) or 0x8000 - m (sign set).  The key is
// monotone in value, gives +0 and -0 the same key 0x8000, keeps subnormals
// in order, and sends -inf to 0x0080 and +inf to 0xFF80.  NaN (m > 0x7F80)
// gets key 0, below every number, and is never kept.  IEEE fp16 patterns are
// sign-magnitude too: the same map works with +inf at 0x7C00 (keys 0x0400
// and 0xFC00 for -inf and +inf), so the scan takes the +inf pattern as an
// argument.  Inside one wave the
// composite (key << 16) | (0xFFFF - rel), rel = column - wave base < 65536,
// is a strict total order equal to (score desc, column asc); across waves and
// spans the 64-bit composite (key << 32) | (0xFFFFFFFF - column) is used.
//
// Scan (one workgroup = four wave64s per (row, span)).  Each wave streams its
// contiguous share of the span with 16-byte loads (64 lanes x 16 B = 1 KiB per
// load instruction, four per lane per chunk, double buffered) and keeps the 64
// best composites seen so far in one VGPR, lane i holding the i-th best.  Let
// T be the k-th kept key.  A wave visits its columns in increasing order, so a
// later element that only ties T loses to it (lower column wins): the filter
// "key > T" is exact.  It is evaluated on raw bf16 bits with two packed 16-bit
// operations per dword: for T >= 0 an element beats T iff its bits, read as
// int16, exceed T's magnitude; for T < 0 iff its bits, read as uint16, are
// below T's bits.  A per-lane packed uint16 max also catches -inf and NaN
// patterns the wave has not flagged yet.  Only when some lane trips does the
// wave take the exact path: keys and composites per element, a 19-comparator
// sort of the lane's eight, and insertion position by position -- one DPP
// wave_shr per new entry when few lanes have one, a bitonic sort and merge of
// 64 when many do.
//
// Merge.  The four wave lists, as 64-bit composites, meet as a two-level tree
// of register bitonic merges.  With several spans per row (up to 64) each
// workgroup writes its span list to memory and the row's last workgroup to
// arrive folds the row's lists the same way (fold_row_if_last); above 64
// spans, and for the fused head, span_merge_kernel folds them in groups.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tk_config.h"
#include "tk_launch.h"
#include "tk_stamps.h"

namespace tk {
namespace {

#include "tk_wave.h"
#include "tk_scan16.h"

struct WaveTopK {
  uint32_t list;   // lane i: i-th best composite so far, 0 = empty
  uint32_t kth;    // wave-uniform copy of list[k - 1]
  uint32_t ext;    // wave-uniform: keys <= ext are beaten by k entries of other waves
  uint32_t floor;  // wave-uniform floor: only keys > floor are kept (0 = none)
  uint32_t flags;  // wave-uniform TK_NONFINITE_NAN / _NEGINF seen so far
  uint32_t inf;    // wave-uniform +inf pattern of the input format
  int km1;         // k - 1
  int qm1;         // ceil(k / 4) - 1
  int wave;        // this wave's index in the workgroup
  uint32_t *tau;   // LDS: published k-th keys of the workgroup's waves
  Xchg x;
};

// Adds the candidates c of lanes m (their composites beat the k-th) to the
// list: one bitonic batch when many, else one insertion each.  Insertions
// test against a copy of the k-th that is refreshed only afterwards: a stale
// (lower) k-th only lets extra candidates through, and inserting one that no
// longer qualifies changes list slots >= k only.
__device__ __forceinline__ void offer(WaveTopK &w, uint32_t c, uint64_t m) {
  if (__popcll(m) >= kBatchInsert) {
    w.list = merge_batch(w.list, c > w.kth ? c : 0u, w.x);
  } else {
    do {
      const int l = __builtin_ctzll(m);
      m &= m - 1;
      w.list = insert_one(w.list, readlane(c, l));
    } while (m);
  }
  w.kth = readlane(w.list, w.km1);
}

// Threshold sharing between the waves of a workgroup.  Each wave publishes
// two keys of its kept list: tau = its k-th entry and q = its ceil(k/4)-th
// entry (0 while it holds fewer).  Two bounds follow, each meaning "k kept
// entries of the workgroup beat every key below it":
//  - one wave's tau: a wave to the left (lower columns) also beats keys equal
//    to tau, since on equal keys the lower column wins; a wave to the right
//    beats only keys < tau;
//  - the smallest q of all four waves: each holds ceil(k/4) entries >= it, so
//    k entries beat every key below it (equal keys may lie either side).
// For evenly spread data the second is about the k-th key of the union.
// Published values only rise, so a stale read is still a valid bound.
__device__ __forceinline__ uint32_t shared_bound(const uint32_t *s_tau, int wave) {
  uint32_t ext = 0, qmin = 0xFFFFFFFFu;
#pragma unroll
  for (int o = 0; o < kWgWaves; ++o) {
    const uint32_t t = __hip_atomic_load(&s_tau[o], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint32_t q = __hip_atomic_load(&s_tau[kWgWaves + o], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint32_t b = o < wave ? t : (t > 0 ? t - 1 : 0u);
    if (o != wave) ext = max(ext, b);
    qmin = min(qmin, q);
  }
  if (qmin > 0) ext = max(ext, qmin - 1);
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)ext);
}

__device__ __forceinline__ void publish(uint32_t *s_tau, int wave, const WaveTopK &w) {
  const uint32_t q = readlane(w.list, w.qm1) >> 16;
  if (lane_id() == 0) {
    __hip_atomic_store(&s_tau[wave], w.kth >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(&s_tau[kWgWaves + wave], q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

__device__ __forceinline__ Filter make_filter(const WaveTopK &w) {
  const uint32_t own = (uint32_t)__builtin_amdgcn_readfirstlane((int)w.kth) >> 16;
  const uint32_t tkey = max(own, (uint32_t)__builtin_amdgcn_readfirstlane((int)w.ext));
  return filter_for(tkey, (uint32_t)__builtin_amdgcn_readfirstlane((int)w.flags),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)w.inf));
}

// Exact path for one 16-byte vector per lane when many lanes trip (while the
// kept set is young): composites of all eight elements, a per-lane sort, then
// insertion position by position.  Its eight elements sit at columns col0 ..
// col0 + 7 with inv0 = 0xFFFF - (col0 - wave base).
__device__ __forceinline__ void take_vector_dense(WaveTopK &w, uint4 d, uint32_t inv0, bool valid) {
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
  uint32_t c[8];
  bool nan = false, ninf = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t b = (dw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
    const uint32_t key = order_key(b, w.inf);
    nan |= (b & 0x7FFFu) > w.inf;
    ninf |= b == (0x8000u | w.inf);
    c[e] = (valid && key > w.ext) ? (key << 16) | (inv0 - (uint32_t)e) : 0u;
  }
  if (ballot(valid && nan)) w.flags |= kNan;
  if (ballot(valid && ninf)) w.flags |= kNinf;
  sort8_desc(c);
  // each lane's values are descending and the k-th only rises: once no lane
  // beats it at some position, no later position can
#pragma unroll 1
  for (int p = 0; p < 8; ++p) {
    const uint64_t m = lanes_ugt(c[0], w.kth);
    if (!m) break;
    offer(w, c[0], m);
    c[0] = c[1]; c[1] = c[2]; c[2] = c[3]; c[3] = c[4]; c[4] = c[5]; c[5] = c[6]; c[6] = c[7];
  }
}

// Exact path for one 16-byte vector per lane when few lanes trip: the eight
// per-element tests against T on the raw bits (lanes `valid`; a conservative
// pre-test, since T only rises), then for each element position with hits the
// composites of all lanes at once and one insertion per hit.  NONNEG selects
// the filter form: for T >= 0 only non-negative bit patterns can pass, whose
// key is bits + 0x8000.  NaN patterns that pass are flagged, never kept.
// inv0 = 0xFFFF - rel of this lane's element 0.
template <bool NONNEG>
__device__ __forceinline__ void take_lanes_value(WaveTopK &w, uint4 d, uint32_t inv0, uint64_t valid, const Filter &f) {
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
  uint64_t m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t word = dw[e >> 1];
    const uint32_t b = (e & 1) ? word >> 16 : word & 0xFFFFu;
    m[e] = (NONNEG ? lanes_sgt((int32_t)(int16_t)b, f.t16) : lanes_ult(b, f.tu)) & valid;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (!m[e]) continue;
    const uint32_t word = dw[e >> 1];
    const uint32_t b = (e & 1) ? word >> 16 : word & 0xFFFFu;
    const uint32_t key = NONNEG ? (b > w.inf ? 0u : b | 0x8000u) : order_key(b, w.inf);
    if (m[e] & lanes_eq(key, 0u)) w.flags |= kNan;
    const uint32_t c = key ? (key << 16) | (inv0 - (uint32_t)e) : 0u;
    uint64_t h = m[e] & lanes_ugt(c, w.kth);
    while (h) {  // against a stale k-th: see offer
      const int l = __builtin_ctzll(h);
      h &= h - 1;
      w.list = insert_one(w.list, readlane(c, l));
    }
  }
  w.kth = readlane(w.list, w.km1);
}

constexpr int kDenseLanes = 16;  // this many tripping lanes pick the dense path

// Exact path for columns [lo, hi) one per lane (row edges and tiny spans).
__device__ void take_columns(WaveTopK &w, const uint16_t *row, int64_t lo, int64_t hi, int64_t base) {
  for (int64_t c0 = lo; c0 < hi; c0 += kWave) {
    const int64_t col = c0 + lane_id();
    const bool valid = col < hi;
    const uint32_t b = valid ? (uint32_t)row[col] : 0u;
    const uint32_t key = order_key(b, w.inf);
    if (ballot(valid && (b & 0x7FFFu) > w.inf)) w.flags |= kNan;
    if (ballot(valid && b == (0x8000u | w.inf))) w.flags |= kNinf;
    const uint32_t c = (valid && key > w.ext) ? (key << 16) | (0xFFFFu - (uint32_t)(col - base)) : 0u;
    const uint64_t m = lanes_ugt(c, w.kth);
    if (m) offer(w, c, m);
  }
}

// One chunk of kChunkVecs vectors per lane.  Vector u of this lane is the
// wave's vector (first + u * 64 + lane); lanes whose vector lies at or past
// nvec read zeros (the buffer's range check) and are masked out of the exact
// path.  Trip bits are taken once against the thresholds at the chunk start:
// the thresholds only rise while the chunk is processed, so a lane that did
// not trip then cannot hold anything that matters later.
__device__ __forceinline__ void take_chunk(WaveTopK &w, const uint4 (&v)[kChunkVecs], uint32_t first, uint32_t nvec,
                                           int64_t col_first, int64_t base) {
  w.ext = max(shared_bound(w.tau, w.wave), w.floor);
  const Filter f0 = make_filter(w);
  uint64_t vt[kChunkVecs], ft[kChunkVecs];
  lane_trips<kChunkVecs>(v, f0, vt, ft);
  static_assert(kChunkVecs == 4, "rotation below");
  if (!(vt[0] | vt[1] | vt[2] | vt[3] | ft[0] | ft[1] | ft[2] | ft[3])) return;
  const uint32_t l = (uint32_t)lane_id();
  uint4 x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];  // rotated once per vector below
  // 0xFFFF - rel of element 0 of this lane's vector (first + l)
  uint32_t inv0 = 0xFFFFu - (uint32_t)(col_first - base) - (uint32_t)kVecElems * (first + l);
  uint32_t vi = first + l;
#pragma unroll 1
  for (int u = 0; u < kChunkVecs; ++u) {
    const uint64_t valid = lanes_ult(vi, nvec);
    const uint64_t mv = vt[0] & valid, mf = ft[0] & valid;
    if (mv | mf) {
      const uint4 d = x0;
      if (__popcll(mv | mf) >= kDenseLanes) {
        take_vector_dense(w, d, inv0, vi < nvec);
        // the young set just grew a lot: share it and take the others' news
        publish(w.tau, w.wave, w);
        w.ext = max(shared_bound(w.tau, w.wave), w.floor);
      } else {
        if (mf) take_flags(w.flags, w.inf, d, mf, f0.ftrip);
        if (mv) {
          const Filter f = make_filter(w);
          if (f.nonneg) take_lanes_value<true>(w, d, inv0, mv, f);
          else take_lanes_value<false>(w, d, inv0, mv, f);
        }
      }
    }
    vt[0] = vt[1];
    vt[1] = vt[2];
    vt[2] = vt[3];
    vt[3] = 0;
    ft[0] = ft[1];
    ft[1] = ft[2];
    ft[2] = ft[3];
    ft[3] = 0;
    if (!(vt[0] | vt[1] | vt[2] | ft[0] | ft[1] | ft[2])) break;
    x0 = x1;
    x1 = x2;
    x2 = x3;
    inv0 -= (uint32_t)(kWave * kVecElems);
    vi += (uint32_t)kWave;
  }
  publish(w.tau, w.wave, w);
}

// Streams nvec 16-byte vectors starting at vp (its first element is column
// col_first), two chunks in flight.  A holds the first chunk, already loaded.
__device__ __forceinline__ void take_body(WaveTopK &w, const uint4 *vp, uint32_t nvec, int64_t col_first,
                                          int64_t base, uint4 (&A)[kChunkVecs]) {
  constexpr uint32_t kStep = (uint32_t)kChunkVecs * kWave;  // vectors per chunk
  const uint32_t lane_off = (uint32_t)lane_id() * 16u;
  uint4 B[kChunkVecs];
  // Issue priority falls with progress (3 in the first half of the share, 2
  // to three quarters, 1 to nine tenths, 0 after): a SIMD otherwise favours
  // its oldest waves, which then run ahead while the youngest lag, and the
  // kernel ends in a tail with too few waves left to keep HBM busy.  Waves
  // that are behind now issue first.  (Steps at 1/4, 1/2, 3/4 measured 0.5 us
  // slower on 1024 x 151936 rows; at 7/10, 17/20, 19/20, 2 us slower.)
  const uint32_t q1 = nvec / 2, q2 = nvec - nvec / 4, q3 = nvec - nvec / 10;
  __builtin_amdgcn_s_setprio(3);
  for (uint32_t first = 0; first < nvec; first += 2 * kStep) {
    if (first >= q3) __builtin_amdgcn_s_setprio(0);
    else if (first >= q2) __builtin_amdgcn_s_setprio(1);
    else if (first >= q1) __builtin_amdgcn_s_setprio(2);
    load_chunk(B, vp, nvec, first + kStep, lane_off);
    take_chunk(w, A, first, nvec, col_first, base);
    if (first + kStep >= nvec) break;
    load_chunk(A, vp, nvec, first + 2 * kStep, lane_off);
    take_chunk(w, B, first + kStep, nvec, col_first, base);
  }
}

// A floor from the end of a wave's share, for rows that rise along it: there
// every vector would beat the list before it and take the exact path.  The
// k-th largest lane maximum of the share's last chunk's worth of vectors (its
// final 256, so that every lane holds four) is reached by k elements of the
// share, so no key below it can be among the wave's k best (equal keys pass:
// a lower column may win).  Those vectors are read here for their maxima
// only; their elements are taken in column order when the scan gets there.
// A wave asks for it when nearly every lane of its first chunk has its
// largest key in its last vector (a lane's vectors lie 64 apart, so a rising
// share puts every lane's maximum there; evenly spread data puts about a
// quarter of them there).
__device__ __forceinline__ uint32_t lookahead_floor(const uint4 *vp, uint32_t nvec, uint32_t lane_off, uint32_t inf,
                                                    int km1) {
  constexpr uint32_t kStep = (uint32_t)kChunkVecs * kWave;
  const uint32_t last = nvec - kStep;  // the share's last kStep vectors: every lane holds four
  uint4 L[kChunkVecs];
  load_chunk(L, vp, nvec, last, lane_off);
  const uint32_t top = sort64_desc(lane_max_key(L, last, nvec, inf), make_xchg());
  const uint32_t te = readlane(top, km1);
  return te > 1 ? te - 1 : 0u;
}

// Fused merge of a split row.  Every scan workgroup of row r has written its
// span list; the last one to arrive folds all S lists into the row's outputs,
// with the order and rules of span_merge_kernel, and resets the row's counter
// to zero for the next call on the stream.  The lists, counts and flags are
// written and read with agent-scope atomic accesses, which bypass the
// non-coherent cache levels (each XCD has its own L2), so no cache writeback
// or invalidation is needed: a workgroup waits until its stores have
// completed, then counts its arrival; the last arrival reads every list.
__device__ __forceinline__ void fold_row_if_last(const ScanArgs &a, int64_t r, int S, const uint16_t *row, int wave,
                                              int l) {
  __shared__ int s_last;
  __shared__ uint64_t s_acc[kWgWaves][kWave];
  __shared__ int32_t s_cnt[kWgWaves];
  __shared__ uint32_t s_fl[kWgWaves];
  const int64_t rb = r - a.row0;  // the row's counter within this launch
  __builtin_amdgcn_s_waitcnt(0);  // this wave's list stores have completed
  __syncthreads();
  TK_STAMP(8);
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&a.row_done[rb], 1, __ATOMIC_RELAXED, kAgent) == S - 1;
  __syncthreads();
  TK_STAMP(9);
  if (!s_last) return;
  TK_STAMP_VALUE(13, 1);
  const Xchg x = make_xchg();
  uint64_t acc = 0;
  int cnt = 0;
  uint32_t fl = 0;
  // each wave folds lists wave, wave + 4, ...; four lists' loads in flight at once
  for (int i0 = wave; i0 < S; i0 += 4 * kWgWaves) {
    uint64_t v[4];
    int c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j * kWgWaves;
      const int64_t sb = r * S + i;
      c[j] = 0;
      v[j] = 0;
      if (i < S) {
        c[j] = __hip_atomic_load(&a.span_count[sb], __ATOMIC_RELAXED, kAgent);
        fl |= __hip_atomic_load(&a.span_flags[sb], __ATOMIC_RELAXED, kAgent);
        if (l < a.k) v[j] = __hip_atomic_load(&a.span_list[sb * a.k + l], __ATOMIC_RELAXED, kAgent);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (i0 + j * kWgWaves >= S) break;
      const uint64_t vj = l < c[j] ? v[j] : 0;
      acc = (i0 == wave && j == 0) ? vj : merge_sorted64(acc, vj, x);
      cnt += c[j];
    }
  }
  s_acc[wave][l] = acc;
  if (l == 0) {
    s_cnt[wave] = cnt;
    s_fl[wave] = fl;
  }
  __syncthreads();
  TK_STAMP(10);
  // the waves' results as a tree: 0 and 2 take 1 and 3, then 0 takes 2
  if ((wave & 1) == 0) {
    acc = merge_sorted64(acc, s_acc[wave + 1][l], x);
    cnt += s_cnt[wave + 1];
    fl |= s_fl[wave + 1];
  }
  if (wave == 2) {
    s_acc[2][l] = acc;
    if (l == 0) {
      s_cnt[2] = cnt;
      s_fl[2] = fl;
    }
  }
  __syncthreads();
  if (wave == 0) {
    acc = merge_sorted64(acc, s_acc[2][l], x);
    cnt += s_cnt[2];
    fl |= s_fl[2];
    TK_STAMP(11);
    const int k = a.k;
    if (cnt > k) cnt = k;
    const int64_t ob = r * k;
    if (l < k) {
      if (l < cnt) {
        a.out_idx[ob + l] = (int32_t)(col_of(acc) + a.col_base);
        a.out_val[ob + l] = value_bits(acc, row);
      } else {
        a.out_idx[ob + l] = TK_FILL_IDX;
        a.out_val[ob + l] = (uint16_t)TK_FILL_VAL;
      }
    }
    if (l == 0) {
      a.out_count[r] = cnt;
      a.out_nonfinite[r] = fl;
      __hip_atomic_store(&a.row_done[rb], 0, __ATOMIC_RELAXED, kAgent);
    }
    TK_STAMP(12);
  }
}

__global__ __launch_bounds__(kWgThreads) void span_scan_kernel(ScanArgs a) {
  __shared__ uint64_t s_list[kWgWaves][kWave];
  __shared__ int32_t s_count[kWgWaves];
  __shared__ uint32_t s_flags[kWgWaves];
  __shared__ uint32_t s_tau[2 * kWgWaves];
  __shared__ uint32_t s_samp[kWgWaves][kWave];

  const int64_t blk = blockIdx.x;
  const int64_t r = a.row0 + blk / a.spans;
  const int s = (int)(blk % a.spans);
  const int S = a.spans;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));  // uniform per wave
  const int l = lane_id();
  const uint16_t *row = a.in + r * a.stride;
  TK_STAMP(0);
  TK_STAMP_HW(14);
  TK_STAMP_VALUE(13, 0);

  // The row's 16-byte grid: vector j covers columns [a0 + 8j, a0 + 8j + 8).
  const int64_t a0 = (int64_t)((8u - (uint32_t)(((uintptr_t)row >> 1) & 7u)) & 7u);
  const int64_t nv_row = a.cols > a0 ? (a.cols - a0) / kVecElems : 0;
  int64_t j0 = 0, j1 = 0, head_lo = 0, head_hi = 0, tail_lo = 0, tail_hi = 0;
  if (nv_row > 0) {
    j0 = nv_row * s / S;
    j1 = nv_row * (s + 1) / S;
    if (s == 0) head_hi = a0;
    if (s == S - 1) {
      tail_lo = a0 + kVecElems * nv_row;
      tail_hi = a.cols;
    }
  } else if (s == 0) {
    head_hi = a.cols;
  }
  const int64_t n = j1 - j0;
  const int64_t wv0 = j0 + n * wave / kWgWaves;
  const int64_t wv1 = j0 + n * (wave + 1) / kWgWaves;
  const int64_t base = (wave == 0 && head_hi > head_lo) ? head_lo : a0 + kVecElems * wv0;

  // Floors from a sample: the first chunk of each wave, loaded here and handed
  // on to take_body.  Each wave sorts its 64 per-lane maximum keys; every wave
  // then merges the four sorted lists into the top 64 of the 256 (the same
  // result in every wave).  Two floors follow:
  //  - exact: the k-th largest lane maximum T has k elements (one per lane) at
  //    or above it, so no key below T can be among the top k of the span; only
  //    keys >= T are kept.  This spares young lists most of their filling.
  //  - speculative (rank j = spec_rank < k, chosen on the host from k and the
  //    span width, and only when every wave's share spans at least kSpecChunks
  //    chunks): the j-th largest lane maximum, about the sample's j-th largest
  //    key.  The result is verified: if the lists end with k entries (all
  //    above that floor), every dropped element is beaten by k kept ones and
  //    the answer is exact; otherwise the span is scanned again under the
  //    exact floor, which the choice of j makes rare.
  uint32_t exact_floor = 0, spec_floor = 0;
  const uint4 *wvp = reinterpret_cast<const uint4 *>(row + a0) + wv0;
  const uint32_t wn = (uint32_t)(wv1 - wv0);
  uint4 A[kChunkVecs];
  if (wn > 0) load_chunk(A, wvp, wn, 0, (uint32_t)l * 16u);
  const bool speculate =
      a.spec_rank > 0 && !a.exact && n / kWgWaves >= (int64_t)kSpecChunks * kChunkVecs * kWave;
  const uint32_t lm = wn == 0 ? 0u : S > 1 ? lane_max_key(A, 0, wn, a.inf) : lane_max_key_keys(A, 0, wn, a.inf);
  {
    const Xchg x = make_xchg();
    s_samp[wave][l] = sort64_desc(lm, x);
    __syncthreads();
    uint32_t v[kWgWaves];  // pairwise tree of the sorted lists: the top 64 of all
#pragma unroll
    for (int o = 0; o < kWgWaves; ++o) v[o] = s_samp[o][l];
#pragma unroll
    for (int step = 1; step < kWgWaves; step *= 2)
#pragma unroll
      for (int o = 0; o + step < kWgWaves; o += 2 * step)
        v[o] = bitonic_merge64_desc(max(v[o], partner<63>(v[o + step], x)), x);
    const uint32_t top = v[0];
    const uint32_t te = readlane(top, a.k - 1);
    const uint32_t ts = speculate ? readlane(top, a.spec_rank - 1) : 0u;
    exact_floor = te > 0 ? te - 1 : 0;
    spec_floor = ts > 0 ? ts - 1 : 0;
  }
  // Rows that rise along this wave's share: a floor of the wave's own from the
  // share's end.  It is exact, so it also holds when the speculation fails;
  // the choice to speculate (and so the rescan loop below) stays the same in
  // every wave of the workgroup.
  uint32_t rise_floor = 0;
  if (wn >= (uint32_t)(kLookChunks * kChunkVecs * kWave)) {
    const uint32_t l3 = vec_max_key(A[kChunkVecs - 1], a.inf);
    if (__popcll(ballot(lm > 0 && l3 >= lm)) >= kLookLanes)
      rise_floor = lookahead_floor(wvp, wn, (uint32_t)l * 16u, a.inf, a.k - 1);
  }
  uint32_t floor = exact_floor;
  bool verify = false;
  if (spec_floor > exact_floor) {
    floor = spec_floor;
    verify = true;
  }
  floor = max(floor, rise_floor);
  TK_STAMP(1);

  int total = 0;
  uint32_t flags = 0;
  for (;;) {
    if (threadIdx.x < 2 * kWgWaves) s_tau[threadIdx.x] = 0;
    __syncthreads();
    WaveTopK w;
    w.list = 0;
    w.kth = 0;
    w.ext = floor;
    w.floor = floor;
    w.flags = 0;
    w.inf = a.inf;
    w.km1 = a.k - 1;
    w.qm1 = (a.k + kWgWaves - 1) / kWgWaves - 1;
    w.wave = wave;
    w.tau = s_tau;
    w.x = make_xchg();

    if (wave == 0 && head_hi > head_lo) take_columns(w, row, head_lo, head_hi, base);
    if (wn > 0) take_body(w, wvp, wn, a0 + kVecElems * wv0, base, A);
    if (wave == kWgWaves - 1 && tail_hi > tail_lo) take_columns(w, row, tail_lo, tail_hi, base);
    TK_WAVE_STAMP(2 + wave);

    // publish this wave's list
    const uint64_t valid_mask = ballot(w.list != 0);
    s_list[wave][l] = composite64(w.list, base);
    if (l == 0) {
      const int cnt = __popcll(valid_mask);
      s_count[wave] = cnt < a.k ? cnt : a.k;
      s_flags[wave] = w.flags | ((readlane(w.list, 0) >> 16) == 0x8000u + a.inf ? kPinf : 0u);
    }
    __syncthreads();
    TK_STAMP(6);

    total = 0;
    flags = 0;
#pragma unroll
    for (int o = 0; o < kWgWaves; ++o) {
      total += s_count[o];
      flags |= s_flags[o];
    }
    if (!verify || total >= a.k) break;  // exact, or the speculation verified
    // too few entries reach the speculative floor: scan again under the exact one
    floor = max(exact_floor, rise_floor);
    verify = false;
    if (wn > 0) load_chunk(A, wvp, wn, 0, (uint32_t)l * 16u);
    __syncthreads();  // every wave has read the counts above
  }
  if (total > a.k) total = a.k;

  // The four wave lists meet as a tree in registers: waves 0 and 2 merge
  // their list with the next wave's, then wave 0 merges in wave 2's result.
  // A wave's entries past its count (beaten by k of its own, or empty
  // zeros) can only land at merged ranks >= k, so whole lists are merged.
  const Xchg xm = make_xchg();
  uint64_t acc = s_list[wave][l];
  if ((wave & 1) == 0) acc = merge_sorted64(acc, s_list[wave + 1][l], xm);
  if (wave == 2) s_list[2][l] = acc;  // wave 0 does not read its own slot's partner until after the barrier
  __syncthreads();
  if (wave == 0) {
    acc = merge_sorted64(acc, s_list[2][l], xm);
    if (S == 1) {
      const int64_t ob = r * a.k;
      if (l < total) {
        a.out_idx[ob + l] = (int32_t)(col_of(acc) + a.col_base);
        a.out_val[ob + l] = value_bits(acc, row);
      } else if (l < a.k) {
        a.out_idx[ob + l] = TK_FILL_IDX;
        a.out_val[ob + l] = (uint16_t)TK_FILL_VAL;
      }
      if (l == 0) {
        a.out_count[r] = total;
        a.out_nonfinite[r] = flags;
      }
    } else {
      // agent-scope stores: coherent across the XCDs' caches (see fold_row_if_last)
      const int64_t sb = r * S + s;
      if (l < total) __hip_atomic_store(&a.span_list[sb * a.k + l], acc, __ATOMIC_RELAXED, kAgent);
      if (l == 0) {
        __hip_atomic_store(&a.span_count[sb], total, __ATOMIC_RELAXED, kAgent);
        __hip_atomic_store(&a.span_flags[sb], flags, __ATOMIC_RELAXED, kAgent);
      }
    }
    TK_STAMP(7);
  }
  if (S > 1 && a.row_done) fold_row_if_last(a, r, S, row, wave, l);
}

// ---------------------------------------------------------------------------
// k = 1: the row's best entry alone (greedy decoding takes this argmax).  The
// same span split, loads and raw-bit filter as span_scan_kernel, with the
// kept list reduced to one wave-uniform composite: T = max(the wave's best
// key, the bound from the other waves' best keys), an element matters only if
// its key exceeds T, and a tripped chunk costs one per-lane maximum of the
// tripping vectors' composites and one wave-wide maximum.  No floors, no list
// merges: a split row keeps one composite per span, and the row's last
// workgroup takes the maximum of its S <= kMergeGroup span results.

struct WaveArgmax {
  uint32_t best;    // wave-uniform best in-wave composite (key << 16 | 0xFFFF - rel), 0 = none
  uint32_t flags;   // wave-uniform TK_NONFINITE_NAN / _NEGINF seen so far
  uint32_t inf;     // +inf pattern of the input format
  int wave;
  uint32_t *s_key;  // LDS: best key published by each wave of the workgroup
  Xchg x;
};

__device__ __forceinline__ uint32_t wave_max(uint32_t v, const Xchg &x) {
  v = max(v, partner<1>(v, x));
  v = max(v, partner<2>(v, x));
  v = max(v, partner<4>(v, x));
  v = max(v, partner<8>(v, x));
  v = max(v, partner<16>(v, x));
  v = max(v, partner<32>(v, x));
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ uint64_t wave_max64(uint64_t v, const Xchg &x) {
  uint64_t y;
  y = partner64<1>(v, x); v = v > y ? v : y;
  y = partner64<2>(v, x); v = v > y ? v : y;
  y = partner64<4>(v, x); v = v > y ? v : y;
  y = partner64<8>(v, x); v = v > y ? v : y;
  y = partner64<16>(v, x); v = v > y ? v : y;
  y = partner64<32>(v, x); v = v > y ? v : y;
  return v;
}

// Keys at or below this bound lose to another wave's best: to a wave on the
// left (lower columns) also on equal keys, to a wave on the right only on
// lower ones.  Published keys only rise, so a stale read is still a bound.
__device__ __forceinline__ uint32_t argmax_bound(const WaveArgmax &w) {
  uint32_t ext = 0;
#pragma unroll
  for (int o = 0; o < kWgWaves; ++o) {
    if (o == w.wave) continue;
    const uint32_t t = __hip_atomic_load(&w.s_key[o], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    ext = max(ext, o < w.wave ? t : (t > 0 ? t - 1 : 0u));
  }
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)ext);
}

// This lane's best composite among the eight elements of d (element e at
// 0xFFFF - rel = inv0 - e); NaN gives 0 and sets nan.  On equal keys the
// lower column has the larger composite.  (Positive NaN patterns reach this
// path through the value trip, whose int16 test they always pass; the flag
// trip only sees patterns from -inf upwards as uint16.)
__device__ __forceinline__ uint32_t vector_best(uint4 d, uint32_t inv0, uint32_t inf, bool &nan) {
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t b = (dw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
    const uint32_t key = order_key(b, inf);
    nan |= key == 0;
    m = max(m, key ? (key << 16) | (inv0 - (uint32_t)e) : 0u);
  }
  return m;
}

// One chunk (as take_chunk): trip bits against T at the chunk start, then the
// tripping lanes' vector maxima and one wave maximum.
__device__ __forceinline__ void argmax_chunk(WaveArgmax &w, const uint4 (&v)[kChunkVecs], uint32_t first,
                                             uint32_t nvec, int64_t col_first, int64_t base) {
  const Filter f = filter_for(max(w.best >> 16, argmax_bound(w)), w.flags, w.inf);
  uint64_t vt[kChunkVecs], ft[kChunkVecs];
  lane_trips<kChunkVecs>(v, f, vt, ft);
  uint64_t any_v = 0, any_f = 0;
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    const uint64_t valid = lanes_ult(first + (uint32_t)(u * kWave + lane_id()), nvec);
    vt[u] &= valid;
    ft[u] &= valid;
    any_v |= vt[u];
    any_f |= ft[u];
  }
  if (any_f) {
#pragma unroll
    for (int u = 0; u < kChunkVecs; ++u)
      if (ft[u]) take_flags(w.flags, w.inf, v[u], ft[u], f.ftrip);
  }
  if (!any_v) return;
  const uint32_t l = (uint32_t)lane_id();
  const uint32_t inv0 = 0xFFFFu - (uint32_t)(col_first - base) - (uint32_t)kVecElems * (first + l);
  uint32_t m = 0;
  bool nan = false;
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u)
    if ((vt[u] >> l) & 1u) m = max(m, vector_best(v[u], inv0 - (uint32_t)(u * kWave * kVecElems), w.inf, nan));
  if (ballot(nan)) w.flags |= kNan;
  const uint32_t best = max(w.best, wave_max(m, w.x));
  if (best != w.best) {
    w.best = best;
    if (l == 0) __hip_atomic_store(&w.s_key[w.wave], best >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// Columns [lo, hi) one per lane (row edges, tiny spans): every element.
__device__ void argmax_columns(WaveArgmax &w, const uint16_t *row, int64_t lo, int64_t hi, int64_t base) {
  uint32_t m = 0;
  for (int64_t c0 = lo; c0 < hi; c0 += kWave) {
    const int64_t col = c0 + lane_id();
    const bool valid = col < hi;
    const uint32_t b = valid ? (uint32_t)row[col] : 0u;
    const uint32_t key = valid ? order_key(b, w.inf) : 0u;
    if (ballot(valid && (b & 0x7FFFu) > w.inf)) w.flags |= kNan;
    if (ballot(valid && b == (0x8000u | w.inf))) w.flags |= kNinf;
    m = max(m, key ? (key << 16) | (0xFFFFu - (uint32_t)(col - base)) : 0u);
  }
  w.best = max(w.best, wave_max(m, w.x));
}

__global__ __launch_bounds__(kWgThreads) void argmax_scan_kernel(ArgmaxArgs a) {
  __shared__ uint32_t s_key[kWgWaves];
  __shared__ uint64_t s_best[kWgWaves];
  __shared__ uint32_t s_fl[kWgWaves];

  const int64_t blk = blockIdx.x;
  const int64_t r = a.row0 + blk / a.spans;
  const int s = (int)(blk % a.spans);
  const int S = a.spans;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int l = lane_id();
  const uint16_t *row = a.in + r * a.stride;

  // the span and wave shares of span_scan_kernel
  const int64_t a0 = (int64_t)((8u - (uint32_t)(((uintptr_t)row >> 1) & 7u)) & 7u);
  const int64_t nv_row = a.cols > a0 ? (a.cols - a0) / kVecElems : 0;
  int64_t j0 = 0, j1 = 0, head_hi = 0, tail_lo = 0, tail_hi = 0;
  if (nv_row > 0) {
    j0 = nv_row * s / S;
    j1 = nv_row * (s + 1) / S;
    if (s == 0) head_hi = a0;
    if (s == S - 1) {
      tail_lo = a0 + kVecElems * nv_row;
      tail_hi = a.cols;
    }
  } else if (s == 0) {
    head_hi = a.cols;
  }
  const int64_t n = j1 - j0;
  const int64_t wv0 = j0 + n * wave / kWgWaves;
  const int64_t wv1 = j0 + n * (wave + 1) / kWgWaves;
  const int64_t base = (wave == 0 && head_hi > 0) ? 0 : a0 + kVecElems * wv0;

  if (threadIdx.x < kWgWaves) s_key[threadIdx.x] = 0;
  __syncthreads();
  WaveArgmax w;
  w.best = 0;
  w.flags = 0;
  w.inf = a.inf;
  w.wave = wave;
  w.s_key = s_key;
  w.x = make_xchg();

  if (wave == 0 && head_hi > 0) argmax_columns(w, row, 0, head_hi, base);
  const uint4 *vp = reinterpret_cast<const uint4 *>(row + a0) + wv0;
  const uint32_t nvec = (uint32_t)(wv1 - wv0);
  if (nvec > 0) {
    constexpr uint32_t kStep = (uint32_t)kChunkVecs * kWave;
    const uint32_t lane_off = (uint32_t)l * 16u;
    const int64_t col_first = a0 + kVecElems * wv0;
    uint4 A[kChunkVecs], B[kChunkVecs];
    load_chunk(A, vp, nvec, 0, lane_off);
    for (uint32_t first = 0; first < nvec; first += 2 * kStep) {
      load_chunk(B, vp, nvec, first + kStep, lane_off);
      argmax_chunk(w, A, first, nvec, col_first, base);
      if (first + kStep >= nvec) break;
      load_chunk(A, vp, nvec, first + 2 * kStep, lane_off);
      argmax_chunk(w, B, first + kStep, nvec, col_first, base);
    }
  }
  if (wave == kWgWaves - 1 && tail_hi > tail_lo) argmax_columns(w, row, tail_lo, tail_hi, base);

  if (l == 0) {
    s_best[wave] = composite64(w.best, base);
    s_fl[wave] = w.flags;
  }
  __syncthreads();
  if (wave != 0) return;
  uint64_t best = 0;
  uint32_t fl = 0;
#pragma unroll
  for (int o = 0; o < kWgWaves; ++o) {
    best = best > s_best[o] ? best : s_best[o];
    fl |= s_fl[o];
  }
  if (S > 1) {
    // span result to its slot (flags in bits 48..50), then the arrival count;
    // the last workgroup of the row takes the maximum of all slots
    const int64_t rb = r - a.row0;
    if (l == 0) __hip_atomic_store(&a.span_slot[rb * S + s], best | ((uint64_t)fl << 48), __ATOMIC_RELAXED, kAgent);
    __builtin_amdgcn_s_waitcnt(0);
    int last = 0;
    if (l == 0) last = __hip_atomic_fetch_add(&a.row_done[rb], 1, __ATOMIC_RELAXED, kAgent) == S - 1;
    if (!ballot(last)) return;
    const uint64_t v = l < S ? __hip_atomic_load(&a.span_slot[rb * S + l], __ATOMIC_RELAXED, kAgent) : 0;
    const uint32_t f = (uint32_t)(v >> 48);
    fl = (ballot(f & kNan) ? kNan : 0u) | (ballot(f & kNinf) ? kNinf : 0u);
    best = wave_max64(v & 0x0000FFFFFFFFFFFFull, make_xchg());
    if (l == 0) __hip_atomic_store(&a.row_done[rb], 0, __ATOMIC_RELAXED, kAgent);
  }
  if (l == 0) {
    if ((uint32_t)(best >> 32) == 0x8000u + a.inf) fl |= kPinf;
    if (best) {
      a.out_idx[r] = (int32_t)(col_of(best) + a.col_base);
      a.out_val[r] = value_bits(best, row);
    } else {
      a.out_idx[r] = TK_FILL_IDX;
      a.out_val[r] = (uint16_t)TK_FILL_VAL;
    }
    a.out_count[r] = best ? 1 : 0;
    a.out_nonfinite[r] = fl;
  }
}

// Folds up to kMergeGroup sorted candidate lists of one row into one.  Each
// wave loads its share of the lists straight into registers (lane j holds
// entry j; every load in flight at once) and folds them pairwise with bitonic
// merges of the 64-bit composites -- the same (score desc, column asc) order
// as the scan; the waves' results then meet in a tree through LDS.
// WAVES = 16 folds up to kMergeGroup lists, WAVES = 8 or 4 up to a half or a
// quarter of that (four lists per wave; launch_span_merge picks the smallest
// workgroup that holds the group).  WAVES is a power of two for the tree.
template <int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void span_merge_kernel(MergeArgs a) {
  static_assert((WAVES & (WAVES - 1)) == 0, "the waves' tree pairs wave i with i + w");
  constexpr int kWaves = WAVES;
  constexpr int kPerWave = kMergeGroup / (kMergeThreads / kWave);  // lists one wave folds
  static_assert(kMergeGroup % (kMergeThreads / kWave) == 0, "lists per wave");
  __shared__ uint64_t s_acc[kWaves][kWave];
  __shared__ int32_t s_cnt[kWaves];
  __shared__ uint32_t s_fl[kWaves];

  const int64_t blk = blockIdx.x;
  const int64_t r = a.row0 + blk / a.lists_out;
  const int g = (int)(blk % a.lists_out);
  const int first = g * a.group;
  int n = a.lists_in - first;
  if (n > a.group) n = a.group;
  const int k = a.k;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int l = lane_id();
  const Xchg x = make_xchg();
  const int64_t in_base = r * a.lists_in + first;

  uint64_t v[kPerWave];
  int c[kPerWave];
  uint32_t fl = 0;
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int li = wave + j * kWaves;
    c[j] = 0;
    v[j] = 0;
    if (li < n) {
      c[j] = __builtin_amdgcn_readfirstlane(a.count_in[in_base + li]);
      fl |= a.flags_in[in_base + li];
      if (l < k) v[j] = a.list_in[(in_base + li) * k + l];
    }
  }
  // empty lists (pruned spans of the fused head) are skipped
  uint64_t acc = 0;
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    if (!c[j]) continue;
    const uint64_t vj = l < c[j] ? v[j] : 0;
    acc = cnt == 0 ? vj : merge_sorted64(acc, vj, x);
    cnt += c[j];
  }

  // the waves' results meet as a tree: at step w, wave i (a multiple of 2w)
  // takes the merge of its result and wave i + w's
  s_acc[wave][l] = acc;
  if (l == 0) {
    s_cnt[wave] = cnt;
    s_fl[wave] = fl;
  }
#pragma unroll
  for (int w = 1; w < kWaves; w *= 2) {
    __syncthreads();
    if ((wave & (2 * w - 1)) == 0) {
      const int other = __builtin_amdgcn_readfirstlane(s_cnt[wave + w]);
      if (other) acc = cnt ? merge_sorted64(acc, s_acc[wave + w][l], x) : s_acc[wave + w][l];
      cnt += other;
      fl |= s_fl[wave + w];
      s_acc[wave][l] = acc;
      if (l == 0) {
        s_cnt[wave] = cnt;
        s_fl[wave] = fl;
      }
    }
  }
  if (wave != 0) return;
  if (cnt > k) cnt = k;
  const uint32_t flags = fl;

  if (a.lists_out == 1) {
    const int64_t ob = r * k;
    if (l < k) {
      if (l < cnt && a.in) {
        a.out_idx[ob + l] = (int32_t)(col_of(acc) + a.col_base);
        a.out_val[ob + l] = value_bits(acc, a.in + r * a.stride);
      } else if (l < cnt) {
        a.out_idx[ob + l] = (int32_t)(signed_col(acc) + a.col_base);
        a.out_val[ob + l] = signed_value_bits(acc);
      } else {
        a.out_idx[ob + l] = TK_FILL_IDX;
        a.out_val[ob + l] = (uint16_t)TK_FILL_VAL;
      }
    }
    if (l == 0) {
      a.out_count[r] = cnt;
      a.out_nonfinite[r] = flags;
    }
    if (a.sketch && l < k) a.sketch[r * k + l] = 0;  // zero again for the next call on the stream
  } else {
    const int64_t ob = r * a.lists_out + g;
    if (l < cnt) a.list_out[ob * k + l] = acc;
    if (l == 0) {
      a.count_out[ob] = cnt;
      a.flags_out[ob] = flags;
    }
  }
}

}  // namespace

// Merge of per-shard results (vocabulary-sharded top-k): one wave per row
// folds the row's entry lists of all shards with the same bitonic merges.
// Entries carry global column indices and their own bf16 bits, so the
// composite is key << 32 | (0x7FFFFFFF - idx) << 1 | sign bit: the same (score
// desc, index asc) order for indices below 2^31, with the sign of a zero
// carried along (its key does not tell +0 from -0).
__device__ __forceinline__ uint64_t shard_composite(uint32_t val, int32_t idx) {
  return ((uint64_t)order_key(val) << 32) | ((uint64_t)(0x7FFFFFFFu - (uint32_t)idx) << 1) | ((val >> 15) & 1u);
}

__global__ __launch_bounds__(kWgThreads) void shard_merge_kernel(ShardMergeArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int l = lane_id();
  const int64_t r = (int64_t)blockIdx.x * kWgWaves + wave;
  if (r >= a.rows) return;
  const Xchg x = make_xchg();
  const int k = a.k;
  uint64_t acc = 0;
  int cnt = 0;
  uint32_t fl = 0;
  // eight shards at a time, every load in flight at once: all k entries of a
  // shard's row are read (the inputs are dense [shards][rows][k]) and those
  // past its count, whatever they hold, are masked afterwards, so no load
  // waits on another
  constexpr int kShardBatch = 8;
  for (int g0 = 0; g0 < a.shards; g0 += kShardBatch) {
    uint32_t val[kShardBatch];
    int32_t idx[kShardBatch];
    int c[kShardBatch];
#pragma unroll
    for (int j = 0; j < kShardBatch; ++j) {
      const int g = g0 + j;
      c[j] = 0;
      val[j] = 0;
      idx[j] = 0;
      if (g < a.shards) {
        const int64_t sr = (int64_t)g * a.rows + r;
        c[j] = a.count_in[sr];
        fl |= a.mask_in[sr];
        if (l < k) {
          val[j] = a.val_in[sr * k + l];
          idx[j] = a.idx_in[sr * k + l];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kShardBatch; ++j) {
      if (g0 + j >= a.shards) break;
      const uint64_t v = l < c[j] && l < k ? shard_composite(val[j], idx[j]) : 0;
      acc = (g0 == 0 && j == 0) ? v : merge_sorted64(acc, v, x);
      cnt += c[j];
    }
  }
  if (cnt > k) cnt = k;
  const int64_t ob = r * k;
  if (l < k) {
    if (l < cnt) {
      a.out_idx[ob + l] = signed_col(acc);
      a.out_val[ob + l] = signed_value_bits(acc);
    } else {
      a.out_idx[ob + l] = TK_FILL_IDX;
      a.out_val[ob + l] = (uint16_t)TK_FILL_VAL;
    }
  }
  if (l == 0) {
    a.out_count[r] = cnt;
    a.out_nonfinite[r] = fl;
  }
}

hipError_t launch_shard_merge(const ShardMergeArgs &a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const int64_t blocks = (a.rows + kWgWaves - 1) / kWgWaves;
  hipLaunchKernelGGL(shard_merge_kernel, dim3((uint32_t)blocks), dim3(kWgThreads), 0, stream, a);
  return hipGetLastError();
}

// Measurement probe (not part of the top-k): streams nvec 16-byte vectors,
// split evenly over the grid's workgroups and each workgroup's four waves,
// with the scan's loads -- chunks of four nontemporal vectors per lane, two
// chunks in flight, range-checked descriptors -- and folds them with XOR.
// Nothing is written unless the fold hits a sentinel, so the loads cannot be
// dropped; with nvec = 0 the kernel is empty.  Its time is the floor any scan
// of those bytes with that grid can reach.
__global__ __launch_bounds__(kWgThreads) void read_probe_kernel(const uint4 *in, int64_t nvec, uint32_t *sink) {
  constexpr uint32_t kStep = (uint32_t)kChunkVecs * kWave;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t g = gridDim.x, b = blockIdx.x;
  const int64_t j0 = nvec * b / g, j1 = nvec * (b + 1) / g;
  const int64_t w0 = j0 + (j1 - j0) * wave / kWgWaves, w1 = j0 + (j1 - j0) * (wave + 1) / kWgWaves;
  const uint32_t wn = (uint32_t)(w1 - w0);
  uint32_t acc = 0;
  TK_STAMP(0);
  TK_STAMP_HW(14);
  auto fold = [&](const uint4 (&v)[kChunkVecs]) {
#pragma unroll
    for (int u = 0; u < kChunkVecs; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  };
  if (wn > 0) {
    const uint4 *vp = in + w0;
    const uint32_t lane_off = (uint32_t)lane_id() * 16u;
    uint4 A[kChunkVecs], B[kChunkVecs];
    load_chunk(A, vp, wn, 0, lane_off);
    for (uint32_t first = 0; first < wn; first += 2 * kStep) {
      load_chunk(B, vp, wn, first + kStep, lane_off);
      fold(A);
      if (first + kStep >= wn) break;
      load_chunk(A, vp, wn, first + 2 * kStep, lane_off);
      fold(B);
    }
  }
  if (acc == 0x9E3779B9u) sink[b & 8191] = acc;
  TK_WAVE_STAMP(2 + wave);  // after the last fold: every load of the wave has returned
}

hipError_t launch_read_probe(const void *in, int64_t nvec, int32_t workgroups, uint32_t *sink, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3((uint32_t)workgroups), dim3(kWgThreads), 0, stream,
                     (const uint4 *)in, nvec, sink);
  return hipGetLastError();
}

__global__ void zero_fill_kernel(int32_t *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_fill(int32_t *p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

// The fixed scratch of tk_topk_bf16_noalloc: one array per device, held
// until the process ends, for callers that cannot allocate.  Its first
// kFusedMaxRows int32 are the fused folds' arrival counters, which every
// call leaves at zero.  In host code `scratch` names a host-side stand-in,
// never device memory: kernels and fills get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kFixedScratchBytes];

namespace {
std::mutex g_fixed_mu;
void *g_fixed_ptr[kMaxDevices];
}  // namespace

hipError_t fixed_scratch(int dev, hipStream_t stream, void **ptr) {
  *ptr = nullptr;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_fixed_mu);
  if (!g_fixed_ptr[dev]) {
    // the caller has made `dev` current: this is that device's copy
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // device globals start zeroed; the fill makes the counters' zero state
    // explicit, ordered before this call's kernels on the caller's stream
    const hipError_t f = launch_zero_fill((int32_t *)p, kFusedMaxRows, stream);
    if (f != hipSuccess) return f;
    g_fixed_ptr[dev] = p;
  }
  *ptr = g_fixed_ptr[dev];
  return hipSuccess;
}

hipError_t launch_span_scan(const ScanArgs &a, int64_t rows_in_launch, hipStream_t stream) {
  const int64_t blocks = rows_in_launch * a.spans;
  hipLaunchKernelGGL(span_scan_kernel, dim3((uint32_t)blocks), dim3(kWgThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_argmax(const ArgmaxArgs &a, int64_t rows_in_launch, hipStream_t stream) {
  if (rows_in_launch <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_scan_kernel, dim3((uint32_t)(rows_in_launch * a.spans)), dim3(kWgThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_span_merge(const MergeArgs &a, int64_t rows_in_launch, hipStream_t stream) {
  const int64_t blocks = rows_in_launch * a.lists_out;
  constexpr int kPerWave = kMergeGroup / (kMergeThreads / kWave);
  if (a.group <= 4 * kPerWave)
    hipLaunchKernelGGL(span_merge_kernel<4>, dim3((uint32_t)blocks), dim3(4 * kWave), 0, stream, a);
  else if (a.group <= 8 * kPerWave)
    hipLaunchKernelGGL(span_merge_kernel<8>, dim3((uint32_t)blocks), dim3(8 * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL(span_merge_kernel<kMergeThreads / kWave>, dim3((uint32_t)blocks), dim3(kMergeThreads), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace tk

#ifdef TK_STAGE_STAMPS
// Copies the stage table of the last stamped launches (bytes at most its
// size); synchronous.  Present in the stamp build only.
extern "C" int tk_stage_stamps(void *dst, size_t bytes) {
  if (bytes > sizeof(tk_stamp_table)) return 1;
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(tk_stamp_table), bytes) == hipSuccess ? 0 : 1;
}
#endif
