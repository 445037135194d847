// Exact row-wise top-k of IEEE fp32 rows (gfx950): the same operation as the
// bf16 scan (TensorFold PR #713, change 3, and its Exactness table: score
// descending, lower column first on ties, NaN excluded and flagged,
// infinities ranked, zeros equal), for 32-bit logits.
//
// Order key.  An fp32 pattern b with magnitude m = b & 0x7FFFFFFF maps to
// 0x80000000 + m (sign clear) or 0x80000000 - m (sign set): monotone in value,
// +0 and -0 share 0x80000000, -inf -> 0x00800000, +inf -> 0xFF800000, NaN
// (m > 0x7F800000) -> 0, never kept.  Composites are 64-bit, key << 32 |
// (0xFFFFFFFF - column) with the absolute column, in the wave lists as in the
// span lists: a strict total order equal to (score desc, column asc), with
// no limit on the width one wave may scan.
//
// The scan follows the bf16 kernel's design (one workgroup = four wave64s per
// (row, span), a per-wave list of the 64 best composites in registers, one
// lane per entry, a raw-bit filter that skips vectors without a candidate,
// floors from a pooled first-chunk sample, thresholds shared in LDS, issue
// priority falling with progress, the four wave lists meeting as a tree of
// register merges, and the last workgroup of a split row folding the span
// lists), with four fp32 elements per 16-byte vector and 64-bit list
// entries.  Unlike the bf16 scan, candidates of the exact path collect in an
// LDS ring and enter the list in sorted batches (kRing32Flush).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tk_config.h"
#include "tk_launch.h"
#include "tk_topk.h"

namespace tk {
namespace {

#include "tk_wave.h"
#include "tk_lists.h"

constexpr int kElems32 = 4;  // fp32 per 16-byte vector
constexpr int kWideSpecChunks32 = 4;  // k > 64: a speculative floor needs this many chunks per wave

__device__ __forceinline__ uint32_t key32(uint32_t b) {
  const uint32_t mag = b & 0x7FFFFFFFu;
  const uint32_t key = (b & 0x80000000u) ? 0x80000000u - mag : 0x80000000u + mag;
  return mag > 0x7F800000u ? 0u : key;
}

__device__ __forceinline__ uint64_t lanes_ugt64(uint64_t a, uint64_t b) { return ballot(a > b); }

// One 64-bit composite into the descending list (see insert_one).
__device__ __forceinline__ uint64_t insert_one64(uint64_t list, uint64_t c) {
  const uint32_t plo = (uint32_t)__builtin_amdgcn_update_dpp((int)0xFFFFFFFFu, (int)(uint32_t)list, 0x138, 0xF, 0xF, false);
  const uint32_t phi =
      (uint32_t)__builtin_amdgcn_update_dpp((int)0xFFFFFFFFu, (int)(uint32_t)(list >> 32), 0x138, 0xF, 0xF, false);
  const uint64_t prev = ((uint64_t)phi << 32) | plo;
  const uint64_t lo = prev < c ? prev : c;
  return list > lo ? list : lo;
}

// Descending bitonic sort of one 64-bit value per lane (the stages of sort64_desc).
__device__ __forceinline__ uint64_t sort64_desc64(uint64_t v, const Xchg &x) {
  v = cx_stage64<1, 1>(v, x);
  v = cx_stage64<3, 2>(v, x);
  v = cx_stage64<1, 1>(v, x);
  v = cx_stage64<7, 4>(v, x);
  v = cx_stage64<2, 2>(v, x);
  v = cx_stage64<1, 1>(v, x);
  v = cx_stage64<15, 8>(v, x);
  v = cx_stage64<4, 4>(v, x);
  v = cx_stage64<2, 2>(v, x);
  v = cx_stage64<1, 1>(v, x);
  v = cx_stage64<31, 16>(v, x);
  v = cx_stage64<8, 8>(v, x);
  v = cx_stage64<4, 4>(v, x);
  v = cx_stage64<2, 2>(v, x);
  v = cx_stage64<1, 1>(v, x);
  v = cx_stage64<63, 32>(v, x);
  v = cx_stage64<16, 16>(v, x);
  v = cx_stage64<8, 8>(v, x);
  v = cx_stage64<4, 4>(v, x);
  v = cx_stage64<2, 2>(v, x);
  v = cx_stage64<1, 1>(v, x);
  return v;
}

struct Wave32 {
  uint64_t list;   // lane i: i-th best composite so far, 0 = empty
  uint64_t kth;    // wave-uniform copy of list[k - 1]
  uint32_t ext;    // wave-uniform: keys <= ext are beaten by k entries of the workgroup
  uint32_t floor;  // wave-uniform floor: only keys > floor are kept (0 = none)
  uint32_t flags;  // wave-uniform NaN / -inf flags seen so far
  int km1, qm1, wave;
  uint32_t *tau;   // LDS: published k-th and ceil(k/4)-th keys of the waves
  uint64_t *ring;  // LDS: this wave's kRing32 pending composites
  uint32_t r0;     // wave-uniform ring index of the oldest pending composite
  uint32_t nr;     // wave-uniform count of pending composites
  Xchg x;
};

// Candidates of the exact path wait in an LDS ring (a power of two, above
// the 31 left after a merge plus the 256 one vector can add) and enter the
// list as sorted batches once 32 are pending: appending costs about ten
// instructions per element position, an insertion of one 64-bit entry about
// twenty per entry.  On MI355X the ring took 1024 x 151936 fp32 rows at
// k = 64 from 110-115 to 105-106 us, 16 x 248320 at k = 20 from 25.4 to
// 21.2 us and 64 x 151936 at k = 16 from 29.3 to 25.4 us (batches at 64
// pending: 106, 20.8, 27.1 us; at 16: 108, 21.7, 25.9 us).
constexpr int kRing32 = 512;
constexpr int kRing32Flush = 32;

// Adds the candidates c of lanes m (and of no other lane): one bitonic batch
// when many, else one insertion each (against a k-th refreshed only
// afterwards: see offer).
__device__ __forceinline__ void offer64(Wave32 &w, uint64_t c, uint64_t m) {
  if (__popcll(m) >= kBatchInsert) {
    const bool take = (m >> lane_id()) & 1ull;
    w.list = merge_sorted64(w.list, sort64_desc64(take ? c : 0, w.x), w.x);
  } else {
    do {
      const int l = __builtin_ctzll(m);
      m &= m - 1;
      w.list = insert_one64(w.list, readlane64(c, l));
    } while (m);
  }
  w.kth = readlane64(w.list, w.km1);
}

// Threshold sharing, as in the bf16 scan (shared_bound / publish there).
__device__ __forceinline__ uint32_t shared_bound32(const uint32_t *s_tau, int wave) {
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

__device__ __forceinline__ void publish32(const Wave32 &w) {
  const uint32_t q = (uint32_t)(readlane64(w.list, w.qm1) >> 32);
  if (lane_id() == 0) {
    __hip_atomic_store(&w.tau[w.wave], (uint32_t)(w.kth >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(&w.tau[kWgWaves + w.wave], q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// Raw-bit filter from T = max(k-th kept key, ext): an element may matter only
// if its key exceeds T.  T >= 2^31: bits, as int32, above T - 2^31 (only
// non-negative patterns, +NaN included, pass).  T < 2^31: bits, as uint32,
// at most 0xFFFFFFFF - T (every non-negative pattern passes, and negatives
// whose magnitude is below 2^31 - T).
struct Filter32 {
  bool nonneg;
  int32_t t32;
  uint32_t tum1;
  bool check_flags;  // some of -inf / negative NaN not flagged yet
  uint32_t ftrip;    // patterns >= ftrip: -inf (0xFF800000) or negative NaN
};

__device__ __forceinline__ Filter32 filter32_for(uint32_t t, uint32_t flags) {
  Filter32 f;
  f.nonneg = t >= 0x80000000u;
  f.t32 = (int32_t)(t - 0x80000000u);
  f.tum1 = 0xFFFFFFFFu - t;
  f.check_flags = (flags & (kNan | kNinf)) != (kNan | kNinf);
  f.ftrip = (flags & kNinf) ? 0xFF800001u : 0xFF800000u;
  return f;
}


__device__ __forceinline__ uint64_t value_trip(uint4 d, const Filter32 &f) {
  if (f.nonneg) {
    const int32_t a = max(max((int32_t)d.x, (int32_t)d.y), max((int32_t)d.z, (int32_t)d.w));
    return __builtin_amdgcn_sicmp(a, f.t32, 38);  // >
  }
  const uint32_t a = min(min(d.x, d.y), min(d.z, d.w));
  return __builtin_amdgcn_uicmp(a, f.tum1, 37);  // <=
}

__device__ __forceinline__ uint64_t flag_trip(uint4 d, const Filter32 &f) {
  if (!f.check_flags) return 0;
  const uint32_t a = max(max(d.x, d.y), max(d.z, d.w));
  return lanes_uge(a, f.ftrip);
}

// The oldest min(64, pending) candidates leave the ring as one batch, sorted
// and merged into the list; the k-th and the published keys follow.
__device__ __forceinline__ void flush32(Wave32 &w) {
  __builtin_amdgcn_wave_barrier();  // the ring's stores above precede its loads
  const uint32_t take = min(w.nr, (uint32_t)kWave);
  const uint32_t l = (uint32_t)lane_id();
  const uint64_t v = l < take ? w.ring[(w.r0 + l) & (kRing32 - 1)] : 0;
  w.r0 = (w.r0 + take) & (kRing32 - 1);
  w.nr -= take;
  w.list = merge_sorted64(w.list, sort64_desc64(v, w.x), w.x);
  w.kth = readlane64(w.list, w.km1);
  publish32(w);
}

// Exact path for one vector of four elements per lane (lanes `lanes`): per
// element, the lanes whose key exceeds t append their composites to the
// ring (see wide32_vector), and -inf / NaN patterns are flagged.
__device__ __forceinline__ void take_vector32(Wave32 &w, uint4 d, uint32_t col0, uint64_t lanes, uint32_t t) {
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
  uint64_t nan = 0, ninf = 0;
#pragma unroll
  for (int e = 0; e < kElems32; ++e) {
    const uint32_t b = dw[e];
    const uint32_t key = key32(b);
    nan |= lanes & lanes_eq(key, 0u);
    ninf |= lanes & lanes_eq(b, 0xFF800000u);
    const uint64_t h = lanes & lanes_ugt(key, t);
    if (h) {
      const uint32_t slot = __builtin_amdgcn_mbcnt_hi((uint32_t)(h >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)h, w.r0 + w.nr));
      if (__builtin_amdgcn_inverse_ballot_w64(h))
        w.ring[slot & (kRing32 - 1)] = ((uint64_t)key << 32) | (0xFFFFFFFFu - (col0 + (uint32_t)e));
      w.nr += (uint32_t)__popcll(h);
    }
  }
  if (nan) w.flags |= kNan;
  if (ninf) w.flags |= kNinf;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer format on gfx9-family parts
constexpr int kLoadPolicy = 2;            // nontemporal: the input is read once

// Vectors [first, first + kChunkVecs * 64) of the wave's nvec at vp (lane l's
// vector u is first + u * 64 + l); vectors at or past nvec read zeros.
__device__ __forceinline__ void load_chunk32(uint4 (&dst)[kChunkVecs], const uint4 *vp, uint32_t nvec, uint32_t first,
                                             uint32_t lane_off) {
  first = (uint32_t)__builtin_amdgcn_readfirstlane((int)first);
  nvec = (uint32_t)__builtin_amdgcn_readfirstlane((int)nvec);
  uint32_t left = (uint32_t)__builtin_amdgcn_readfirstlane((int)(nvec - min(first, nvec)));
  left = min(left, (uint32_t)(kChunkVecs * kWave));
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)(vp + first), (short)0, (int)(left * 16u), kBufferWord3);
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    const u32x4 x =
        __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(lane_off + (uint32_t)(u * kWave * 16)), 0, kLoadPolicy);
    dst[u] = make_uint4(x.x, x.y, x.z, x.w);
  }
}

__device__ __forceinline__ uint32_t lane_max_key32(const uint4 (&v)[kChunkVecs], uint32_t nvec) {
  uint32_t m = 0;
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    const uint32_t mu = max(max(key32(v[u].x), key32(v[u].y)), max(key32(v[u].z), key32(v[u].w)));
    if ((uint32_t)(u * kWave + lane_id()) < nvec) m = max(m, mu);
  }
  return m;
}

// This lane's R largest keys in a loaded chunk (vectors at or past nvec,
// counted from the chunk's start, give none), in descending order: R
// distinct elements.
template <int R>
__device__ __forceinline__ void lane_top_keys32(const uint4 (&v)[kChunkVecs], uint32_t nvec, uint32_t (&t)[R]) {
#pragma unroll
  for (int j = 0; j < R; ++j) t[j] = 0;
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    const bool in = (uint32_t)(u * kWave + lane_id()) < nvec;
    const uint32_t e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t key = in ? key32(e[i]) : 0u;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const uint32_t hi = max(t[j], key);
        key = min(t[j], key);
        t[j] = hi;
      }
    }
  }
}

// A floor of the wave's own from the end of its share (its final 256
// vectors), for rows that rise along it (the 16-bit scans describe the rule):
// the k-th largest of each lane's R largest keys there, minus one; 0 for none.
template <int R>
__device__ __forceinline__ uint32_t rising_floor32(const uint4 *vp, uint32_t nvec, uint32_t lane_off, int k,
                                                   const Xchg &x) {
  constexpr uint32_t kStep = (uint32_t)kChunkVecs * kWave;
  const uint32_t last = nvec - kStep;  // the share's last kStep vectors: every lane holds four
  uint4 L[kChunkVecs];
  load_chunk32(L, vp, nvec, last, lane_off);
  uint32_t t[R];
  lane_top_keys32<R>(L, nvec - last, t);
  const uint32_t te = rank_of_lane_keys<R>(t, k - 1, x);
  return te > 1 ? te - 1 : 0u;
}

// Nearly every lane of the first chunk has its largest key in its last
// vector: the wave's share rises (lanes' vectors lie 64 apart).
__device__ __forceinline__ bool share_rises32(const uint4 (&A)[kChunkVecs], uint32_t lm) {
  const uint4 v = A[kChunkVecs - 1];
  const uint32_t l3 = max(max(key32(v.x), key32(v.y)), max(key32(v.z), key32(v.w)));
  return __popcll(ballot(lm > 0 && l3 >= lm)) >= kLookLanes;
}

// This lane's two largest keys in a loaded chunk (*m2 = 0 with fewer than
// two): distinct elements, for the deeper floor of few-row k > 128 splits.
__device__ __forceinline__ void lane_top2_keys32(const uint4 (&v)[kChunkVecs], uint32_t nvec, uint32_t *m1,
                                                 uint32_t *m2) {
  uint32_t a = 0, b = 0;
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    const bool in = (uint32_t)(u * kWave + lane_id()) < nvec;
    const uint32_t e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t key = in ? key32(e[i]) : 0u;
      b = max(b, min(a, key));
      a = max(a, key);
    }
  }
  *m1 = a;
  *m2 = b;
}

// One chunk: trips against the thresholds at its start (they only rise),
// then the exact path for the tripped vectors in order.
__device__ __forceinline__ void take_chunk32(Wave32 &w, const uint4 (&v)[kChunkVecs], uint32_t first, uint32_t nvec,
                                             uint32_t col_first) {
  w.ext = max(shared_bound32(w.tau, w.wave), w.floor);
  uint32_t t = max((uint32_t)(w.kth >> 32), w.ext);
  const Filter32 f = filter32_for(t, w.flags);
  const uint32_t l = (uint32_t)lane_id();
  uint64_t any = 0, trip[kChunkVecs];
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    trip[u] = (value_trip(v[u], f) | flag_trip(v[u], f)) & lanes_ult(first + (uint32_t)(u * kWave) + l, nvec);
    any |= trip[u];
  }
  if (!any) return;
  uint4 x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];  // rotated once per vector: one copy of the exact path
  uint64_t t0 = trip[0], t1 = trip[1], t2 = trip[2], t3 = trip[3];
  uint32_t col = col_first + kElems32 * (first + l);
#pragma unroll 1
  for (int u = 0; u < kChunkVecs; ++u) {
    if (t0) {
      take_vector32(w, x0, col, t0, t);
      if (w.nr >= (uint32_t)kRing32Flush) {
        do {
          flush32(w);
        } while (w.nr >= (uint32_t)kRing32Flush);
        t = max((uint32_t)(w.kth >> 32), w.ext);
      }
    }
    x0 = x1;
    x1 = x2;
    x2 = x3;
    t0 = t1;
    t1 = t2;
    t2 = t3;
    t3 = 0;
    if (!(t0 | t1 | t2)) break;
    col += kElems32 * kWave;
  }
}

// Streams nvec vectors from vp (element 0 is column col_first), two chunks in
// flight; A holds the first chunk, already loaded.  Issue priority falls
// with progress, as in the bf16 scan (steps at 1/2, 3/4 and 9/10 of the
// share: 0.7 us faster than every quarter on 1024 x 151936 fp32 rows).
__device__ __forceinline__ void take_body32(Wave32 &w, const uint4 *vp, uint32_t nvec, uint32_t col_first,
                                            uint4 (&A)[kChunkVecs]) {
  constexpr uint32_t kStep = (uint32_t)kChunkVecs * kWave;
  const uint32_t lane_off = (uint32_t)lane_id() * 16u;
  uint4 B[kChunkVecs];
  const uint32_t q1 = nvec / 2, q2 = nvec - nvec / 4, q3 = nvec - nvec / 10;
  __builtin_amdgcn_s_setprio(3);
  for (uint32_t first = 0; first < nvec; first += 2 * kStep) {
    if (first >= q3) __builtin_amdgcn_s_setprio(0);
    else if (first >= q2) __builtin_amdgcn_s_setprio(1);
    else if (first >= q1) __builtin_amdgcn_s_setprio(2);
    load_chunk32(B, vp, nvec, first + kStep, lane_off);
    take_chunk32(w, A, first, nvec, col_first);
    if (first + kStep >= nvec) break;
    load_chunk32(A, vp, nvec, first + 2 * kStep, lane_off);
    take_chunk32(w, B, first + kStep, nvec, col_first);
  }
}

// Columns [lo, hi) one per lane (row edges outside the 16-byte grid).
__device__ void take_columns32(Wave32 &w, const uint32_t *row, int64_t lo, int64_t hi) {
  for (int64_t c0 = lo; c0 < hi; c0 += kWave) {
    const int64_t col = c0 + lane_id();
    const bool valid = col < hi;
    const uint32_t b = valid ? row[col] : 0u;
    const uint32_t key = key32(b);
    if (ballot(valid && key == 0)) w.flags |= kNan;
    if (ballot(valid && b == 0xFF800000u)) w.flags |= kNinf;
    const uint64_t c = (valid && key > w.ext) ? ((uint64_t)key << 32) | (0xFFFFFFFFu - (uint32_t)col) : 0;
    const uint64_t m = lanes_ugt64(c, w.kth);
    if (m) offer64(w, c, m);
  }
}

__device__ __forceinline__ int32_t col_of32(uint64_t x) { return (int32_t)(0xFFFFFFFFu - (uint32_t)x); }

// fp32 bits of an entry: the key is invertible except for the zeros' shared
// key, whose sign is read back from the input.
__device__ __forceinline__ uint32_t value_bits32(uint64_t x, const uint32_t *row) {
  const uint32_t key = (uint32_t)(x >> 32);
  if (key > 0x80000000u) return key - 0x80000000u;
  if (key < 0x80000000u) return 0x80000000u | (0x80000000u - key);
  return row[col_of32(x)];
}

// The last workgroup of a split row folds the row's span lists (see
// fold_row_if_last in the bf16 scan: agent-scope atomic stores and loads, an
// arrival counter that returns to zero).
__device__ __forceinline__ void fold_row32_if_last(const ScanArgs32 &a, int64_t r, int S, const uint32_t *row,
                                                   int wave, int l) {
  __shared__ int s_last;
  __shared__ uint64_t s_acc[kWgWaves][kWave];
  __shared__ int32_t s_cnt[kWgWaves];
  __shared__ uint32_t s_fl[kWgWaves];
  const int64_t rb = r - a.row0;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&a.row_done[rb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
  __syncthreads();
  if (!s_last) return;
  const Xchg x = make_xchg();
  uint64_t acc = 0;
  int cnt = 0;
  uint32_t fl = 0;
  // each wave folds lists wave, wave + 4, ...; four lists' loads in flight at once
  for (int i0 = wave; i0 < S; i0 += 4 * kWgWaves) {
    uint64_t v[4];
    int c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + q * kWgWaves;
      const int64_t sb = r * S + i;
      c[q] = 0;
      v[q] = 0;
      if (i < S) {
        c[q] = __hip_atomic_load(&a.span_count[sb], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        fl |= __hip_atomic_load(&a.span_flags[sb], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (l < a.k) v[q] = __hip_atomic_load(&a.span_list[sb * a.k + l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (i0 + q * kWgWaves >= S) break;
      const uint64_t vq = l < c[q] ? v[q] : 0;
      acc = (i0 == wave && q == 0) ? vq : merge_sorted64(acc, vq, x);
      cnt += c[q];
    }
  }
  s_acc[wave][l] = acc;
  if (l == 0) {
    s_cnt[wave] = cnt;
    s_fl[wave] = fl;
  }
  __syncthreads();
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
  if (wave != 0) return;
  acc = merge_sorted64(acc, s_acc[2][l], x);
  cnt += s_cnt[2];
  fl |= s_fl[2];
  const int k = a.k;
  if (cnt > k) cnt = k;
  const int64_t ob = r * k;
  if (l < k) {
    if (l < cnt) {
      a.out_idx[ob + l] = col_of32(acc);
      a.out_val[ob + l] = value_bits32(acc, row);
    } else {
      a.out_idx[ob + l] = TK_FILL_IDX;
      a.out_val[ob + l] = 0x7FC00000u;
    }
  }
  if (l == 0) {
    a.out_count[r] = cnt;
    a.out_nonfinite[r] = fl;
    __hip_atomic_store(&a.row_done[rb], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ __launch_bounds__(kWgThreads) void span_scan32_kernel(ScanArgs32 a) {
  __shared__ uint64_t s_list[kWgWaves][kWave];
  __shared__ int32_t s_count[kWgWaves];
  __shared__ uint32_t s_flags[kWgWaves];
  __shared__ uint32_t s_tau[2 * kWgWaves];
  __shared__ uint32_t s_samp[kWgWaves][kWave];
  __shared__ uint64_t s_ring[kWgWaves][kRing32];

  const int64_t blk = blockIdx.x;
  const int64_t r = a.row0 + blk / a.spans;
  const int s = (int)(blk % a.spans);
  const int S = a.spans;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int l = lane_id();
  const uint32_t *row = a.in + r * a.stride;

  // The row's 16-byte grid: vector j covers columns [a0 + 4j, a0 + 4j + 4).
  const int64_t a0 = (int64_t)((4u - (uint32_t)(((uintptr_t)row >> 2) & 3u)) & 3u);
  const int64_t nv_row = a.cols > a0 ? (a.cols - a0) / kElems32 : 0;
  int64_t j0 = 0, j1 = 0, head_lo = 0, head_hi = 0, tail_lo = 0, tail_hi = 0;
  if (nv_row > 0) {
    j0 = nv_row * s / S;
    j1 = nv_row * (s + 1) / S;
    if (s == 0) head_hi = a0;
    if (s == S - 1) {
      tail_lo = a0 + kElems32 * nv_row;
      tail_hi = a.cols;
    }
  } else if (s == 0) {
    head_hi = a.cols;
  }
  const int64_t n = j1 - j0;
  const int64_t wv0 = j0 + n * wave / kWgWaves;
  const int64_t wv1 = j0 + n * (wave + 1) / kWgWaves;

  // Floors from a pooled first-chunk sample, as in the bf16 scan.
  const uint4 *wvp = reinterpret_cast<const uint4 *>(row + a0) + wv0;
  const uint32_t wn = (uint32_t)(wv1 - wv0);
  uint4 A[kChunkVecs];
  if (wn > 0) load_chunk32(A, wvp, wn, 0, (uint32_t)l * 16u);
  const bool speculate = a.spec_rank > 0 && !a.exact && n / kWgWaves >= (int64_t)kSpecChunks * kChunkVecs * kWave;
  uint32_t exact_floor, spec_floor;
  const uint32_t lm = wn > 0 ? lane_max_key32(A, wn) : 0u;
  {
    const Xchg x = make_xchg();
    s_samp[wave][l] = sort64_desc(lm, x);
    __syncthreads();
    uint32_t v[kWgWaves];
#pragma unroll
    for (int o = 0; o < kWgWaves; ++o) v[o] = s_samp[o][l];
#pragma unroll
    for (int step = 1; step < kWgWaves; step *= 2)
#pragma unroll
      for (int o = 0; o + step < kWgWaves; o += 2 * step)
        v[o] = bitonic_merge64_desc(max(v[o], partner<63>(v[o + step], x)), x);
    const uint32_t te = readlane(v[0], a.k - 1);
    const uint32_t ts = speculate ? readlane(v[0], a.spec_rank - 1) : 0u;
    exact_floor = te > 0 ? te - 1 : 0;
    spec_floor = ts > 0 ? ts - 1 : 0;
  }
  // rows that rise along this wave's share: a floor of its own from the end
  // (exact, so it also holds if the speculation fails; the choice to
  // speculate stays the same in every wave)
  uint32_t rise_floor = 0;
  if (wn >= (uint32_t)(kLookChunks * kChunkVecs * kWave) && share_rises32(A, lm))
    rise_floor = rising_floor32<1>(wvp, wn, (uint32_t)l * 16u, a.k, make_xchg());
  uint32_t floor = exact_floor;
  bool verify = false;
  if (spec_floor > exact_floor) {
    floor = spec_floor;
    verify = true;
  }
  floor = max(floor, rise_floor);

  int total = 0;
  uint32_t flags = 0;
  for (;;) {
    if (threadIdx.x < 2 * kWgWaves) s_tau[threadIdx.x] = 0;
    __syncthreads();
    Wave32 w;
    w.list = 0;
    w.kth = 0;
    w.ext = floor;
    w.floor = floor;
    w.flags = 0;
    w.km1 = a.k - 1;
    w.qm1 = (a.k + kWgWaves - 1) / kWgWaves - 1;
    w.wave = wave;
    w.tau = s_tau;
    w.ring = s_ring[wave];
    w.r0 = 0;
    w.nr = 0;
    w.x = make_xchg();

    if (wave == 0 && head_hi > head_lo) take_columns32(w, row, head_lo, head_hi);
    if (wn > 0) take_body32(w, wvp, wn, (uint32_t)(a0 + kElems32 * wv0), A);
    while (w.nr > 0) flush32(w);
    if (wave == kWgWaves - 1 && tail_hi > tail_lo) take_columns32(w, row, tail_lo, tail_hi);

    const uint64_t valid_mask = ballot(w.list != 0);
    s_list[wave][l] = w.list;
    if (l == 0) {
      const int cnt = __popcll(valid_mask);
      s_count[wave] = cnt < a.k ? cnt : a.k;
      s_flags[wave] = w.flags | ((uint32_t)(readlane64(w.list, 0) >> 32) == 0xFF800000u ? kPinf : 0u);
    }
    __syncthreads();

    total = 0;
    flags = 0;
#pragma unroll
    for (int o = 0; o < kWgWaves; ++o) {
      total += s_count[o];
      flags |= s_flags[o];
    }
    if (!verify || total >= a.k) break;  // exact, or the speculation verified
    floor = max(exact_floor, rise_floor);  // too few entries reach the speculative floor
    verify = false;
    if (wn > 0) load_chunk32(A, wvp, wn, 0, (uint32_t)l * 16u);
    __syncthreads();
  }
  if (total > a.k) total = a.k;

  // The four wave lists meet as a tree in registers (as in the 16-bit scan):
  // waves 0 and 2 merge the next wave's list into theirs, then wave 0 merges
  // in wave 2's result.  Entries past a wave's count are empty zeros or
  // beaten by k of its own, so whole lists are merged.
  const Xchg xm = make_xchg();
  uint64_t acc = s_list[wave][l];
  if ((wave & 1) == 0) acc = merge_sorted64(acc, s_list[wave + 1][l], xm);
  if (wave == 2) s_list[2][l] = acc;  // no other wave reads slot 2 before the barrier
  __syncthreads();
  if (wave == 0) {
    acc = merge_sorted64(acc, s_list[2][l], xm);
    if (S == 1) {
      const int64_t ob = r * a.k;
      if (l < total) {
        a.out_idx[ob + l] = col_of32(acc);
        a.out_val[ob + l] = value_bits32(acc, row);
      } else if (l < a.k) {
        a.out_idx[ob + l] = TK_FILL_IDX;
        a.out_val[ob + l] = 0x7FC00000u;
      }
      if (l == 0) {
        a.out_count[r] = total;
        a.out_nonfinite[r] = flags;
      }
    } else {
      const int64_t sb = r * S + s;
      if (l < total) __hip_atomic_store(&a.span_list[sb * a.k + l], acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (l == 0) {
        __hip_atomic_store(&a.span_count[sb], total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.span_flags[sb], flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (S > 1) fold_row32_if_last(a, r, S, row, wave, l);
}

// ---------------------------------------------------------------------------
// k = 1 on fp32 rows: the argmax scan of the 16-bit formats (tk_kernels.hip)
// with 32-bit keys -- one wave-uniform best composite (key << 32 | ~column,
// absolute columns), T = max(its key, the other waves' published best keys
// under the left/right rule), a tripped chunk costing one per-lane maximum
// over the tripping vectors and one 64-bit wave maximum; split rows keep one
// composite and one flags word per span for the row's last workgroup.

__device__ __forceinline__ uint64_t wave_max64(uint64_t v, const Xchg &x) {
  uint64_t y;
  y = partner64<1>(v, x); v = v > y ? v : y;
  y = partner64<2>(v, x); v = v > y ? v : y;
  y = partner64<4>(v, x); v = v > y ? v : y;
  y = partner64<8>(v, x); v = v > y ? v : y;
  y = partner64<16>(v, x); v = v > y ? v : y;
  y = partner64<32>(v, x); v = v > y ? v : y;
  return readlane64(v, 0);
}

struct WaveArgmax32 {
  uint64_t best;    // wave-uniform best composite, 0 = none
  uint32_t flags;   // wave-uniform NaN / -inf flags
  int wave;
  uint32_t *s_key;  // LDS: each wave's best key
  Xchg x;
};

__device__ __forceinline__ uint32_t argmax_bound32(const WaveArgmax32 &w) {
  uint32_t ext = 0;
#pragma unroll
  for (int o = 0; o < kWgWaves; ++o) {
    if (o == w.wave) continue;
    const uint32_t t = __hip_atomic_load(&w.s_key[o], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    ext = max(ext, o < w.wave ? t : (t > 0 ? t - 1 : 0u));
  }
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)ext);
}

__device__ __forceinline__ void argmax_update32(WaveArgmax32 &w, uint64_t m, bool nan, bool ninf) {
  if (ballot(nan)) w.flags |= kNan;
  if (ballot(ninf)) w.flags |= kNinf;
  const uint64_t wm = wave_max64(m, w.x);
  if (wm > w.best) {
    w.best = wm;
    if (lane_id() == 0)
      __hip_atomic_store(&w.s_key[w.wave], (uint32_t)(wm >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// One chunk (lane l's vector u = first + 64 u + l, its element e at column
// col_first + 4 (first + 64 u + l) + e).
__device__ __forceinline__ void argmax_chunk32(WaveArgmax32 &w, const uint4 (&v)[kChunkVecs], uint32_t first,
                                               uint32_t nvec, uint32_t col_first) {
  const uint32_t t = max((uint32_t)(w.best >> 32), argmax_bound32(w));
  const Filter32 f = filter32_for(t, w.flags);
  const uint32_t l = (uint32_t)lane_id();
  uint64_t trip[kChunkVecs], any = 0;
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    trip[u] = (value_trip(v[u], f) | flag_trip(v[u], f)) & lanes_ult(first + (uint32_t)(u * kWave) + l, nvec);
    any |= trip[u];
  }
  if (!any) return;
  uint4 x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];  // rotated: no dynamic index into registers
  uint64_t t0 = trip[0], t1 = trip[1], t2 = trip[2], t3 = trip[3];
  uint32_t col = col_first + kElems32 * (first + l);
  uint64_t m = 0;
  bool nan = false, ninf = false;
#pragma unroll 1
  for (int u = 0; u < kChunkVecs; ++u) {
    if ((t0 >> l) & 1u) {
      const uint32_t dw[4] = {x0.x, x0.y, x0.z, x0.w};
#pragma unroll
      for (int e = 0; e < kElems32; ++e) {
        const uint32_t key = key32(dw[e]);
        nan |= key == 0;
        ninf |= dw[e] == 0xFF800000u;
        const uint64_t c = key ? ((uint64_t)key << 32) | (0xFFFFFFFFu - (col + (uint32_t)e)) : 0;
        m = m > c ? m : c;
      }
    }
    x0 = x1;
    x1 = x2;
    x2 = x3;
    t0 = t1;
    t1 = t2;
    t2 = t3;
    t3 = 0;
    if (!(t0 | t1 | t2)) break;
    col += kElems32 * kWave;
  }
  argmax_update32(w, m, nan, ninf);
}

__device__ void argmax_columns32(WaveArgmax32 &w, const uint32_t *row, int64_t lo, int64_t hi) {
  uint64_t m = 0;
  bool nan = false, ninf = false;
  for (int64_t c0 = lo; c0 < hi; c0 += kWave) {
    const int64_t col = c0 + lane_id();
    const bool valid = col < hi;
    const uint32_t b = valid ? row[col] : 0u;
    const uint32_t key = valid ? key32(b) : 0u;
    nan |= valid && key == 0;
    ninf |= valid && b == 0xFF800000u;
    const uint64_t c = key ? ((uint64_t)key << 32) | (0xFFFFFFFFu - (uint32_t)col) : 0;
    m = m > c ? m : c;
  }
  argmax_update32(w, m, nan, ninf);
}

__global__ __launch_bounds__(kWgThreads) void argmax_scan32_kernel(ArgmaxArgs32 a) {
  __shared__ uint32_t s_key[kWgWaves];
  __shared__ uint64_t s_best[kWgWaves];
  __shared__ uint32_t s_fl[kWgWaves];

  const int64_t blk = blockIdx.x;
  const int64_t r = a.row0 + blk / a.spans;
  const int s = (int)(blk % a.spans);
  const int S = a.spans;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int l = lane_id();
  const uint32_t *row = a.in + r * a.stride;

  // the span and wave shares of span_scan32_kernel
  const int64_t a0 = (int64_t)((4u - (uint32_t)(((uintptr_t)row >> 2) & 3u)) & 3u);
  const int64_t nv_row = a.cols > a0 ? (a.cols - a0) / kElems32 : 0;
  int64_t j0 = 0, j1 = 0, head_hi = 0, tail_lo = 0, tail_hi = 0;
  if (nv_row > 0) {
    j0 = nv_row * s / S;
    j1 = nv_row * (s + 1) / S;
    if (s == 0) head_hi = a0;
    if (s == S - 1) {
      tail_lo = a0 + kElems32 * nv_row;
      tail_hi = a.cols;
    }
  } else if (s == 0) {
    head_hi = a.cols;
  }
  const int64_t n = j1 - j0;
  const int64_t wv0 = j0 + n * wave / kWgWaves;
  const int64_t wv1 = j0 + n * (wave + 1) / kWgWaves;

  if (threadIdx.x < kWgWaves) s_key[threadIdx.x] = 0;
  __syncthreads();
  WaveArgmax32 w;
  w.best = 0;
  w.flags = 0;
  w.wave = wave;
  w.s_key = s_key;
  w.x = make_xchg();

  if (wave == 0 && head_hi > 0) argmax_columns32(w, row, 0, head_hi);
  const uint4 *vp = reinterpret_cast<const uint4 *>(row + a0) + wv0;
  const uint32_t nvec = (uint32_t)(wv1 - wv0);
  if (nvec > 0) {
    constexpr uint32_t kStep = (uint32_t)kChunkVecs * kWave;
    const uint32_t lane_off = (uint32_t)l * 16u;
    const uint32_t col_first = (uint32_t)(a0 + kElems32 * wv0);
    uint4 A[kChunkVecs], B[kChunkVecs];
    load_chunk32(A, vp, nvec, 0, lane_off);
    for (uint32_t first = 0; first < nvec; first += 2 * kStep) {
      load_chunk32(B, vp, nvec, first + kStep, lane_off);
      argmax_chunk32(w, A, first, nvec, col_first);
      if (first + kStep >= nvec) break;
      load_chunk32(A, vp, nvec, first + 2 * kStep, lane_off);
      argmax_chunk32(w, B, first + kStep, nvec, col_first);
    }
  }
  if (wave == kWgWaves - 1 && tail_hi > tail_lo) argmax_columns32(w, row, tail_lo, tail_hi);

  if (l == 0) {
    s_best[wave] = w.best;
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
    const int64_t rb = r - a.row0;
    if (l == 0) {
      __hip_atomic_store(&a.span_slot[rb * S + s], best, __ATOMIC_RELAXED, kAgent);
      __hip_atomic_store(&a.span_flag[rb * S + s], fl, __ATOMIC_RELAXED, kAgent);
    }
    __builtin_amdgcn_s_waitcnt(0);
    int last = 0;
    if (l == 0) last = __hip_atomic_fetch_add(&a.row_done[rb], 1, __ATOMIC_RELAXED, kAgent) == S - 1;
    if (!ballot(last)) return;
    const uint64_t v = l < S ? __hip_atomic_load(&a.span_slot[rb * S + l], __ATOMIC_RELAXED, kAgent) : 0;
    const uint32_t f = l < S ? __hip_atomic_load(&a.span_flag[rb * S + l], __ATOMIC_RELAXED, kAgent) : 0u;
    fl = (ballot(f & kNan) ? kNan : 0u) | (ballot(f & kNinf) ? kNinf : 0u);
    best = wave_max64(v, make_xchg());
    if (l == 0) __hip_atomic_store(&a.row_done[rb], 0, __ATOMIC_RELAXED, kAgent);
  }
  if (l == 0) {
    if ((uint32_t)(best >> 32) == 0x80000000u + 0x7F800000u) fl |= kPinf;
    if (best) {
      a.out_idx[r] = col_of32(best);
      a.out_val[r] = value_bits32(best, row);
    } else {
      a.out_idx[r] = TK_FILL_IDX;
      a.out_val[r] = 0x7FC00000u;
    }
    a.out_count[r] = best ? 1 : 0;
    a.out_nonfinite[r] = fl;
  }
}

// ---------------------------------------------------------------------------
// 64 < k <= 256 on fp32 rows: the multi-register scan of tk_wide.hip with the
// 64-bit composites of this file -- each wave keeps 64 R composites (R = 2 or
// 4 registers of 64 bits, tk_lists.h), filters on raw bits (Filter32), takes
// the pooled exact and verified speculative floors, collects candidates in
// an LDS ring merged into the list 64 at a time (an insertion into four
// 64-bit registers costs about fifty instructions: the ring took 1024 x
// 151936 rows at k = 256 from 221-229 to 117-129 us), shares thresholds,
// merges the four lists as a register tree, and folds split rows in their
// last workgroup.

// Pending candidates of a wave: a ring of 64-bit composites in LDS (a power
// of two, above the 63 left after a batch plus the 256 one vector can add).
constexpr int kWideRing32 = 512;

template <int R>
struct WaveWide32 {
  uint64_t L[R];
  uint64_t kth;    // wave-uniform copy of rank k - 1
  uint32_t ext;    // wave-uniform: keys <= ext are beaten by k entries of the workgroup (or the floor)
  uint32_t floor;
  uint32_t flags;
  int km1, qm1, wave;
  uint32_t *tau;
  uint64_t *ring;  // LDS: this wave's kWideRing32 pending composites
  uint32_t r0;     // wave-uniform ring index of the oldest pending composite
  uint32_t nr;     // wave-uniform count of pending composites
  Xchg x;
};

template <int R>
__device__ __forceinline__ void wide32_offer(WaveWide32<R> &w, uint64_t c, uint64_t m) {
  if (__popcll(m) >= kBatchInsert) {
    const bool take = (m >> lane_id()) & 1ull;
    wide_merge_batch64<R>(w.L, take ? c : 0, w.x);
  } else {
    do {
      const int l = __builtin_ctzll(m);
      m &= m - 1;
      wide_insert_one64<R>(w.L, readlane64(c, l));
    } while (m);
  }
  w.kth = wide_at64<R>(w.L, w.km1);
}

template <int R>
__device__ __forceinline__ void wide32_publish(const WaveWide32<R> &w) {
  const uint32_t q = (uint32_t)(readlane64(w.L[0], w.qm1) >> 32);
  if (lane_id() == 0) {
    __hip_atomic_store(&w.tau[w.wave], (uint32_t)(w.kth >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(&w.tau[kWgWaves + w.wave], q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// The oldest min(64, pending) candidates leave the ring as one batch, sorted
// and cascaded into the list; the k-th and the published keys follow.
template <int R>
__device__ __forceinline__ void wide32_flush(WaveWide32<R> &w) {
  __builtin_amdgcn_wave_barrier();  // the ring's stores above precede its loads
  const uint32_t take = min(w.nr, (uint32_t)kWave);
  const uint32_t l = (uint32_t)lane_id();
  const uint64_t v = l < take ? w.ring[(w.r0 + l) & (kWideRing32 - 1)] : 0;
  w.r0 = (w.r0 + take) & (kWideRing32 - 1);
  w.nr -= take;
  wide_merge_batch64<R>(w.L, v, w.x);
  w.kth = wide_at64<R>(w.L, w.km1);
  wide32_publish<R>(w);
}

// One vector of four elements per lane (lanes `lanes`): per element, the
// lanes whose key exceeds t (the k-th's key at the last batch, or ext) append
// their composites to the ring, and -inf / NaN patterns are flagged.  Every
// vector of a chunk lies at higher columns than the entries the k-th came
// from, so an equal key loses to it and the key test is exact; pending
// composites only lag the k-th (extra candidates land at ranks >= k).
template <int R>
__device__ __forceinline__ void wide32_vector(WaveWide32<R> &w, uint4 d, uint32_t col0, uint64_t lanes, uint32_t t) {
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
  uint64_t nan = 0, ninf = 0;
#pragma unroll
  for (int e = 0; e < kElems32; ++e) {
    const uint32_t b = dw[e];
    const uint32_t key = key32(b);
    nan |= lanes & lanes_eq(key, 0u);
    ninf |= lanes & lanes_eq(b, 0xFF800000u);
    const uint64_t h = lanes & lanes_ugt(key, t);
    if (h) {
      const uint32_t slot = __builtin_amdgcn_mbcnt_hi((uint32_t)(h >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)h, w.r0 + w.nr));
      if (__builtin_amdgcn_inverse_ballot_w64(h))
        w.ring[slot & (kWideRing32 - 1)] = ((uint64_t)key << 32) | (0xFFFFFFFFu - (col0 + (uint32_t)e));
      w.nr += (uint32_t)__popcll(h);
    }
  }
  if (nan) w.flags |= kNan;
  if (ninf) w.flags |= kNinf;
}

// One chunk: trips against the thresholds at its start, then the tripped
// vectors in column order; every 64 pending candidates are merged into the
// list as a batch, after which the key threshold is taken again.
template <int R>
__device__ __forceinline__ void wide32_chunk(WaveWide32<R> &w, const uint4 (&v)[kChunkVecs], uint32_t first,
                                             uint32_t nvec, uint32_t col_first) {
  w.ext = max(shared_bound32(w.tau, w.wave), w.floor);
  uint32_t t = max((uint32_t)(w.kth >> 32), w.ext);
  const Filter32 f = filter32_for(t, w.flags);
  const uint32_t l = (uint32_t)lane_id();
  uint64_t trip[kChunkVecs], any = 0;
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    trip[u] = (value_trip(v[u], f) | flag_trip(v[u], f)) & lanes_ult(first + (uint32_t)(u * kWave) + l, nvec);
    any |= trip[u];
  }
  if (!any) return;
  uint4 x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
  uint64_t t0 = trip[0], t1 = trip[1], t2 = trip[2], t3 = trip[3];
  uint32_t col = col_first + kElems32 * (first + l);
#pragma unroll 1
  for (int u = 0; u < kChunkVecs; ++u) {
    if (t0) {
      wide32_vector<R>(w, x0, col, t0, t);
      if (w.nr >= (uint32_t)kWave) {
        do {
          wide32_flush<R>(w);
        } while (w.nr >= (uint32_t)kWave);
        t = max((uint32_t)(w.kth >> 32), w.ext);
      }
    }
    x0 = x1;
    x1 = x2;
    x2 = x3;
    t0 = t1;
    t1 = t2;
    t2 = t3;
    t3 = 0;
    if (!(t0 | t1 | t2)) break;
    col += kElems32 * kWave;
  }
}

template <int R>
__device__ __forceinline__ void wide32_body(WaveWide32<R> &w, const uint4 *vp, uint32_t nvec, uint32_t col_first,
                                            uint4 (&A)[kChunkVecs]) {
  constexpr uint32_t kStep = (uint32_t)kChunkVecs * kWave;
  const uint32_t lane_off = (uint32_t)lane_id() * 16u;
  uint4 B[kChunkVecs];
  // progress priority in quarters: the steps of take_body32 measured 0.7 us
  // slower here on 1024 x 151936 fp32 rows at k = 128
  const uint32_t q1 = nvec / 4, q2 = nvec / 2, q3 = nvec - nvec / 4;
  __builtin_amdgcn_s_setprio(3);
  for (uint32_t first = 0; first < nvec; first += 2 * kStep) {
    if (first >= q3) __builtin_amdgcn_s_setprio(0);
    else if (first >= q2) __builtin_amdgcn_s_setprio(1);
    else if (first >= q1) __builtin_amdgcn_s_setprio(2);
    load_chunk32(B, vp, nvec, first + kStep, lane_off);
    wide32_chunk<R>(w, A, first, nvec, col_first);
    if (first + kStep >= nvec) break;
    load_chunk32(A, vp, nvec, first + 2 * kStep, lane_off);
    wide32_chunk<R>(w, B, first + kStep, nvec, col_first);
  }
}

template <int R>
__device__ void wide32_columns(WaveWide32<R> &w, const uint32_t *row, int64_t lo, int64_t hi) {
  for (int64_t c0 = lo; c0 < hi; c0 += kWave) {
    const int64_t col = c0 + lane_id();
    const bool valid = col < hi;
    const uint32_t b = valid ? row[col] : 0u;
    const uint32_t key = key32(b);
    if (ballot(valid && key == 0)) w.flags |= kNan;
    if (ballot(valid && b == 0xFF800000u)) w.flags |= kNinf;
    const uint64_t c = (valid && key > w.ext) ? ((uint64_t)key << 32) | (0xFFFFFFFFu - (uint32_t)col) : 0;
    const uint64_t m = lanes_ugt64(c, w.kth);
    if (m) wide32_offer<R>(w, c, m);
  }
}

// Last-workgroup fold of a split row (the protocol of fold_row32_if_last),
// lists of up to 64 R entries merged as R-register lists.
template <int R>
__device__ __forceinline__ void wide32_fold_if_last(const ScanArgs32 &a, int64_t r, int S, const uint32_t *row,
                                                    int wave, int l, uint64_t (*s_acc)[kWave * R]) {
  __shared__ int s_last;
  __shared__ int32_t s_cnt[kWgWaves];
  __shared__ uint32_t s_fl[kWgWaves];
  const int64_t rb = r - a.row0;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) s_last = __hip_atomic_fetch_add(&a.row_done[rb], 1, __ATOMIC_RELAXED, kAgent) == S - 1;
  __syncthreads();
  if (!s_last) return;
  const Xchg x = make_xchg();
  const int k = a.k;
  uint64_t acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = 0;
  int cnt = 0;
  uint32_t fl = 0;
  // each wave folds lists wave, wave + 4, ...; four lists' loads in flight at once
  for (int i0 = wave; i0 < S; i0 += 4 * kWgWaves) {
    uint64_t B[4][R];
    int c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + q * kWgWaves;
      const int64_t sb = r * S + i;
      c[q] = i < S ? __hip_atomic_load(&a.span_count[sb], __ATOMIC_RELAXED, kAgent) : 0;
      if (i < S) fl |= __hip_atomic_load(&a.span_flags[sb], __ATOMIC_RELAXED, kAgent);
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const int e = j * kWave + l;
        B[q][j] = e < c[q] ? __hip_atomic_load(&a.span_list[sb * k + e], __ATOMIC_RELAXED, kAgent) : 0;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (i0 + q * kWgWaves >= S) break;
      cnt += c[q];
      if (i0 == wave && q == 0) {
#pragma unroll
        for (int j = 0; j < R; ++j) acc[j] = B[q][j];
      } else {
        wide_merge_lists64<R>(acc, B[q], x);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < R; ++j) s_acc[wave][j * kWave + l] = acc[j];
  if (l == 0) {
    s_cnt[wave] = cnt;
    s_fl[wave] = fl;
  }
  __syncthreads();
#pragma unroll
  for (int step = 1; step < kWgWaves; step *= 2) {
    if (wave % (2 * step) == 0) {
      uint64_t B[R];
#pragma unroll
      for (int j = 0; j < R; ++j) B[j] = s_acc[wave + step][j * kWave + l];
      wide_merge_lists64<R>(acc, B, x);
#pragma unroll
      for (int j = 0; j < R; ++j) s_acc[wave][j * kWave + l] = acc[j];
    }
    __syncthreads();
  }
  if (wave != 0) return;
#pragma unroll
  for (int o = 1; o < kWgWaves; ++o) {
    cnt += s_cnt[o];
    fl |= s_fl[o];
  }
  if (cnt > k) cnt = k;
  const int64_t ob = r * k;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int e = j * kWave + l;
    if (e < k) {
      if (e < cnt) {
        a.out_idx[ob + e] = col_of32(acc[j]);
        a.out_val[ob + e] = value_bits32(acc[j], row);
      } else {
        a.out_idx[ob + e] = TK_FILL_IDX;
        a.out_val[ob + e] = 0x7FC00000u;
      }
    }
  }
  if (l == 0) {
    a.out_count[r] = cnt;
    a.out_nonfinite[r] = fl;
    __hip_atomic_store(&a.row_done[rb], 0, __ATOMIC_RELAXED, kAgent);
  }
}

template <int R>
__global__ __launch_bounds__(kWgThreads) void wide_scan32_kernel(ScanArgs32 a) {
  __shared__ uint64_t s_list[kWgWaves][kWave * R];
  __shared__ int32_t s_count[kWgWaves];
  __shared__ uint32_t s_flags[kWgWaves];
  __shared__ uint32_t s_tau[2 * kWgWaves];
  __shared__ uint32_t s_samp[2 * kWgWaves][kWave];
  __shared__ uint64_t s_ring[kWgWaves][kWideRing32];

  const int64_t blk = blockIdx.x;
  const int64_t r = a.row0 + blk / a.spans;
  const int s = (int)(blk % a.spans);
  const int S = a.spans;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int l = lane_id();
  const uint32_t *row = a.in + r * a.stride;

  // the span and wave shares of span_scan32_kernel
  const int64_t a0 = (int64_t)((4u - (uint32_t)(((uintptr_t)row >> 2) & 3u)) & 3u);
  const int64_t nv_row = a.cols > a0 ? (a.cols - a0) / kElems32 : 0;
  int64_t j0 = 0, j1 = 0, head_hi = 0, tail_lo = 0, tail_hi = 0;
  if (nv_row > 0) {
    j0 = nv_row * s / S;
    j1 = nv_row * (s + 1) / S;
    if (s == 0) head_hi = a0;
    if (s == S - 1) {
      tail_lo = a0 + kElems32 * nv_row;
      tail_hi = a.cols;
    }
  } else if (s == 0) {
    head_hi = a.cols;
  }
  const int64_t n = j1 - j0;
  const int64_t wv0 = j0 + n * wave / kWgWaves;
  const int64_t wv1 = j0 + n * (wave + 1) / kWgWaves;
  const uint4 *wvp = reinterpret_cast<const uint4 *>(row + a0) + wv0;
  const uint32_t wn = (uint32_t)(wv1 - wv0);

  // floors from the workgroup's first chunk (R-register lists: k may exceed
  // one register): the lane maxima, or -- with k > 128 and no speculation,
  // where the k-th lane maximum is nearly the smallest -- each lane's two
  // largest keys (see the 16-bit wide scan)
  const Xchg x = make_xchg();
  uint4 A[kChunkVecs];
  if (wn > 0) load_chunk32(A, wvp, wn, 0, (uint32_t)l * 16u);
  const bool speculate =
      a.spec_rank > 0 && !a.exact && n / kWgWaves >= (int64_t)kWideSpecChunks32 * kChunkVecs * kWave;
  const bool pairs = R == 4 && a.k > 2 * kWave && !speculate;
  uint32_t m1 = 0;  // this lane's largest key of the first chunk
  {
    uint32_t m2 = 0;
    if (wn > 0) {
      if (pairs) lane_top2_keys32(A, wn, &m1, &m2);
      else m1 = lane_max_key32(A, wn);
    }
    s_samp[2 * wave][l] = sort64_desc(m1, x);
    if (pairs) s_samp[2 * wave + 1][l] = sort64_desc(m2, x);
  }
  __syncthreads();
  uint32_t exact_floor, spec_floor = 0;
  {
    // P = the top 64 R of the sorted lists, as a tree of bitonic merges:
    // 64 + 64 -> 128, then 128 + 128 -> 256 (and with pairs, the top 256 of
    // two such 256s)
    uint32_t P[R];
    uint32_t Q[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= 2 && !pairs) break;
      const int o0 = pairs ? 2 * i : 4 * i, o1 = pairs ? 2 * i + 1 : 4 * i + 2;
      const uint32_t a1[1] = {s_samp[o0][l]}, b1[1] = {s_samp[o1][l]};
      wide_merge_full<1>(a1, b1, Q[i], x);
    }
    if constexpr (R == 2) {
      P[0] = Q[0][0];
      P[1] = Q[0][1];
      wide_merge_top<2>(P, Q[1], x);
    } else {
      wide_merge_full<2>(Q[0], Q[1], P, x);
      if (pairs) {
        uint32_t V[4];
        wide_merge_full<2>(Q[2], Q[3], V, x);
        wide_merge_top<4>(P, V, x);
      }
    }
    const uint32_t te = wide_at<R>(P, a.k - 1);
    exact_floor = te > 0 ? te - 1 : 0;
    if (speculate) {
      const uint32_t ts = wide_at<R>(P, a.spec_rank - 1);
      spec_floor = ts > 0 ? ts - 1 : 0;
    }
  }
  // rows that rise along this wave's share: a floor of its own from the end,
  // from each lane's R largest keys there (64 R distinct elements); the
  // choice to speculate stays the same in every wave
  uint32_t rise_floor = 0;
  if (wn >= (uint32_t)(kLookChunks * kChunkVecs * kWave) && share_rises32(A, m1))
    rise_floor = rising_floor32<R>(wvp, wn, (uint32_t)l * 16u, a.k, x);
  uint32_t floor = exact_floor;
  bool verify = false;
  if (spec_floor > exact_floor) {
    floor = spec_floor;
    verify = true;
  }
  floor = max(floor, rise_floor);

  WaveWide32<R> w;
  int total = 0;
  uint32_t flags = 0;
  for (;;) {
    if (threadIdx.x < 2 * kWgWaves) s_tau[threadIdx.x] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < R; ++j) w.L[j] = 0;
    w.kth = 0;
    w.ext = floor;
    w.floor = floor;
    w.flags = 0;
    w.km1 = a.k - 1;
    w.qm1 = (a.k + kWgWaves - 1) / kWgWaves - 1;
    w.wave = wave;
    w.tau = s_tau;
    w.ring = s_ring[wave];
    w.r0 = 0;
    w.nr = 0;
    w.x = x;

    if (wave == 0 && head_hi > 0) wide32_columns<R>(w, row, 0, head_hi);
    if (wn > 0) wide32_body<R>(w, wvp, wn, (uint32_t)(a0 + kElems32 * wv0), A);
    while (w.nr > 0) wide32_flush<R>(w);
    if (wave == kWgWaves - 1 && tail_hi > tail_lo) wide32_columns<R>(w, row, tail_lo, tail_hi);

    int cnt = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      s_list[wave][j * kWave + l] = w.L[j];
      cnt += __popcll(ballot(w.L[j] != 0));
    }
    if (l == 0) {
      s_count[wave] = cnt < a.k ? cnt : a.k;
      s_flags[wave] = w.flags | ((uint32_t)(readlane64(w.L[0], 0) >> 32) == 0xFF800000u ? kPinf : 0u);
    }
    __syncthreads();
    total = 0;
    flags = 0;
#pragma unroll
    for (int o = 0; o < kWgWaves; ++o) {
      total += s_count[o];
      flags |= s_flags[o];
    }
    if (!verify || total >= a.k) break;  // exact, or the speculation verified
    floor = max(exact_floor, rise_floor);
    verify = false;
    if (wn > 0) load_chunk32(A, wvp, wn, 0, (uint32_t)l * 16u);
    __syncthreads();
  }
  if (total > a.k) total = a.k;

  // the four wave lists meet as a tree of register merges (see the 16-bit
  // scan): waves 0 and 2 take the next wave's list, wave 0 then wave 2's
  const int64_t sb = r * S + s;
  uint64_t acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = s_list[wave][j * kWave + l];
  if ((wave & 1) == 0) {
    uint64_t B[R];
#pragma unroll
    for (int j = 0; j < R; ++j) B[j] = s_list[wave + 1][j * kWave + l];
    wide_merge_lists64<R>(acc, B, x);
  }
  if (wave == 2) {  // no other wave reads slot 2 before the barrier
#pragma unroll
    for (int j = 0; j < R; ++j) s_list[2][j * kWave + l] = acc[j];
  }
  __syncthreads();
  if (wave == 0) {
    uint64_t B[R];
#pragma unroll
    for (int j = 0; j < R; ++j) B[j] = s_list[2][j * kWave + l];
    wide_merge_lists64<R>(acc, B, x);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int e = j * kWave + l;
      if (e >= a.k) break;
      if (S == 1) {
        if (e < total) {
          a.out_idx[r * a.k + e] = col_of32(acc[j]);
          a.out_val[r * a.k + e] = value_bits32(acc[j], row);
        } else {
          a.out_idx[r * a.k + e] = TK_FILL_IDX;
          a.out_val[r * a.k + e] = 0x7FC00000u;
        }
      } else if (e < total) {
        __hip_atomic_store(&a.span_list[sb * a.k + e], acc[j], __ATOMIC_RELAXED, kAgent);
      }
    }
  }
  if (S == 1) {
    if (threadIdx.x == 0) {
      a.out_count[r] = total;
      a.out_nonfinite[r] = flags;
    }
    return;
  }
  if (threadIdx.x == 0) {
    __hip_atomic_store(&a.span_count[sb], total, __ATOMIC_RELAXED, kAgent);
    __hip_atomic_store(&a.span_flags[sb], flags, __ATOMIC_RELAXED, kAgent);
  }
  __syncthreads();  // the merge tree's reads of s_list are done; the fold reuses it
  wide32_fold_if_last<R>(a, r, S, row, wave, l, s_list);
}

}  // namespace

hipError_t launch_span_scan32(const ScanArgs32 &a, int64_t rows_in_launch, hipStream_t stream) {
  const int64_t blocks = rows_in_launch * a.spans;
  hipLaunchKernelGGL(span_scan32_kernel, dim3((uint32_t)blocks), dim3(kWgThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_argmax32(const ArgmaxArgs32 &a, int64_t rows_in_launch, hipStream_t stream) {
  if (rows_in_launch <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_scan32_kernel, dim3((uint32_t)(rows_in_launch * a.spans)), dim3(kWgThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_wide_scan32(const ScanArgs32 &a, int64_t rows_in_launch, hipStream_t stream) {
  if (rows_in_launch <= 0) return hipSuccess;
  const dim3 grid((uint32_t)(rows_in_launch * a.spans)), block(kWgThreads);
  if (a.k <= 2 * kWave) {
    hipLaunchKernelGGL(wide_scan32_kernel<2>, grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL(wide_scan32_kernel<4>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace tk
