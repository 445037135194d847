// Exact row-wise top-k for 64 < k <= 256 over bf16 and fp16 rows (gfx950).
//
// The operation and its order are those of the k <= 64 scan (TensorFold PR
// #713, change 3: highest score first, the lower column on equal scores, one
// answer whatever the split; the same order key, NaN policy and flags); only
// the kept set is larger than a wavefront.  The pages give the library a
// compile-time max_k; this file is what lets it exceed the lane count.
//
// Kept set.  A wave keeps its 64 R best composites in R VGPRs (R = 2 for
// k <= 128, 4 for k <= 256): register j, lane i holds rank 64 j + i of the
// concatenated descending list.  Candidates do not enter it one by one: the
// lanes of one element position that pass the filter append their
// composites to a ring in LDS (slots from mbcnt over the hit mask: about ten
// instructions for the whole position, against about twenty per entry for
// an insertion into four registers), and every 64 pending ones enter as one
// batch, sorted and cascaded down the registers: against register j, the
// lane-wise max of the register and the reversed batch is the top 64 of both
// (a bitonic sequence, sorted in six stages) and stays; the lane-wise min,
// sorted likewise, is carried to register j + 1.  Registers whose last entry
// already beats the batch's first are skipped.  The k-th and the published
// keys lag the pending candidates, which only lets extra ones through (the
// k = 256 scan is bound by its VALU issue: on 1024 x 151936 rows the ring
// took it from 79-84 to 67-73 us).
// The filter, the trip masks, the chunk loads and the flags are those of the
// k <= 64 scan.  The exact floor is the k-th largest of the 256 lane maxima
// of each wave's first chunk (k lanes hold an element at or above it; on
// few-row splits at k > 128, of each lane's two largest keys); a speculative
// floor (a lower rank of the same sample, verified after the scan and
// followed by a rescan under the exact floor when it fails) spares most of
// the candidates on wide spans.  The four wave lists meet as a tree of
// bitonic list merges in registers; split rows are folded by their last
// workgroup with the same 64-bit list merges.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tk_config.h"
#include "tk_launch.h"
#include "tk_stamps.h"

namespace tk {
namespace {

#include "tk_wave.h"
#include "tk_scan16.h"
#include "tk_lists.h"

// A speculative floor is tried only when each wave's share spans at least this
// many chunks (shorter shares are mostly sample already).
constexpr int kWideSpecChunks = 4;
// Pending candidates of a wave: a ring in LDS (a power of two, above the 63
// left after a batch plus the 512 one vector can add).  A batch leaves it
// once 64 are pending (at 32 or 128 the 1024 x 151936 rows measured 1-4 us
// slower at k = 128 and 256).
constexpr int kWideRing = 1024;

template <int R>
struct WaveWide {
  uint32_t L[R];
  uint32_t kth;    // wave-uniform copy of rank k - 1
  uint32_t ext;    // wave-uniform: keys <= ext are beaten by k entries of other waves (or the floor)
  uint32_t floor;  // wave-uniform floor: only keys > floor are kept
  uint32_t flags;  // wave-uniform TK_NONFINITE_NAN / _NEGINF seen so far
  uint32_t inf;
  int km1;         // k - 1
  int qm1;         // ceil(k / 4) - 1 (< 64)
  int wave;
  uint32_t *tau;   // LDS: [k-th key of each wave][ceil(k/4)-th key of each wave]
  uint32_t *ring;  // LDS: this wave's kWideRing pending composites
  uint32_t r0;     // wave-uniform ring index of the oldest pending composite
  uint32_t nr;     // wave-uniform count of pending composites
  Xchg x;
};

// Candidates c of lanes m, each beating the k-th: one batch when many, else
// one insertion each (a stale k-th only lets extra candidates through, which
// changes ranks >= k only).
template <int R>
__device__ __forceinline__ void wide_offer(WaveWide<R> &w, uint32_t c, uint64_t m) {
  if (__popcll(m) >= kBatchInsert) {
    wide_merge_batch<R>(w.L, c > w.kth ? c : 0u, w.x);
  } else {
    do {
      const int l = __builtin_ctzll(m);
      m &= m - 1;
      wide_insert_one<R>(w.L, readlane(c, l));
    } while (m);
  }
  w.kth = wide_at<R>(w.L, w.km1);
}

// The threshold sharing of the k <= 64 scan: a wave's k-th key bounds the
// others (on equal keys the left wave wins), and the smallest ceil(k/4)-th
// key of the four bounds every wave (k entries of the workgroup beat what is
// below it).
__device__ __forceinline__ uint32_t wide_bound(const uint32_t *s_tau, int wave) {
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

template <int R>
__device__ __forceinline__ void wide_publish(WaveWide<R> &w) {
  const uint32_t q = readlane(w.L[0], w.qm1) >> 16;
  if (lane_id() == 0) {
    __hip_atomic_store(&w.tau[w.wave], w.kth >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(&w.tau[kWgWaves + w.wave], q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// The oldest min(64, pending) candidates leave the ring as one batch: sorted
// and cascaded into the list (the top 64 R of both stay); the k-th and the
// published keys follow the list.
template <int R>
__device__ __forceinline__ void wide_flush(WaveWide<R> &w) {
  __builtin_amdgcn_wave_barrier();  // the ring's stores above precede its loads
  const uint32_t take = min(w.nr, (uint32_t)kWave);
  const uint32_t l = (uint32_t)lane_id();
  const uint32_t v = l < take ? w.ring[(w.r0 + l) & (kWideRing - 1)] : 0u;
  w.r0 = (w.r0 + take) & (kWideRing - 1);
  w.nr -= take;
  wide_merge_batch<R>(w.L, v, w.x);
  w.kth = wide_at<R>(w.L, w.km1);
  wide_publish<R>(w);
}

// The eight per-element tests of one tripped vector against T on the raw
// bits (lanes `valid`); for each element position with hits, the composites
// of the hitting lanes are appended to the ring (their slots counted by
// mbcnt over the hit mask), whatever their number.  NONNEG: T >= 0, so only
// non-negative bit patterns pass, with key = bits + 0x8000.  NaN patterns
// that pass are flagged, never kept.  A composite that passes beats the k-th
// of the list (its key exceeds the k-th's key); pending composites are not
// in the list yet, so the k-th and the published keys lag, which only lets
// extra candidates through (they land at ranks >= k).
template <int R, bool NONNEG>
__device__ __forceinline__ void wide_take_vector(WaveWide<R> &w, uint4 d, uint32_t inv0, uint64_t valid,
                                                 const Filter &f) {
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
  uint64_t m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t word = dw[e >> 1];
    const uint32_t b = (e & 1) ? word >> 16 : word & 0xFFFFu;
    m[e] = (NONNEG ? lanes_sgt((int32_t)(int16_t)b, f.t16) : lanes_ult(b, f.tu)) & valid;
  }
  uint64_t nan = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (!m[e]) continue;
    const uint32_t word = dw[e >> 1];
    const uint32_t b = (e & 1) ? word >> 16 : word & 0xFFFFu;
    const uint32_t key = NONNEG ? (b > w.inf ? 0u : b | 0x8000u) : order_key(b, w.inf);
    const uint64_t h = m[e] & ~lanes_eq(key, 0u);
    nan |= m[e] & ~h;
    if (h) {
      const uint32_t slot = __builtin_amdgcn_mbcnt_hi((uint32_t)(h >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)h, w.r0 + w.nr));
      if (__builtin_amdgcn_inverse_ballot_w64(h)) w.ring[slot & (kWideRing - 1)] = (key << 16) | (inv0 - (uint32_t)e);
      w.nr += (uint32_t)__popcll(h);
    }
  }
  if (nan) w.flags |= kNan;
}

// One loaded chunk (vector u of this lane = the wave's vector first + 64 u +
// lane): trip masks against T at the chunk start, then for each tripped
// vector the composites above T go to the ring; every 64 pending ones are
// merged into the list as a batch, after which T is taken again.  Positive
// NaN patterns pass the value test and are flagged here.
template <int R>
__device__ __forceinline__ void wide_chunk(WaveWide<R> &w, const uint4 (&v)[kChunkVecs], uint32_t first, uint32_t nvec,
                                           int64_t col_first, int64_t base) {
  w.ext = max(wide_bound(w.tau, w.wave), w.floor);
  const Filter f0 = filter_for(max(w.kth >> 16, w.ext), w.flags, w.inf);
  uint64_t vt[kChunkVecs], ft[kChunkVecs];
  lane_trips<kChunkVecs>(v, f0, vt, ft);
  uint64_t any_v = 0;
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    const uint64_t valid = lanes_ult(first + (uint32_t)(u * kWave + lane_id()), nvec);
    vt[u] &= valid;
    ft[u] &= valid;
    any_v |= vt[u];
    if (ft[u]) take_flags(w.flags, w.inf, v[u], ft[u], f0.ftrip);
  }
  if (!any_v) return;
  const uint32_t l = (uint32_t)lane_id();
  // vectors rotated through x0 (no dynamic index into register arrays)
  uint4 x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
  uint64_t m0 = vt[0], m1 = vt[1], m2 = vt[2], m3 = vt[3];
  uint32_t iv = 0xFFFFu - (uint32_t)(col_first - base) - (uint32_t)kVecElems * (first + l);
  Filter f = f0;
#pragma unroll 1
  for (int u = 0; u < kChunkVecs; ++u) {
    if (m0) {
      if (f.nonneg) wide_take_vector<R, true>(w, x0, iv, m0, f);
      else wide_take_vector<R, false>(w, x0, iv, m0, f);
      if (w.nr >= (uint32_t)kWave) {
        do {
          wide_flush<R>(w);
        } while (w.nr >= (uint32_t)kWave);
        f = filter_for(max(w.kth >> 16, w.ext), w.flags, w.inf);
      }
    }
    m0 = m1;
    m1 = m2;
    m2 = m3;
    m3 = 0;
    if (!(m0 | m1 | m2)) break;
    x0 = x1;
    x1 = x2;
    x2 = x3;
    iv -= (uint32_t)(kWave * kVecElems);
  }
}

// Columns [lo, hi) one per lane (row edges, tiny spans).
template <int R>
__device__ void wide_columns(WaveWide<R> &w, const uint16_t *row, int64_t lo, int64_t hi, int64_t base) {
  for (int64_t c0 = lo; c0 < hi; c0 += kWave) {
    const int64_t col = c0 + lane_id();
    const bool valid = col < hi;
    const uint32_t b = valid ? (uint32_t)row[col] : 0u;
    const uint32_t key = order_key(b, w.inf);
    if (ballot(valid && (b & 0x7FFFu) > w.inf)) w.flags |= kNan;
    if (ballot(valid && b == (0x8000u | w.inf))) w.flags |= kNinf;
    const uint32_t c = (valid && key > w.ext) ? (key << 16) | (0xFFFFu - (uint32_t)(col - base)) : 0u;
    const uint64_t m = lanes_ugt(c, w.kth);
    if (m) wide_offer<R>(w, c, m);
  }
}

// ---- R-register lists of 64-bit composites (the fold of split rows) ----

// Last-workgroup fold of a split row (the protocol of the k <= 64 scan):
// arrival counted after the span's stores completed; the last arrival loads
// every span list with agent-scope loads, each wave folding lists wave,
// wave + 4, ..., then a tree over the four waves through LDS.
template <int R>
__device__ __forceinline__ void wide_fold_if_last(const ScanArgs &a, int64_t r, int S, const uint16_t *row, int wave,
                                                  int l, uint64_t (*s_acc)[kWave * R]) {
  __shared__ int s_last;
  __shared__ int32_t s_cnt[kWgWaves];
  __shared__ uint32_t s_fl[kWgWaves];
  const int64_t rb = r - a.row0;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  TK_STAMP(8);
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&a.row_done[rb], 1, __ATOMIC_RELAXED, kAgent) == S - 1;
  __syncthreads();
  TK_STAMP(9);
  if (!s_last) return;
  TK_STAMP_VALUE(13, 1);
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
  TK_STAMP(10);
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
  TK_STAMP(11);
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
        a.out_idx[ob + e] = (int32_t)(col_of(acc[j]) + a.col_base);
        a.out_val[ob + e] = value_bits(acc[j], row);
      } else {
        a.out_idx[ob + e] = TK_FILL_IDX;
        a.out_val[ob + e] = (uint16_t)TK_FILL_VAL;
      }
    }
  }
  if (l == 0) {
    a.out_count[r] = cnt;
    a.out_nonfinite[r] = fl;
    __hip_atomic_store(&a.row_done[rb], 0, __ATOMIC_RELAXED, kAgent);
  }
  TK_STAMP(12);
}

template <int R>
__global__ __launch_bounds__(kWgThreads) void wide_scan_kernel(ScanArgs a) {
  __shared__ uint64_t s_list[kWgWaves][kWave * R];
  __shared__ int32_t s_count[kWgWaves];
  __shared__ uint32_t s_flags[kWgWaves];
  __shared__ uint32_t s_tau[2 * kWgWaves];
  __shared__ uint32_t s_samp[2 * kWgWaves][kWave];
  __shared__ uint32_t s_ring[kWgWaves][kWideRing];

  const int64_t blk = blockIdx.x;
  const int64_t r = a.row0 + blk / a.spans;
  const int s = (int)(blk % a.spans);
  const int S = a.spans;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int l = lane_id();
  const uint16_t *row = a.in + r * a.stride;
  TK_STAMP(0);
  TK_STAMP_HW(14);
  TK_STAMP_VALUE(13, 0);

  // the span and wave shares of the k <= 64 scan
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
  const uint4 *wvp = reinterpret_cast<const uint4 *>(row + a0) + wv0;
  const uint32_t wn = (uint32_t)(wv1 - wv0);

  // Floors from the workgroup's first chunk, as in the k <= 64 scan: exact =
  // the k-th largest of the 256 lane maxima (k lanes hold an element at or
  // above it); speculative = the spec_rank-th largest (spec_rank < k, chosen
  // on the host from k and the span width), verified after the scan -- if the
  // lists then hold k entries, everything dropped is beaten by k kept ones;
  // otherwise the span is scanned again under the exact floor.  With k > 128
  // and no speculation (few-row splits, whose spans are too short for it) the
  // k-th lane maximum is nearly the smallest one, so there the exact floor
  // comes from each lane's two largest keys (512 distinct elements): on
  // 15 x 98592 rows at k = 256 it admits a fifth of the elements and took the
  // call from 51.6 to 43.5 us.  Elsewhere the second sort and the extra
  // merges cost more than they save (k = 128, and every speculating span).
  const Xchg x = make_xchg();
  uint4 A[kChunkVecs];
  if (wn > 0) load_chunk(A, wvp, wn, 0, (uint32_t)l * 16u);
  const bool speculate =
      a.spec_rank > 0 && !a.exact && n / kWgWaves >= (int64_t)kWideSpecChunks * kChunkVecs * kWave;
  const bool pairs = R == 4 && a.k > 2 * kWave && !speculate;
  uint32_t m1 = 0;  // this lane's largest key of the first chunk
  {
    uint32_t m2 = 0;
    if (wn > 0) {
      if (pairs) lane_top2_keys(A, 0, wn, a.inf, &m1, &m2);
      else m1 = lane_max_key(A, 0, wn, a.inf);
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
  // Rows that rise along this wave's share (nearly every lane's first-chunk
  // maximum in its last vector): a floor of its own from the share's final
  // 256 vectors, as in the k <= 64 scan, from each lane's R largest keys there
  // (64 R distinct elements, so the k-th exists); exact, so it also holds if
  // the speculation fails.  The choice to speculate stays the same in every
  // wave of the workgroup.
  uint32_t rise_floor = 0;
  if (wn >= (uint32_t)(kLookChunks * kChunkVecs * kWave) &&
      __popcll(ballot(m1 > 0 && vec_max_key(A[kChunkVecs - 1], a.inf) >= m1)) >= kLookLanes) {
    constexpr uint32_t kStep = (uint32_t)kChunkVecs * kWave;
    const uint32_t last = wn - kStep;  // the share's last kStep vectors: every lane holds four
    uint4 L[kChunkVecs];
    load_chunk(L, wvp, wn, last, (uint32_t)l * 16u);
    uint32_t t[R];
    lane_top_keys<R>(L, last, wn, a.inf, t);
    const uint32_t te = rank_of_lane_keys<R>(t, a.k - 1, x);
    if (te > 1) rise_floor = te - 1;
  }
  uint32_t floor = exact_floor;
  bool verify = false;
  if (spec_floor > exact_floor) {
    floor = spec_floor;
    verify = true;
  }
  floor = max(floor, rise_floor);
  TK_STAMP(1);

  WaveWide<R> w;
  int total = 0;
  uint32_t flags = 0;
  for (;;) {
    if (threadIdx.x < 2 * kWgWaves) s_tau[threadIdx.x] = 0;
    __syncthreads();
    w.x = x;
#pragma unroll
    for (int j = 0; j < R; ++j) w.L[j] = 0;
    w.kth = 0;
    w.ext = floor;
    w.floor = floor;
    w.flags = 0;
    w.inf = a.inf;
    w.km1 = a.k - 1;
    w.qm1 = (a.k + kWgWaves - 1) / kWgWaves - 1;
    w.wave = wave;
    w.tau = s_tau;
    w.ring = s_ring[wave];
    w.r0 = 0;
    w.nr = 0;

    if (wave == 0 && head_hi > 0) wide_columns<R>(w, row, 0, head_hi, base);
    if (wn > 0) {
      constexpr uint32_t kStep = (uint32_t)kChunkVecs * kWave;
      const uint32_t lane_off = (uint32_t)l * 16u;
      const int64_t col_first = a0 + kVecElems * wv0;
      uint4 B[kChunkVecs];
      // progress-based issue priority, as in the k <= 64 scan (waves that are
      // behind issue first), here in quarters of the share: on 1024 x 151936
      // rows it took k = 128 from 68.1 to 62.4 us and k = 256 from 96.9 to
      // 85.2 us; steps at 1/2, 3/4, 9/10 measured 0.1-0.7 us slower
      const uint32_t q1 = wn / 4, q2 = wn / 2, q3 = wn - wn / 4;
      __builtin_amdgcn_s_setprio(3);
      for (uint32_t first = 0; first < wn; first += 2 * kStep) {
        if (first >= q3) __builtin_amdgcn_s_setprio(0);
        else if (first >= q2) __builtin_amdgcn_s_setprio(1);
        else if (first >= q1) __builtin_amdgcn_s_setprio(2);
        load_chunk(B, wvp, wn, first + kStep, lane_off);
        wide_chunk<R>(w, A, first, wn, col_first, base);
        if (first + kStep >= wn) break;
        load_chunk(A, wvp, wn, first + 2 * kStep, lane_off);
        wide_chunk<R>(w, B, first + kStep, wn, col_first, base);
      }
    }
    while (w.nr > 0) wide_flush<R>(w);
    if (wave == kWgWaves - 1 && tail_hi > tail_lo) wide_columns<R>(w, row, tail_lo, tail_hi, base);
    TK_WAVE_STAMP(2 + wave);

    // the wave's list, its count and flags to LDS
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      s_list[wave][j * kWave + l] = composite64(w.L[j], base);
      cnt += __popcll(ballot(w.L[j] != 0));
    }
    if (l == 0) {
      s_count[wave] = cnt < a.k ? cnt : a.k;
      s_flags[wave] = w.flags | ((readlane(w.L[0], 0) >> 16) == 0x8000u + a.inf ? kPinf : 0u);
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
    floor = max(exact_floor, rise_floor);
    verify = false;
    if (wn > 0) load_chunk(A, wvp, wn, 0, (uint32_t)l * 16u);
    __syncthreads();  // every wave has read the counts above
  }
  if (total > a.k) total = a.k;

  // The four wave lists meet as a tree of register merges (as in the k <= 64
  // scan): waves 0 and 2 merge the next wave's list into theirs, then wave 0
  // merges in wave 2's result and writes the top k.  A wave's entries past
  // its count are empty zeros or beaten by k of its own, so they can only
  // land at merged ranks >= k and whole lists are merged.  (Ranking every
  // entry by binary searches in the other three lists read ~200 KB of LDS
  // per workgroup at k = 256.)
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
          a.out_idx[r * a.k + e] = (int32_t)(col_of(acc[j]) + a.col_base);
          a.out_val[r * a.k + e] = value_bits(acc[j], row);
        } else {
          a.out_idx[r * a.k + e] = TK_FILL_IDX;
          a.out_val[r * a.k + e] = (uint16_t)TK_FILL_VAL;
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
    TK_STAMP(7);
    return;
  }
  if (threadIdx.x == 0) {
    __hip_atomic_store(&a.span_count[sb], total, __ATOMIC_RELAXED, kAgent);
    __hip_atomic_store(&a.span_flags[sb], flags, __ATOMIC_RELAXED, kAgent);
  }
  TK_STAMP(7);
  // the merge tree's reads of s_list are done once every wave has passed this
  // point; the fold then reuses s_list as its exchange buffer
  __syncthreads();
  wide_fold_if_last<R>(a, r, S, row, wave, l, s_list);
}

}  // namespace

hipError_t launch_wide_scan(const ScanArgs &a, int64_t rows_in_launch, hipStream_t stream) {
  if (rows_in_launch <= 0) return hipSuccess;
  const dim3 grid((uint32_t)(rows_in_launch * a.spans)), block(kWgThreads);
  if (a.k <= 2 * kWave) {
    hipLaunchKernelGGL(wide_scan_kernel<2>, grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL(wide_scan_kernel<4>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace tk

#ifdef TK_STAGE_STAMPS
// Copies the stage table of the last stamped wide-scan launches (bytes at
// most its size); synchronous.  Present in the stamp build only.
extern "C" int tk_stage_stamps_wide(void *dst, size_t bytes) {
  if (bytes > sizeof(tk_stamp_table)) return 1;
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(tk_stamp_table), bytes) == hipSuccess ? 0 : 1;
}
#endif
