// Scan helpers for 16-bit sign-magnitude rows (bf16, fp16) shared by the
// scan kernels of tk_kernels.hip (k <= 64, k = 1) and tk_wide.hip (k > 64):
// the order key, the raw-bit fast filter and its lane trip masks, flag
// detection, the streaming chunk loads, and the 64-bit composites that carry
// an entry across waves and spans.  Meant to be included inside the kernels'
// anonymous namespace (in namespace tk), after tk_wave.h.
#pragma once

typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr uint32_t kBf16Inf = 0x7F80u;  // bf16 +inf pattern (fp16: 0x7C00, passed at run time)

__device__ __forceinline__ void cx(uint32_t &a, uint32_t &b) {  // a <- max, b <- min
  const uint32_t hi = max(a, b);
  b = min(a, b);
  a = hi;
}

// Descending sort of eight values (a 19-comparator network).
__device__ __forceinline__ void sort8_desc(uint32_t (&c)[8]) {
  cx(c[0], c[2]); cx(c[1], c[3]); cx(c[4], c[6]); cx(c[5], c[7]);
  cx(c[0], c[4]); cx(c[1], c[5]); cx(c[2], c[6]); cx(c[3], c[7]);
  cx(c[0], c[1]); cx(c[2], c[3]); cx(c[4], c[5]); cx(c[6], c[7]);
  cx(c[2], c[4]); cx(c[3], c[5]);
  cx(c[1], c[4]); cx(c[3], c[6]);
  cx(c[1], c[2]); cx(c[3], c[4]); cx(c[5], c[6]);
}

// inf = the format's +inf pattern (bf16 0x7F80, fp16 0x7C00): magnitudes
// above it are NaN.
__device__ __forceinline__ uint32_t order_key(uint32_t b, uint32_t inf = kBf16Inf) {
  const uint32_t mag = b & 0x7FFFu;
  const uint32_t key = (b & 0x8000u) ? 0x8000u - mag : 0x8000u + mag;
  return mag > inf ? 0u : key;
}

// Wave-uniform thresholds of the fast filter from T = max(k-th kept key, ext):
// an element may matter only if its key exceeds T.
struct Filter {
  bool nonneg;     // T >= +-0: trip when int16(bits) > t16
  int32_t t16;     // T's magnitude (T >= 0)
  uint32_t tu;     // T < 0: trip when uint16(bits) < tu (= T's bits); 0x10000 while nothing bounds it
  uint32_t ftrip;  // trip when uint16(bits) >= ftrip: -inf / NaN patterns not flagged yet
};

// The filter for threshold key tkey (wave-uniform), given the flags already
// raised and the format's +inf pattern.
__device__ __forceinline__ Filter filter_for(uint32_t tkey, uint32_t flags, uint32_t inf) {
  Filter f;
  f.nonneg = tkey >= 0x8000u;
  f.t16 = (int32_t)tkey - 0x8000;
  f.tu = 0x10000u - tkey;
  const uint32_t ninf = 0x8000u | inf;
  f.ftrip = (flags & kNinf) ? ((flags & kNan) ? 0x10000u : ninf + 1u) : ninf;
  return f;
}

__device__ __forceinline__ v2i16 as_i16x2(uint32_t x) { return __builtin_bit_cast(v2i16, x); }
__device__ __forceinline__ v2u16 as_u16x2(uint32_t x) { return __builtin_bit_cast(v2u16, x); }

// vt[u]: the lanes whose vector u holds an element whose key may exceed T;
// ft[u]: the lanes whose vector u holds a -inf / NaN pattern not flagged yet.
// (Never a false negative; a false positive only costs the exact path.)
template <int N>
__device__ __forceinline__ void lane_trips(const uint4 (&v)[N], const Filter &f, uint64_t (&vt)[N], uint64_t (&ft)[N]) {
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const v2u16 h = __builtin_elementwise_max(__builtin_elementwise_max(as_u16x2(v[u].x), as_u16x2(v[u].y)),
                                              __builtin_elementwise_max(as_u16x2(v[u].z), as_u16x2(v[u].w)));
    ft[u] = lanes_uge(max((uint32_t)h.x, (uint32_t)h.y), f.ftrip);
  }
  if (f.nonneg) {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const v2i16 a = __builtin_elementwise_max(__builtin_elementwise_max(as_i16x2(v[u].x), as_i16x2(v[u].y)),
                                                __builtin_elementwise_max(as_i16x2(v[u].z), as_i16x2(v[u].w)));
      vt[u] = lanes_sgt(max((int32_t)a.x, (int32_t)a.y), f.t16);
    }
  } else {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const v2u16 lo = __builtin_elementwise_min(__builtin_elementwise_min(as_u16x2(v[u].x), as_u16x2(v[u].y)),
                                                 __builtin_elementwise_min(as_u16x2(v[u].z), as_u16x2(v[u].w)));
      vt[u] = lanes_ult(min((uint32_t)lo.x, (uint32_t)lo.y), f.tu);
    }
  }
}

// Flags the -inf / NaN patterns at or above ftrip in the vectors of lanes
// `lanes`; nothing is kept here (a -inf that can be kept also passes T).
__device__ __forceinline__ void take_flags(uint32_t &flags, uint32_t inf, uint4 d, uint64_t lanes, uint32_t ftrip) {
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t word = dw[e >> 1];
    const uint32_t b = (e & 1) ? word >> 16 : word & 0xFFFFu;
    const uint64_t m = lanes_uge(b, ftrip) & lanes;
    if (m & lanes_eq(b, 0x8000u | inf)) flags |= kNinf;
    if (m & lanes_ugt(b, 0x8000u | inf)) flags |= kNan;
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer format on gfx9-family parts
// Cache policy of the streaming loads: nontemporal (the `nt` bit on gfx950).
// The input is read once, so it should not displace lines in the caches; on
// a plain read of 311 MB this lifts the achieved rate from ~5.7 to ~6.5 TB/s.
constexpr int kLoadPolicy = 2;

// Loads vectors [first, first + kChunkVecs * 64) of the wave's nvec vectors at
// vp.  The descriptor is rebuilt per chunk in scalar registers (base advanced,
// range shrunk), so the per-lane offset stays loop-invariant and the range
// check zero-fills lanes past the end -- every load is issued unconditionally
// and the wait counts are the same on every path.
__device__ __forceinline__ void load_chunk(uint4 (&dst)[kChunkVecs], const uint4 *vp, uint32_t nvec, uint32_t first,
                                           uint32_t lane_off) {
  // all wave-uniform; readfirstlane keeps the descriptor in scalar registers
  first = (uint32_t)__builtin_amdgcn_readfirstlane((int)first);
  nvec = (uint32_t)__builtin_amdgcn_readfirstlane((int)nvec);
  const uint32_t left = (uint32_t)__builtin_amdgcn_readfirstlane((int)(nvec - min(first, nvec)));
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)(vp + first), (short)0, (int)(left * 16u), kBufferWord3);
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    const u32x4 x =
        __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(lane_off + (uint32_t)(u * kWave * 16)), 0, kLoadPolicy);
    dst[u] = make_uint4(x.x, x.y, x.z, x.w);
  }
}

// This lane's largest order key in a loaded chunk (vectors [first, first +
// kChunkVecs * 64) of nvec; vectors at or past nvec count as key 0, as does
// NaN), from the packed 16-bit maximum and minimum of its halves: if some
// pattern is non-negative as int16, the largest int16 is the largest value
// (a +NaN there gives key 0); otherwise every pattern is negative and the
// smallest uint16 (the smallest magnitude) is the largest value.  A lane
// whose key comes out 0 or below its true maximum only weakens the floors
// built from these keys (each key is still that of one of the lane's
// elements, or 0).  Sorted over the wave, these give the floors of the scans.
__device__ __forceinline__ uint32_t lane_max_key(const uint4 (&v)[kChunkVecs], uint32_t first, uint32_t nvec,
                                                 uint32_t inf) {
  v2i16 smax = {(short)-32768, (short)-32768};
  v2u16 umin = {(unsigned short)0xFFFF, (unsigned short)0xFFFF};
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    if (first + (uint32_t)(u * kWave + lane_id()) >= nvec) continue;
    smax = __builtin_elementwise_max(smax, __builtin_elementwise_max(
                                               __builtin_elementwise_max(as_i16x2(v[u].x), as_i16x2(v[u].y)),
                                               __builtin_elementwise_max(as_i16x2(v[u].z), as_i16x2(v[u].w))));
    umin = __builtin_elementwise_min(umin, __builtin_elementwise_min(
                                               __builtin_elementwise_min(as_u16x2(v[u].x), as_u16x2(v[u].y)),
                                               __builtin_elementwise_min(as_u16x2(v[u].z), as_u16x2(v[u].w))));
  }
  const int32_t m = max((int32_t)smax.x, (int32_t)smax.y);
  const uint32_t n = min((uint32_t)umin.x, (uint32_t)umin.y);
  if (first + (uint32_t)lane_id() >= nvec) return 0u;  // no vector of this lane in range
  return m >= 0 ? ((uint32_t)m > inf ? 0u : (uint32_t)m | 0x8000u) : order_key(n, inf);
}

// The largest order key of one vector of this lane, by the packed rule of
// lane_max_key (never above the true maximum key).
__device__ __forceinline__ uint32_t vec_max_key(uint4 v, uint32_t inf) {
  const v2i16 smax = __builtin_elementwise_max(__builtin_elementwise_max(as_i16x2(v.x), as_i16x2(v.y)),
                                               __builtin_elementwise_max(as_i16x2(v.z), as_i16x2(v.w)));
  const v2u16 umin = __builtin_elementwise_min(__builtin_elementwise_min(as_u16x2(v.x), as_u16x2(v.y)),
                                               __builtin_elementwise_min(as_u16x2(v.z), as_u16x2(v.w)));
  const int32_t m = max((int32_t)smax.x, (int32_t)smax.y);
  const uint32_t n = min((uint32_t)umin.x, (uint32_t)umin.y);
  return m >= 0 ? ((uint32_t)m > inf ? 0u : (uint32_t)m | 0x8000u) : order_key(n, inf);
}

// This lane's R largest keys in a loaded chunk, in descending order (zeros
// for missing ones): R distinct elements.
template <int R>
__device__ __forceinline__ void lane_top_keys(const uint4 (&v)[kChunkVecs], uint32_t first, uint32_t nvec,
                                              uint32_t inf, uint32_t (&t)[R]) {
#pragma unroll
  for (int j = 0; j < R; ++j) t[j] = 0;
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    const uint32_t dw[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    const bool in = first + (uint32_t)(u * kWave + lane_id()) < nvec;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t key = in ? order_key((dw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu, inf) : 0u;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const uint32_t hi = max(t[j], key);
        key = min(t[j], key);
        t[j] = hi;
      }
    }
  }
}

// The same lane maximum, key by key over the eight halves of each vector
// (exact for lanes with NaN too).  The k <= 64 scan takes it for rows that
// one workgroup scans whole: with the packed maximum the workgroups of
// 1024 x 151936 rows left their floors sooner and together, and the call
// measured 1 us slower (56.4 -> 57.5 us; split rows and the k > 64 scan
// measured 0.3-2 us faster with the packed one).
__device__ __forceinline__ uint32_t lane_max_key_keys(const uint4 (&v)[kChunkVecs], uint32_t first, uint32_t nvec,
                                                      uint32_t inf) {
  uint32_t m = 0;
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    const uint32_t dw[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    uint32_t mu = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) mu = max(mu, order_key((dw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu, inf));
    if (first + (uint32_t)(u * kWave + lane_id()) < nvec) m = max(m, mu);
  }
  return m;
}

// This lane's two largest order keys in a loaded chunk (same rules as
// lane_max_key; *m2 is 0 when the lane holds fewer than two keys).  They are
// distinct elements, so the k-th largest of all lanes' pairs has k elements
// at or above it: a floor twice as deep as the lane maxima give, which the
// k > 64 scans need (with k = 256 and 256 lanes the k-th lane maximum is the
// smallest one).
__device__ __forceinline__ void lane_top2_keys(const uint4 (&v)[kChunkVecs], uint32_t first, uint32_t nvec, uint32_t inf,
                                               uint32_t *m1, uint32_t *m2) {
  uint32_t a = 0, b = 0;
#pragma unroll
  for (int u = 0; u < kChunkVecs; ++u) {
    const uint32_t dw[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    const bool in = first + (uint32_t)(u * kWave + lane_id()) < nvec;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t key = in ? order_key((dw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu, inf) : 0u;
      b = max(b, min(a, key));
      a = max(a, key);
    }
  }
  *m1 = a;
  *m2 = b;
}

__device__ __forceinline__ uint64_t composite64(uint32_t c32, int64_t base) {
  if (!c32) return 0;
  const uint32_t col = (uint32_t)(base + (int64_t)(0xFFFFu - (c32 & 0xFFFFu)));
  return ((uint64_t)(c32 >> 16) << 32) | (uint64_t)(0xFFFFFFFFu - col);
}

__device__ __forceinline__ int32_t col_of(uint64_t x) { return (int32_t)(0xFFFFFFFFu - (uint32_t)x); }

// bf16 bits of an entry: the key is invertible except for the shared key of
// +0 and -0, whose sign is read back from the input.
__device__ __forceinline__ uint16_t value_bits(uint64_t x, const uint16_t *row) {
  const uint32_t key = (uint32_t)(x >> 32);
  if (key > 0x8000u) return (uint16_t)(key - 0x8000u);
  if (key < 0x8000u) return (uint16_t)(0x8000u | (0x8000u - key));
  return row[col_of(x)];
}

// Signed composites key << 32 | (0x7FFFFFFF - column) << 1 | sign: the same
// order as the plain ones for distinct columns, and the value's sign bit
// carried along, so an entry's bits come back without the input (-0 and +0
// share a key).
__device__ __forceinline__ int32_t signed_col(uint64_t x) { return (int32_t)(0x7FFFFFFFu - ((uint32_t)x >> 1)); }

__device__ __forceinline__ uint16_t signed_value_bits(uint64_t x) {
  const uint32_t key = (uint32_t)(x >> 32);
  if (key > 0x8000u) return (uint16_t)(key - 0x8000u);
  if (key < 0x8000u) return (uint16_t)(0x8000u | (0x8000u - key));
  return (uint16_t)(((uint32_t)x & 1u) << 15);
}
