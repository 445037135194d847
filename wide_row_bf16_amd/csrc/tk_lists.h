// Kept lists longer than a wavefront: a descending list of 64 R entries held
// in R registers per lane (register j, lane i = rank 64 j + i), for the
// multi-register scans (tk_wide.hip: 32-bit in-wave composites; tk_f32.hip:
// 64-bit composites) and their folds.  Meant to be included inside the
// kernels' anonymous namespace (in namespace tk), after tk_wave.h.
//  - One insertion applies the one-register rule max(entry, min(shifted, c))
//    to every register at once, the shift being DPP wave_shr:1 with the
//    previous register's lane 63 as lane 0's source (the row edges' columns;
//    the scans' chunks collect candidates in LDS and merge them as batches).
//  - A sorted batch of 64 cascades down the registers: against register j,
//    the lane-wise max of the register and the reversed batch is the top 64
//    of both (a bitonic sequence, sorted in six stages) and stays; the
//    lane-wise min, sorted likewise, goes on to register j + 1.  Registers
//    whose last entry already beats the batch's first are skipped.
//  - Two sorted lists merge as one bitonic network: A followed by B reversed
//    (the whole union, 2R registers), or the lane-wise max of A and B
//    reversed (their top 64 R, R registers), is a bitonic sequence, which
//    half-cleaners sort -- across registers (register j against j + h), then
//    within each register in six DPP stages.  For two lists of 256 that is
//    about 30 compare-exchange stages, against up to 192 for cascading one
//    list down the other register by register.
#pragma once

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  return ((uint64_t)readlane((uint32_t)(v >> 32), l) << 32) | readlane((uint32_t)v, l);
}

// ---- 32-bit entries ----

template <int R>
__device__ __forceinline__ void wide_insert_one(uint32_t (&L)[R], uint32_t c) {
  uint32_t carry[R];
  carry[0] = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 1; j < R; ++j) carry[j] = readlane(L[j - 1], kWave - 1);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const uint32_t prev = (uint32_t)__builtin_amdgcn_update_dpp((int)carry[j], (int)L[j], 0x138, 0xF, 0xF, false);
    L[j] = max(L[j], min(prev, c));
  }
}

// Sorts (descending) a bitonic sequence held in R registers.
template <int R>
__device__ __forceinline__ void wide_bitonic_regs(uint32_t (&C)[R], const Xchg &x) {
#pragma unroll
  for (int h = R / 2; h >= 1; h /= 2)
#pragma unroll
    for (int j = 0; j < R; ++j)
      if ((j & h) == 0) {
        const uint32_t hi = max(C[j], C[j + h]), lo = min(C[j], C[j + h]);
        C[j] = hi;
        C[j + h] = lo;
      }
#pragma unroll
  for (int j = 0; j < R; ++j) C[j] = bitonic_merge64_desc(C[j], x);
}

// The sorted union of two sorted R-register lists, in 2 R registers.
template <int R>
__device__ __forceinline__ void wide_merge_full(const uint32_t (&A)[R], const uint32_t (&B)[R], uint32_t (&C)[2 * R],
                                                const Xchg &x) {
#pragma unroll
  for (int j = 0; j < R; ++j) {
    C[j] = A[j];
    C[R + j] = partner<63>(B[R - 1 - j], x);
  }
  wide_bitonic_regs<2 * R>(C, x);
}

// The top 64 R of two sorted R-register lists, into A.
template <int R>
__device__ __forceinline__ void wide_merge_top(uint32_t (&A)[R], const uint32_t (&B)[R], const Xchg &x) {
#pragma unroll
  for (int j = 0; j < R; ++j) A[j] = max(A[j], partner<63>(B[R - 1 - j], x));
  wide_bitonic_regs<R>(A, x);
}

// Merges a descending 64-entry batch v into the R-register list L (the top
// 64 R of both stay).
template <int R>
__device__ __forceinline__ void wide_merge_sorted(uint32_t (&L)[R], uint32_t v, const Xchg &x) {
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (!ballot(v != 0)) break;
    // the batch's best does not beat this register's last entry: it passes on whole
    if (readlane(v, 0) <= readlane(L[j], kWave - 1)) continue;
    const uint32_t rv = partner<63>(v, x);
    const uint32_t hi = max(L[j], rv), lo = min(L[j], rv);
    L[j] = bitonic_merge64_desc(hi, x);
    if (j + 1 < R) v = bitonic_merge64_desc(lo, x);
  }
}

template <int R>
__device__ __forceinline__ void wide_merge_batch(uint32_t (&L)[R], uint32_t v, const Xchg &x) {
  wide_merge_sorted<R>(L, sort64_desc(v, x), x);
}

template <int R>
__device__ __forceinline__ uint32_t wide_at(const uint32_t (&L)[R], int rank) {
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < R; ++j)
    if ((rank >> 6) == j) v = readlane(L[j], rank & (kWave - 1));
  return v;
}

// The key of rank `rank` (0 = largest) among R keys per lane (each lane's
// keys in descending order): every register sorted across the wave, then the
// sorted lists merged.
template <int R>
__device__ __forceinline__ uint32_t rank_of_lane_keys(const uint32_t (&t)[R], int rank, const Xchg &x) {
  static_assert(R == 1 || R == 2 || R == 4, "one, two or four keys per lane");
  if constexpr (R == 1) {
    return readlane(sort64_desc(t[0], x), rank);
  } else if constexpr (R == 2) {
    const uint32_t a[1] = {sort64_desc(t[0], x)}, b[1] = {sort64_desc(t[1], x)};
    uint32_t Q[2];
    wide_merge_full<1>(a, b, Q, x);
    return wide_at<2>(Q, rank);
  } else {
    const uint32_t a0[1] = {sort64_desc(t[0], x)}, b0[1] = {sort64_desc(t[1], x)};
    const uint32_t a1[1] = {sort64_desc(t[2], x)}, b1[1] = {sort64_desc(t[3], x)};
    uint32_t Q0[2], Q1[2], P[4];
    wide_merge_full<1>(a0, b0, Q0, x);
    wide_merge_full<1>(a1, b1, Q1, x);
    wide_merge_full<2>(Q0, Q1, P, x);
    return wide_at<4>(P, rank);
  }
}

// ---- 64-bit entries ----

__device__ __forceinline__ uint64_t bitonic_merge64_u64(uint64_t v, const Xchg &x) {
  v = cx_stage64<32, 32>(v, x);
  v = cx_stage64<16, 16>(v, x);
  v = cx_stage64<8, 8>(v, x);
  v = cx_stage64<4, 4>(v, x);
  v = cx_stage64<2, 2>(v, x);
  v = cx_stage64<1, 1>(v, x);
  return v;
}

// Top 64 R of the sorted list A and the sorted list B (R registers each,
// descending, 0 = none), into A, as one bitonic network (see above).
template <int R>
__device__ __forceinline__ void wide_merge_lists64(uint64_t (&A)[R], const uint64_t (&B)[R], const Xchg &x) {
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const uint64_t rb = partner64<63>(B[R - 1 - j], x);
    A[j] = A[j] > rb ? A[j] : rb;
  }
#pragma unroll
  for (int h = R / 2; h >= 1; h /= 2)
#pragma unroll
    for (int j = 0; j < R; ++j)
      if ((j & h) == 0) {
        const uint64_t hi = A[j] > A[j + h] ? A[j] : A[j + h], lo = A[j] > A[j + h] ? A[j + h] : A[j];
        A[j] = hi;
        A[j + h] = lo;
      }
#pragma unroll
  for (int j = 0; j < R; ++j) A[j] = bitonic_merge64_u64(A[j], x);
}

// Cascades the sorted list B (R registers, descending, 0 = none) down A
// register by register (cheap when B holds one short batch, which skips
// the registers it cannot change).
template <int R>
__device__ __forceinline__ void wide_merge_cascade64(uint64_t (&A)[R], const uint64_t (&B)[R], const Xchg &x) {
#pragma unroll
  for (int jb = 0; jb < R; ++jb) {
    uint64_t v = B[jb];
    if (!ballot(v != 0)) break;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (!ballot(v != 0)) break;
      if (readlane64(v, 0) <= readlane64(A[j], kWave - 1)) continue;
      const uint64_t rv = partner64<63>(v, x);
      const uint64_t hi = A[j] > rv ? A[j] : rv, lo = A[j] > rv ? rv : A[j];
      A[j] = bitonic_merge64_u64(hi, x);
      if (j + 1 < R) v = bitonic_merge64_u64(lo, x);
    }
  }
}

template <int R>
__device__ __forceinline__ void wide_insert_one64(uint64_t (&L)[R], uint64_t c) {
  uint64_t carry[R];
  carry[0] = ~0ull;
#pragma unroll
  for (int j = 1; j < R; ++j) carry[j] = readlane64(L[j - 1], kWave - 1);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const uint32_t plo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)carry[j], (int)(uint32_t)L[j], 0x138,
                                                               0xF, 0xF, false);
    const uint32_t phi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(carry[j] >> 32),
                                                               (int)(uint32_t)(L[j] >> 32), 0x138, 0xF, 0xF, false);
    const uint64_t prev = ((uint64_t)phi << 32) | plo;
    const uint64_t lo = prev < c ? prev : c;
    L[j] = L[j] > lo ? L[j] : lo;
  }
}

// Descending bitonic sort of one 64-bit value per lane.
__device__ __forceinline__ uint64_t wide_sort64_u64(uint64_t v, const Xchg &x) {
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

// Merges 64 candidates v (any order, 0 = none) into the list.
template <int R>
__device__ __forceinline__ void wide_merge_batch64(uint64_t (&L)[R], uint64_t v, const Xchg &x) {
  uint64_t B[R];
  B[0] = wide_sort64_u64(v, x);
#pragma unroll
  for (int j = 1; j < R; ++j) B[j] = 0;
  wide_merge_cascade64<R>(L, B, x);
}

template <int R>
__device__ __forceinline__ uint64_t wide_at64(const uint64_t (&L)[R], int rank) {
  uint64_t v = 0;
#pragma unroll
  for (int j = 0; j < R; ++j)
    if ((rank >> 6) == j) v = readlane64(L[j], rank & (kWave - 1));
  return v;
}
