// Wave-level helpers shared by the scan kernels (tk_kernels.hip, tk_f32.hip):
// lane masks from compares, lane exchanges by DPP and gfx950 permlane swaps,
// bitonic sorts and merges of one value per lane (32- and 64-bit), and the
// one-element insertion into a descending per-lane list.  Meant to be
// included inside the kernels' own anonymous namespace (in namespace tk).
#pragma once

constexpr uint32_t kNan = TK_NONFINITE_NAN;
constexpr uint32_t kPinf = TK_NONFINITE_POSINF;
constexpr uint32_t kNinf = TK_NONFINITE_NEGINF;

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Lane masks straight from a compare (one v_cmp writing a scalar register
// pair; no detour of the per-lane result through a vector register).
__device__ __forceinline__ uint64_t lanes_sgt(int32_t a, int32_t b) { return __builtin_amdgcn_sicmp(a, b, 38); }
__device__ __forceinline__ uint64_t lanes_ugt(uint32_t a, uint32_t b) { return __builtin_amdgcn_uicmp(a, b, 34); }
__device__ __forceinline__ uint64_t lanes_uge(uint32_t a, uint32_t b) { return __builtin_amdgcn_uicmp(a, b, 35); }
__device__ __forceinline__ uint64_t lanes_ult(uint32_t a, uint32_t b) { return __builtin_amdgcn_uicmp(a, b, 36); }
constexpr int kAgent = __HIP_MEMORY_SCOPE_AGENT;
__device__ __forceinline__ uint64_t lanes_eq(uint32_t a, uint32_t b) { return __builtin_amdgcn_uicmp(a, b, 32); }

__device__ __forceinline__ uint32_t readlane(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Lane exchanges.  Partners at xor distances 1, 2, 3 (quad_perm), 7
// (row_half_mirror), 15 (row_mirror) and 8 (row_ror:8) are single DPP moves;
// distance 4 takes one of two row rotations; distances 16 and 32 use the
// gfx950 permlane swaps.  Which rotation, and which half of a swap, holds
// lane ^ d is found once per wave from lane ids (Xchg), so nothing here depends
// on a rotate or swap direction convention.
struct Xchg {
  bool ror4;  // row_ror:4 delivers lane ^ 4 to this lane (else row_ror:12 does)
  bool sw16;  // the first result of permlane16_swap(v, v) holds lane ^ 16
  bool sw32;  // the first result of permlane32_swap(v, v) holds lane ^ 32
};

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ Xchg make_xchg() {
  const uint32_t l = (uint32_t)lane_id();
  Xchg x;
  x.ror4 = dpp<0x124>(l) == (l ^ 4u);
  const auto s16 = __builtin_amdgcn_permlane16_swap(l, l, false, false);
  x.sw16 = s16[0] == (l ^ 16u);
  const auto s32 = __builtin_amdgcn_permlane32_swap(l, l, false, false);
  x.sw32 = s32[0] == (l ^ 32u);
  return x;
}

// v from lane (lane ^ MASK).
template <int MASK>
__device__ __forceinline__ uint32_t partner(uint32_t v, const Xchg &x) {
  if constexpr (MASK == 1) {
    return dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  } else if constexpr (MASK == 2) {
    return dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  } else if constexpr (MASK == 3) {
    return dpp<0x1B>(v);  // quad_perm [3,2,1,0]
  } else if constexpr (MASK == 7) {
    return dpp<0x141>(v);  // row_half_mirror
  } else if constexpr (MASK == 15) {
    return dpp<0x140>(v);  // row_mirror
  } else if constexpr (MASK == 8) {
    return dpp<0x128>(v);  // row_ror:8
  } else if constexpr (MASK == 4) {
    const uint32_t a = dpp<0x124>(v), b = dpp<0x12C>(v);  // row_ror:4, row_ror:12
    return x.ror4 ? a : b;
  } else if constexpr (MASK == 16) {
    const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return x.sw16 ? s[0] : s[1];
  } else if constexpr (MASK == 32) {
    const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return x.sw32 ? s[0] : s[1];
  } else if constexpr (MASK == 31) {
    return partner<16>(partner<15>(v, x), x);
  } else {
    static_assert(MASK == 63, "unsupported lane distance");
    return partner<32>(partner<31>(v, x), x);
  }
}

// One compare-exchange stage over the 64 lanes: the lane whose LOW bit is
// clear keeps the larger value.
template <int MASK, int LOW>
__device__ __forceinline__ uint32_t cx_stage(uint32_t v, const Xchg &x) {
  const uint32_t y = partner<MASK>(v, x);
  return (lane_id() & LOW) ? min(v, y) : max(v, y);
}

// Descending bitonic sort across the 64 lanes, in the form where every block
// of `size` lanes starts with a mirrored compare (lane ^ (size - 1)) followed
// by half-cleaners (lane ^ size/4, ..., lane ^ 1).
__device__ __forceinline__ uint32_t sort64_desc(uint32_t v, const Xchg &x) {
  v = cx_stage<1, 1>(v, x);
  v = cx_stage<3, 2>(v, x);
  v = cx_stage<1, 1>(v, x);
  v = cx_stage<7, 4>(v, x);
  v = cx_stage<2, 2>(v, x);
  v = cx_stage<1, 1>(v, x);
  v = cx_stage<15, 8>(v, x);
  v = cx_stage<4, 4>(v, x);
  v = cx_stage<2, 2>(v, x);
  v = cx_stage<1, 1>(v, x);
  v = cx_stage<31, 16>(v, x);
  v = cx_stage<8, 8>(v, x);
  v = cx_stage<4, 4>(v, x);
  v = cx_stage<2, 2>(v, x);
  v = cx_stage<1, 1>(v, x);
  v = cx_stage<63, 32>(v, x);
  v = cx_stage<16, 16>(v, x);
  v = cx_stage<8, 8>(v, x);
  v = cx_stage<4, 4>(v, x);
  v = cx_stage<2, 2>(v, x);
  v = cx_stage<1, 1>(v, x);
  return v;
}

// Sorts a bitonic sequence over the 64 lanes into descending order.
__device__ __forceinline__ uint32_t bitonic_merge64_desc(uint32_t v, const Xchg &x) {
  v = cx_stage<32, 32>(v, x);
  v = cx_stage<16, 16>(v, x);
  v = cx_stage<8, 8>(v, x);
  v = cx_stage<4, 4>(v, x);
  v = cx_stage<2, 2>(v, x);
  v = cx_stage<1, 1>(v, x);
  return v;
}

// The 64 best of (list, v): sort v, reverse it against the descending list,
// keep the lane-wise maximum (a bitonic sequence holding the 64 best of the
// union) and sort that.
__device__ __forceinline__ uint32_t merge_batch(uint32_t list, uint32_t v, const Xchg &x) {
  v = partner<63>(sort64_desc(v, x), x);
  return bitonic_merge64_desc(max(list, v), x);
}

// 64-bit versions for the cross-span merge (composite key << 32 | ~column).
template <int MASK>
__device__ __forceinline__ uint64_t partner64(uint64_t v, const Xchg &x) {
  const uint32_t lo = partner<MASK>((uint32_t)v, x), hi = partner<MASK>((uint32_t)(v >> 32), x);
  return ((uint64_t)hi << 32) | lo;
}

template <int MASK, int LOW>
__device__ __forceinline__ uint64_t cx_stage64(uint64_t v, const Xchg &x) {
  const uint64_t y = partner64<MASK>(v, x);
  return (lane_id() & LOW) ? (v < y ? v : y) : (v > y ? v : y);
}

// The 64 best of two descending lists held one entry per lane.
__device__ __forceinline__ uint64_t merge_sorted64(uint64_t a, uint64_t b, const Xchg &x) {
  b = partner64<63>(b, x);
  uint64_t v = a > b ? a : b;
  v = cx_stage64<32, 32>(v, x);
  v = cx_stage64<16, 16>(v, x);
  v = cx_stage64<8, 8>(v, x);
  v = cx_stage64<4, 4>(v, x);
  v = cx_stage64<2, 2>(v, x);
  v = cx_stage64<1, 1>(v, x);
  return v;
}

// Inserts one composite c into the descending list: lanes before its place
// keep their entry, lanes from its place on take the previous lane's entry,
// and its own lane takes c.  list[lane - 1] arrives by DPP wave_shr:1; lane 0
// reads all-ones so that it keeps max(list[0], c).
__device__ __forceinline__ uint32_t insert_one(uint32_t list, uint32_t c) {
  const uint32_t prev = (uint32_t)__builtin_amdgcn_update_dpp((int)0xFFFFFFFFu, (int)list, 0x138, 0xF, 0xF, false);
  return max(list, min(prev, c));
}

// The minimum of v over the wave (wave-uniform result).
__device__ __forceinline__ uint32_t wave_min(uint32_t v, const Xchg &x) {
  v = min(v, partner<1>(v, x));
  v = min(v, partner<2>(v, x));
  v = min(v, partner<4>(v, x));
  v = min(v, partner<8>(v, x));
  v = min(v, partner<16>(v, x));
  v = min(v, partner<32>(v, x));
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
