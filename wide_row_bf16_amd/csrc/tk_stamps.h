// Stage timestamps for measurement builds (compiled with -DTK_STAGE_STAMPS
// into libtk_topk_stamps.so, never into libtk_topk.so, where every macro
// below is empty).  A stamped kernel records, per workgroup (the first
// kStampBlocks of a launch), the 100 MHz real-time counter at the stages of
// its path and its hardware ids; tk_stage_stamps() copies the table out after
// the launch.  Each translation unit that includes this header has its own
// table (device symbols do not cross units without relocatable device
// code): tk_kernels.hip's read-out is tk_stage_stamps, tk_wide.hip's
// tk_stage_stamps_wide.  Slots of a workgroup (uint64 each):
//   0 start                 1 floors computed          2..5 wave w's body done
//   6 lists published       7 merge done, written      8 stores completed (split rows)
//   9 arrival counted       10 last arrival: lists loaded and folded per wave
//   11 waves' results merged 12 outputs written         13 bit 0: the row's last arrival
//   14 XCC_ID << 32 | HW_ID
// The read probe uses slots 0, 2..5 and 14.
#pragma once

#ifdef TK_STAGE_STAMPS
constexpr int kStampBlocks = 8192;
constexpr int kStampSlots = 16;
static __device__ uint64_t tk_stamp_table[kStampBlocks * kStampSlots];

__device__ __forceinline__ void tk_stamp_put(int slot, uint64_t v) {
  if (blockIdx.x < (uint32_t)kStampBlocks) tk_stamp_table[blockIdx.x * kStampSlots + slot] = v;
}
// thread 0 of the workgroup, lane 0 of each wave, hardware ids (hwreg 20
// XCC_ID, hwreg 4 HW_ID, read whole)
#define TK_STAMP(i) \
  do { if (threadIdx.x == 0) tk_stamp_put((i), __builtin_amdgcn_s_memrealtime()); } while (0)
#define TK_WAVE_STAMP(i) \
  do { if ((threadIdx.x & 63u) == 0) tk_stamp_put((i), __builtin_amdgcn_s_memrealtime()); } while (0)
#define TK_STAMP_VALUE(i, v) \
  do { if (threadIdx.x == 0) tk_stamp_put((i), (uint64_t)(v)); } while (0)
#define TK_STAMP_HW(i)                                                                       \
  do {                                                                                       \
    if (threadIdx.x == 0)                                                                    \
      tk_stamp_put((i), ((uint64_t)(uint32_t)__builtin_amdgcn_s_getreg(63508) << 32) |       \
                            (uint32_t)__builtin_amdgcn_s_getreg(63492));                     \
  } while (0)
#else
#define TK_STAMP(i) \
  do {              \
  } while (0)
#define TK_WAVE_STAMP(i) \
  do {                   \
  } while (0)
#define TK_STAMP_VALUE(i, v) \
  do {                       \
  } while (0)
#define TK_STAMP_HW(i) \
  do {                 \
  } while (0)
#endif
