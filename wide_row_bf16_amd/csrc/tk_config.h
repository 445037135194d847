// Compile-time constants of the top-k library, shared by its kernels and its
// host code.  The static_asserts at the end check that the kernels' limits
// equal the public header's (TK_MAX_K, TK_MAX_K_LANE, TK_HEAD_MAX_ROWS), that
// a wave can hold one kept entry per lane, and that every column a wave scans
// fits its 16-bit relative index; an edit to one constant that breaks any of
// these relations stops compilation.  (Cited: TensorFold PR #713, change 3,
// which checks its kernel constants against the calling side at build time.)
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "tk_topk.h"

namespace tk {

constexpr int kWave = 64;                      // CDNA wavefront width
constexpr int kWgWaves = 4;                    // waves per scan workgroup
constexpr int kWgThreads = kWave * kWgWaves;   // 256
constexpr int kMaxK = 64;                      // kept entries of the one-register scans: one per lane
constexpr int kMaxKWide = 256;                 // k of the multi-register scan (four registers per wave)
constexpr int kVecElems = 8;                   // bf16 per 16-byte load
constexpr int kChunkVecs = 4;                  // 16-byte loads per lane per chunk
constexpr int64_t kMaxWaveCols = 65536;        // a wave's relative column fits 16 bits
constexpr int64_t kMaxSpanVecs = 32640;        // 16-byte vectors one workgroup scans at most
constexpr int64_t kMaxSpanCols = kMaxSpanVecs * kVecElems;  // 261120
constexpr int kMergeGroup = 64;                // span lists one merge workgroup folds at most
constexpr int kMergeThreads = 1024;              // sixteen waves: four lists each, then a tree over the waves
constexpr int kFusedMaxRows = 4096;             // rows per launch of the fused (single-dispatch) split path
constexpr int kBatchInsert = 8;                // >= this many new candidates: bitonic batch merge
constexpr int kSpecChunks = 16;                // chunks per wave before a speculative floor pays
constexpr int kSampleElems = kWgWaves * kChunkVecs * kWave * kVecElems;  // pooled sample: each wave's first chunk
constexpr double kSpecFailure = 1e-5;          // target probability that a speculative floor fails
constexpr int kLookLanes = 56;                 // rising share: lanes whose first-chunk maximum sits in their last vector
constexpr int kLookChunks = 6;                 // rising share: chunks of the wave's share for its end floor to pay
constexpr int kHeadSpanCols = 256;             // vocabulary columns per workgroup of the fused head
constexpr int kHeadMaxRows = 64;               // rows of the fused head: four 16-row matrix-core tiles
constexpr size_t kFixedScratchBytes = size_t(2) << 20;  // scratch array of the allocation-free entry point
constexpr int kMaxDevices = 64;                // devices the library keeps per-device state for

static_assert(kMaxKWide == (int)TK_MAX_K, "public and internal max k differ");
static_assert(kMaxK == (int)TK_MAX_K_LANE, "public and internal lane max k differ");
static_assert(kMaxKWide == 4 * kWave, "the multi-register scan keeps at most four registers");
static_assert(kMaxK <= kWave, "a wave holds one kept entry per lane");
static_assert(kHeadMaxRows == (int)TK_HEAD_MAX_ROWS, "public and internal head row limits differ");
static_assert(kWgThreads == 256, "scan kernels are written for four wave64s");
// A wave scans at most ceil(kMaxSpanVecs / kWgWaves) vectors plus two partial
// edges of < kVecElems columns each; its columns must stay within 16 bits.
static_assert(((kMaxSpanVecs + kWgWaves - 1) / kWgWaves) * kVecElems + 2 * kVecElems <= kMaxWaveCols,
              "a wave's column range must fit the 16-bit relative index");
static_assert(kSampleElems == kWgWaves * kChunkVecs * kWave * kVecElems, "sample = one chunk per wave");
static_assert(kFixedScratchBytes == (size_t)TK_NOALLOC_SCRATCH_BYTES, "public and internal fixed scratch differ");
static_assert(kFixedScratchBytes >= 2 * (size_t)kFusedMaxRows * 4, "the fixed scratch holds the arrival counters");

}  // namespace tk
