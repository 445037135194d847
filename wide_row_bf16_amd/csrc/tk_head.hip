// Draft-head logits fused with the row top-k (gfx950): logits = h . w^T for
// up to 64 rows of hidden states h [rows][hidden] against a vocabulary-major
// weight w [vocab][hidden] (bf16, fp32 accumulation, rounded to bf16), and the
// k best logits of every row in the library's order -- without the logits
// ever being written to memory.
//
// What is computed: the drafter of TensorFold PR #713 runs its draft head and
// then the top-k over its rows (15 rows of 98592 columns in change 3); the
// pages give no kernel for the head.  This is the plain reading: each logit
// is the bf16 rounding (to nearest, ties to even) of the fp32 sum of the
// products h[r][i] * w[n][i]; the top-k then follows the rules of
// tk_topk_bf16 on those logits (score descending, lower column first, NaN
// excluded and flagged, infinities ranked and flagged).
//
// Kernel.  One workgroup per span of up to kHeadSpanCols vocabulary columns
// (the host cuts the vocabulary's 16-column tiles into `spans` near-equal
// ranges), four waves, each owning a contiguous quarter of the span's tiles
// (four of a full span, three or four of a span of 12 or 13; a missing
// fourth tile loads nothing and is never written).  The contraction runs on the
// matrix cores: v_mfma_f32_16x16x32_bf16 with A = a 16-row tile of h and B =
// 32 hidden values of 16 vocabulary rows of w (each lane loads 16 contiguous
// bytes of one w row: lane l takes row l % 16, values 8 (l / 16) .. + 7), one
// accumulator per (column tile, row tile); the loads of the next hidden steps
// are in flight while the current ones multiply, and with one row tile each
// span starts its walk over the hidden dimension at its own hashed block.  w
// is read once; h is small and shared by every workgroup.  Buffer
// descriptors clamp both: rows past vocab or past rows read zero.  The
// accumulators are rounded to bf16 into LDS; then each wave takes rows w,
// w + 4, ... and keeps the span's top k of the row in one VGPR (lane i = i-th
// best), as the scan kernels do, and writes it as 64-bit composites
// key << 32 | (0x7FFFFFFF - column) << 1 | sign (the sign tells -0 from +0,
// which share a key) for span_merge_kernel to fold.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tk_config.h"
#include "tk_launch.h"

namespace tk {
namespace {

#include "tk_wave.h"
#include "tk_scan16.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadWaves = kHeadSpanCols / 64;                  // waves per workgroup (four tiles each)
constexpr int kHeadThreads = kHeadWaves * kWave;
constexpr int kHeadTilesPerWave = kHeadSpanCols / 16 / kHeadWaves;
static_assert(kHeadTilesPerWave == 4, "each wave owns four 16-column tiles");
constexpr int kHeadLaneCols = 4;                               // a row's span: four columns per lane
static_assert(kHeadSpanCols <= kHeadLaneCols * kWave, "a row's span fits four columns per lane");
static_assert(kHeadLaneCols == 4, "the per-lane sort and shift of the top-k are written for four");

template <int POLICY>
__device__ __forceinline__ bf16x8 load_frag(__amdgpu_buffer_rsrc_t rsrc, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, POLICY);
  return __builtin_bit_cast(bf16x8, v);
}

// fp32 -> bf16 bits, rounding to nearest with ties to even; NaN stays NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// An offset past every descriptor's range (ranges stay below 2^30 bytes and
// the per-lane offsets below 2^30 too, so the sum cannot wrap): such a load
// returns zeros.  Used instead of branches around loads, which would make the
// compiler wait for every outstanding load at the join.
constexpr uint32_t kHeadPastEnd = 0x7FFFFFF0u;

// w is staged through LDS in blocks of kHeadBlockBytes per row of the wave's
// 64 rows: each load instruction reads whole cache lines of a few rows (16
// bytes per lane), the block is written to the wave's own LDS region with a
// row pitch 16 bytes longer than the block, and the matrix-core
// fragments (16 bytes of one row per lane) are read back from there.  Loaded
// straight in the fragment layout, every line would be split over two
// 64-byte requests of two instructions; measured 3.1 TB/s that way.
constexpr int kHeadBlockBytes = 128;                            // per row and block
constexpr int kHeadRowPitch = kHeadBlockBytes + 16;             // +16: conflict-free fragment reads
constexpr int kHeadWaveRows = kHeadTilesPerWave * 16;           // 64 rows of w per wave
constexpr int kHeadLanesPerRow = kHeadBlockBytes / 16;          // lanes of one load on one row
constexpr int kHeadRowsPerLoad = kWave / kHeadLanesPerRow;      // rows of one load instruction
constexpr int kHeadBlockLoads = kHeadWaveRows / kHeadRowsPerLoad;
constexpr int kHeadBlockSteps = kHeadBlockBytes / 64;           // hidden steps of 32 per block
static_assert(kHeadBlockBytes % 128 == 0 && kHeadWaveRows % kHeadRowsPerLoad == 0, "whole lines per row");

struct HeadBlock {
  u32x4 v[kHeadBlockLoads];
};

template <int RT>
struct HeadA {
  bf16x8 a[kHeadBlockSteps][RT];
};

// With four row tiles the kernel asks for two workgroups per CU: left alone the
// compiler keeps the accumulators in AGPRs beside 182 VGPRs (310 registers, one
// wave per SIMD), so only 256 of the 386 workgroups of a 98592-column head fit
// and the grid ran in two rounds; under the bound it uses 243 VGPRs without
// spills and 64 rows went from 185 to 160 us.  The same bound made two row
// tiles slower (122 -> 146 us), so those kernels keep the default.
template <int RT>
__global__ __launch_bounds__(kHeadThreads, RT == 4 ? 2 : 1) void head_scan_kernel(HeadArgs a) {
  __shared__ uint16_t s_logit[RT * 16][kHeadSpanCols];
  __shared__ __attribute__((aligned(16))) uint8_t s_w[kHeadWaves][kHeadWaveRows * kHeadRowPitch];

  const int s = blockIdx.x;
  const int64_t ntiles = (a.vocab + 15) / 16;
  const int64_t t0 = ntiles * s / a.spans, t1 = ntiles * (s + 1) / a.spans;  // at most 16 tiles (host)
  const int64_t n0 = t0 * 16;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int l = lane_id();
  const int64_t nvalid = a.vocab - n0 < (t1 - t0) * 16 ? a.vocab - n0 : (t1 - t0) * 16;

  // This wave's tiles: a contiguous quarter of the span's (at most four).
  const int nt = (int)(t1 - t0);
  const int tw0 = wave * nt / kHeadWaves;
  const int ntw = (wave + 1) * nt / kHeadWaves - tw0;
  // w's range is the wave's own rows, so the loads of a missing fourth tile
  // fall outside it and read zeros (an empty range reads nothing).  Both
  // ranges end at the last row's `hidden`-th element, never in its row
  // padding: the loads below read whole blocks past `hidden`, which the
  // range check turns into zeros on the last row (and which are zeroed in
  // registers on the others).  Ranges and offsets are multiples of 16 bytes
  // (hidden % 32 == 0, strides % 8 == 0), so no load straddles the end.
  const int64_t wr0 = n0 + 16 * tw0;
  const int64_t wrows = a.vocab - wr0 < 16 * ntw ? a.vocab - wr0 : 16 * ntw;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.w + wr0 * a.w_stride), (short)0,
      wrows > 0 ? (int)(((wrows - 1) * a.w_stride + a.hidden) * 2) : 0, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.h, (short)0, (int)(((a.rows - 1) * a.h_stride + a.hidden) * 2), kBufferWord3);

  f32x4 acc[kHeadTilesPerWave][RT];
#pragma unroll
  for (int j = 0; j < kHeadTilesPerWave; ++j)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[j][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t hidden_bytes = a.hidden * 2;
  const int nblk = (int)((hidden_bytes + kHeadBlockBytes - 1) / kHeadBlockBytes);
  // Logical block b reads hidden block (b + rot) mod nblk, rot hashed from the
  // span.  Without it every wave of the grid reads the same block offset of
  // rows w_stride apart at the same time: requests that share their low
  // address bits and so crowd onto the same memory channels.  With one row
  // tile the rotation measured 117 -> 103 us on 15 x 2048 x 98592, with four
  // (nontemporal loads) 154 -> 146 us on 64 rows; with two it measured
  // slower (118 -> 122 us on 32 rows) and is not used.  Only the order of
  // the fp32 sums changes.
  const int rot = RT != 2 ? (int)((((uint32_t)s * 2654435761u) >> 16) % (uint32_t)nblk) : 0;
  auto phys = [&](int blk) {  // blocks past the last (loaded, never used) keep their index
    if (blk >= nblk) return blk;
    const int p = blk + rot;
    return p >= nblk ? p - nblk : p;
  };
  // block loads: instruction q reads kHeadRowsPerLoad wave rows, lane l row
  // q * kHeadRowsPerLoad + l / kHeadLanesPerRow, bytes 16 (l % kHeadLanesPerRow)
  const int lrow = l / kHeadLanesPerRow, lbyte = 16 * (l % kHeadLanesPerRow);
  const uint32_t g_lane = (uint32_t)(((int64_t)lrow * a.w_stride) * 2 + lbyte);
  const uint32_t g_q = (uint32_t)(kHeadRowsPerLoad * a.w_stride * 2);
  uint8_t *lds_w = s_w[wave];
  const uint32_t st_lane = (uint32_t)(lrow * kHeadRowPitch + lbyte);
  const uint32_t ld_lane = (uint32_t)((l % 16) * kHeadRowPitch + 16 * (l / 16));
  const uint32_t a_off = (uint32_t)(((int64_t)(l % 16) * a.h_stride + 8 * (l / 16)) * 2);
  const uint32_t a_tile = (uint32_t)(16 * a.h_stride * 2);

  // Loads are unconditional (a branch around them makes the compiler wait for
  // every outstanding load at the join); the bytes of a block past `hidden`
  // -- the next row's, or zeros past the buffer's range -- are zeroed in
  // registers, and blocks past the last are loaded but never used.  w is read
  // once, so its loads take the scans' nontemporal policy: a plain read of
  // these blocks (whole lines per request) streams at ~6.5 TB/s with it and
  // ~5.7 without, and the head on 15 x 2048 x 98592 went from 94.7 to 84.0 us
  // per call (32 rows 121.5 -> 113.7, 64 rows 155.5 -> 151.5).
  auto load_block = [&](HeadBlock &B, int logical) {
    const int blk = phys(logical);
    const bool in = (int64_t)blk * kHeadBlockBytes + lbyte < hidden_bytes;
#pragma unroll
    for (int q = 0; q < kHeadBlockLoads; ++q) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
          rw, (int)(g_lane + q * g_q + (uint32_t)blk * kHeadBlockBytes), 0, kLoadPolicy);
      B.v[q] = in ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto load_a = [&](HeadA<RT> &A, int logical) {
    const int blk = phys(logical);
#pragma unroll
    for (int t = 0; t < kHeadBlockSteps; ++t) {
      const int step = kHeadBlockSteps * blk + t;
      const bool in = (int64_t)step * 64 < hidden_bytes;
#pragma unroll
      for (int r = 0; r < RT; ++r)
        A.a[t][r] = load_frag<0>(rh, in ? a_off + r * a_tile + (uint32_t)step * 64u : kHeadPastEnd);
    }
  };
  auto store_block = [&](const HeadBlock &B) {
#pragma unroll
    for (int q = 0; q < kHeadBlockLoads; ++q)
      *reinterpret_cast<u32x4 *>(lds_w + st_lane + q * kHeadRowsPerLoad * kHeadRowPitch) = B.v[q];
  };
  auto mma_block = [&](const HeadA<RT> &A) {
#pragma unroll
    for (int t = 0; t < kHeadBlockSteps; ++t)
#pragma unroll
      for (int j = 0; j < kHeadTilesPerWave; ++j) {
        const bf16x8 b = *reinterpret_cast<const bf16x8 *>(lds_w + ld_lane + j * 16 * kHeadRowPitch + 64 * t);
#pragma unroll
        for (int r = 0; r < RT; ++r)
          acc[j][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A.a[t][r], b, acc[j][r], 0, 0, 0);
      }
  };

  // Block blk is in LDS while block blk + 1 is in registers (in flight) and
  // the h fragments of the next block load.  LDS serves a wave's operations
  // in order, so storing the next block after this block's fragment reads
  // needs no barrier (the region is the wave's own).
  HeadBlock Bn;
  HeadA<RT> A0, A1;
  load_block(Bn, 0);
  load_a(A0, 0);
  store_block(Bn);
  load_block(Bn, 1);
  load_a(A1, 1);
  for (int blk = 0; blk < nblk; blk += 2) {
    mma_block(A0);
    if (blk + 1 >= nblk) break;
    store_block(Bn);
    load_block(Bn, blk + 2);
    load_a(A0, blk + 2);
    mma_block(A1);
    if (blk + 2 >= nblk) break;
    store_block(Bn);
    load_block(Bn, blk + 3);
    load_a(A1, blk + 3);
  }

  // With one row tile, the rows' sketch slots (see HeadArgs) load now, while
  // the logits are formed: wave w takes rows w, w + 4, ..., lane i slot i.
  // Agent-scope loads: other XCDs' workgroups write the slots.
  constexpr int kSketchRows = RT == 1 ? 16 / kHeadWaves : 1;
  uint32_t slot[kSketchRows];
#pragma unroll
  for (int i = 0; i < kSketchRows; ++i) {
    const int row = wave + i * kHeadWaves;
    slot[i] = 0;
    if (RT == 1 && a.sketch && row < a.rows && l < a.k)
      slot[i] = __hip_atomic_load(&a.sketch[row * a.k + l], __ATOMIC_RELAXED, kAgent);
  }

  // accumulators -> bf16 logits in LDS (and, on request, to memory)
#pragma unroll
  for (int j = 0; j < kHeadTilesPerWave; ++j) {
    if (j >= ntw) break;  // another wave's tile
    const int col = (tw0 + j) * 16 + l % 16;
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = t * 16 + 4 * (l / 16) + i;
        const uint32_t b = bf16_rne(acc[j][t][i]);
        s_logit[row][col] = (uint16_t)b;
        if (a.logits && row < a.rows && col < nvalid) a.logits[row * a.logits_stride + n0 + col] = (uint16_t)b;
      }
  }
  __syncthreads();

  // per row: the span's top k, four columns per lane (every lane busy): each
  // lane sorts its four, then position by position the lanes' p-th best are
  // merged in while any beats the k-th kept entry
  const Xchg x = make_xchg();
  const int k = a.k;
#pragma unroll 1
  for (int row = wave; row < a.rows; row += kHeadWaves) {
    // The row's floor from its sketch: once all k slots hold a key, k listed
    // entries (one per slot, from k different spans) reach their minimum, so
    // a key below it cannot be among the row's k best; equal keys are kept
    // (the lower column may win).  An empty slot leaves the floor at 0.
    uint32_t thr = 0;
    if (RT == 1) {
      const uint32_t sv = slot[0];
#pragma unroll
      for (int i = 0; i + 1 < kSketchRows; ++i) slot[i] = slot[i + 1];  // the next row's slots first
      if (a.sketch && !ballot(l < k && sv == 0)) thr = wave_min(l < k ? sv : 0xFFFFFFFFu, x);
    }
    uint32_t c[kHeadLaneCols];
    bool nan = false, ninf = false;
#pragma unroll
    for (int e = 0; e < kHeadLaneCols; ++e) {
      const int col = kHeadLaneCols * l + e;
      const bool valid = col < nvalid;
      const uint32_t b = valid ? (uint32_t)s_logit[row][col] : 0u;
      const uint32_t key = order_key(b);
      nan |= valid && key == 0;
      ninf |= valid && b == 0xFF80u;
      c[e] = (valid && key && key >= thr) ? (key << 16) | (0xFFFFu - (uint32_t)col) : 0u;
    }
    uint32_t flags = (ballot(nan) ? kNan : 0u) | (ballot(ninf) ? kNinf : 0u);
    cx(c[0], c[1]); cx(c[2], c[3]); cx(c[0], c[2]); cx(c[1], c[3]); cx(c[1], c[2]);  // descending
    uint32_t list = 0, kth = 0;
#pragma unroll 1
    for (int p = 0; p < kHeadLaneCols; ++p) {
      uint64_t m = lanes_ugt(c[0], kth);
      if (!m) break;
      if (__popcll(m) >= kBatchInsert) {
        list = merge_batch(list, c[0] > kth ? c[0] : 0u, x);
      } else {
        do {
          const int ln = __builtin_ctzll(m);
          m &= m - 1;
          list = insert_one(list, readlane(c[0], ln));
        } while (m);
      }
      kth = readlane(list, k - 1);
      c[0] = c[1]; c[1] = c[2]; c[2] = c[3]; c[3] = 0;
    }
    const int cnt = min(__popcll(ballot(list != 0)), k);
    if ((readlane(list, 0) >> 16) == 0xFF80u) flags |= kPinf;
    const int64_t sb = (int64_t)row * a.spans + s;
    if (l < cnt) {
      const uint32_t key = list >> 16;
      const uint32_t col = 0xFFFFu - (list & 0xFFFFu);
      const uint32_t sign = key == 0x8000u ? (uint32_t)(s_logit[row][col] >> 15) : 0u;
      a.span_list[sb * k + l] =
          ((uint64_t)key << 32) | ((uint64_t)(0x7FFFFFFFu - (uint32_t)(n0 + col)) << 1) | sign;
    }
    if (l == 0) {
      a.span_count[sb] = cnt;
      a.span_flags[sb] = flags;
      // this span's best key, the head of its list, into the row's slot
      if (RT == 1 && a.sketch && cnt > 0)
        __hip_atomic_fetch_max(&a.sketch[row * k + s % k], list >> 16, __ATOMIC_RELAXED, kAgent);
    }
  }
}

}  // namespace

hipError_t launch_head_scan(const HeadArgs &a, hipStream_t stream) {
  if (a.rows <= 0 || a.spans <= 0) return hipSuccess;
  const dim3 grid((uint32_t)a.spans), block(kHeadThreads);
  if (a.rows <= 16) {
    hipLaunchKernelGGL(head_scan_kernel<1>, grid, block, 0, stream, a);
  } else if (a.rows <= 32) {
    hipLaunchKernelGGL(head_scan_kernel<2>, grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL(head_scan_kernel<4>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace tk
