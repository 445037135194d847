// Seeded top-p sampling over each row's top-k entries (gfx950).
//
// What is computed: the pages only name the parameters of a sampled drafted
// decode (temperature, top-k, top-p, seed: the receipt of TensorFold PR
// #3069, "qwen27 metal: restore the long-copy driver for a lone greedy stream
// on M5") and require seeded sampled decodes to be reproducible token for
// token (the seeded sampled exactness cases in the review of TensorFold PR
// #713).  The library's reading, stated in tk_topk.h at
// tk_sample_topk_bf16: float32 softmax weights relative to the top entry by a
// fixed exp2 routine, float32 cumulative sums in entry order, the smallest
// nucleus reaching top_p of the total, and a 24-bit uniform from
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011) keyed by the seed
// with counter (row, 0, offset).  Every float operation is a single IEEE
// float32 operation in a fixed order (no contraction into fused
// multiply-adds), so a decision taken on these numbers is reproducible.
//
// One wave per row (k <= 64: lane j holds entry j), four rows per workgroup.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tk_launch.h"
#include "tk_topk.h"

#pragma clang fp contract(off)

namespace tk {
namespace {

constexpr int kWaveS = 64;
constexpr int kRowsPerGroup = 4;

__device__ __forceinline__ uint32_t mulhi32(uint32_t a, uint32_t b) {
  return (uint32_t)(((uint64_t)a * b) >> 32);
}

// Philox4x32 with 10 rounds; only the first output word is needed.
__device__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;  // round multipliers
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;  // key increments
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    const uint32_t hi0 = mulhi32(kM0, c0), lo0 = kM0 * c0;
    const uint32_t hi1 = mulhi32(kM1, c2), lo1 = kM1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += kW0;
    k1 += kW1;
  }
  return c0;
}

// 2^t for t <= 0: t = n + f with n = rint(t), |f| <= 1/2; 2^f by a degree-7
// polynomial (Horner, coefficients passed in), times 2^n built as a float.
__device__ __forceinline__ float exp2_fixed(float t, const float (&c)[8]) {
  const float n = __builtin_rintf(t);
  if (!(n >= -125.0f)) return 0.0f;  // also t == -inf
  const float f = t - n;
  float p = c[7];
#pragma unroll
  for (int i = 6; i >= 0; --i) p = p * f + c[i];
  const float scale = __uint_as_float((uint32_t)((int)n + 127) << 23);
  return p * scale;
}

__global__ __launch_bounds__(kWaveS * kRowsPerGroup) void sample_kernel(SampleArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWaveS));
  const int l = (int)__lane_id();
  const int64_t r = (int64_t)blockIdx.x * kRowsPerGroup + wave;
  if (r >= a.rows) return;
  const int64_t base = r * a.k;
  const int c0 = __builtin_amdgcn_readfirstlane(a.count[r]);
  const int n = c0 < a.k ? c0 : a.k;  // a count above k is never read past the row
  int token = -1, kept = 0;
  if (n > 0 && a.greedy) {
    token = a.idx[base];
    kept = 1;
  } else if (n > 0) {
    const bool live = l < n;
    const float x = live ? __uint_as_float((uint32_t)a.val[base + l] << 16) : 0.0f;
    const float x0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    float w;
    if (x0 == __builtin_inff()) {
      w = x == __builtin_inff() ? 1.0f : 0.0f;
    } else {
      w = x == -__builtin_inff() ? 0.0f : exp2_fixed((x - x0) * a.scale, a.coef);
    }
    if (!live) w = 0.0f;
    // cumulative sums in entry order, one float32 addition at a time; lane j
    // ends up holding c_{j+1}
    float c = 0.0f, cum = 0.0f;
    for (int j = 0; j < n; ++j) {
      c = c + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
      cum = l == j ? c : cum;
    }
    const float bound = a.top_p * c;  // c == Z here
    const uint64_t reach = __ballot(live && cum >= bound);
    kept = reach ? __builtin_ctzll(reach) + 1 : n;  // c_n == Z >= bound always holds
    const uint32_t rnd = philox_word0((uint32_t)r, 0u, a.off0, a.off1, a.key0, a.key1);
    const float u = (float)(rnd >> 8) * 0x1p-24f;
    const float ck = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), kept - 1));
    const float h = u * ck;
    const uint64_t above = __ballot(l < kept && cum > h);
    const int j = above ? __builtin_ctzll(above) : kept - 1;
    token = a.idx[base + j];
  }
  if (l == 0) {
    a.out_token[r] = token;
    a.out_kept[r] = kept;
  }
}

}  // namespace

hipError_t launch_sample(const SampleArgs &a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const int64_t blocks = (a.rows + kRowsPerGroup - 1) / kRowsPerGroup;
  hipLaunchKernelGGL(sample_kernel, dim3((uint32_t)blocks), dim3(kWaveS * kRowsPerGroup), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tk
