// A stand-in device layer for host-only builds of the C ABI (tk_api.cpp):
// the HIP calls the ABI makes and the kernels' launch functions, on the host.
// One fake device of 256 CUs; "device" allocations are host memory tracked
// in a table; launches record nothing but check that every scratch range
// they are given lies inside a live allocation (or the fixed array); any
// call that can fail can be made to fail.  Test infrastructure: built with
// g++ (optionally under AddressSanitizer and UndefinedBehaviorSanitizer) by
// tests/test_host_sanitized.py, never part of the library.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <map>
#include <string>

#include "hip_stub.h"
#include "tk_config.h"
#include "tk_launch.h"

namespace {

std::map<uintptr_t, size_t> g_live;  // base -> bytes
StubCounters g_count;
int g_fail_at = 0;     // fail the n-th fallible call (1-based); 0: none
int g_fallible = 0;    // fallible calls since the last reset
int g_errors = 0;      // extent violations seen by the launch checks
alignas(256) unsigned char g_fixed[tk::kFixedScratchBytes];

std::string g_trace;

// d device, a attribute, p pool, s pool attribute, m malloc, f free, l launch,
// z zero fill, x fixed scratch
bool fail_now(char kind) {
  g_trace.push_back(kind);
  return ++g_fallible == g_fail_at;
}

// Every byte of [p, p + bytes) inside one live allocation or the fixed array.
void check_extent(const void *p, size_t bytes, const char *what) {
  if (!p || bytes == 0) return;
  const uintptr_t a = (uintptr_t)p;
  if (a >= (uintptr_t)g_fixed && a + bytes <= (uintptr_t)g_fixed + sizeof(g_fixed)) return;
  auto it = g_live.upper_bound(a);
  if (it != g_live.begin()) {
    --it;
    if (a >= it->first && a + bytes <= it->first + it->second) return;
  }
  fprintf(stderr, "stub: %s [%p, +%zu) is outside every allocation\n", what, p, bytes);
  ++g_errors;
}

hipError_t launch_result(const char *what) {
  ++g_count.launches;
  (void)what;
  return fail_now(what[0] == 'z' ? 'z' : 'l') ? hipErrorLaunchFailure : hipSuccess;
}

}  // namespace

extern "C" {

void stub_reset(int fail_at) {
  g_fail_at = fail_at;
  g_fallible = 0;
  g_count = StubCounters{};
  g_trace.clear();
}
const char *stub_trace(void) { return g_trace.c_str(); }
int stub_fallible_calls(void) { return g_fallible; }
int stub_errors(void) { return g_errors; }
size_t stub_live_allocations(void) { return g_live.size(); }
StubCounters stub_counters(void) { return g_count; }
void *stub_fixed_base(void) { return g_fixed; }

hipError_t hipGetDevice(int *device) {
  if (fail_now('d')) return hipErrorNoDevice;
  *device = 0;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t attr, int device) {
  (void)attr;
  (void)device;
  if (fail_now('a')) return hipErrorInvalidDevice;
  *value = 256;
  return hipSuccess;
}

hipError_t hipDeviceGetDefaultMemPool(hipMemPool_t *pool, int device) {
  (void)device;
  if (fail_now('p')) return hipErrorInvalidDevice;
  *pool = (hipMemPool_t)&g_count;
  return hipSuccess;
}

hipError_t hipMemPoolSetAttribute(hipMemPool_t pool, hipMemPoolAttr attr, void *value) {
  (void)pool;
  (void)attr;
  (void)value;
  return fail_now('s') ? hipErrorInvalidValue : hipSuccess;
}

hipError_t hipMallocAsync(void **ptr, size_t bytes, hipStream_t stream) {
  (void)stream;
  ++g_count.mallocs;
  if (fail_now('m')) return hipErrorOutOfMemory;
  void *p = aligned_alloc(256, (bytes + 255) & ~size_t(255));
  if (!p) return hipErrorOutOfMemory;
  g_live[(uintptr_t)p] = bytes;
  *ptr = p;
  return hipSuccess;
}

hipError_t hipFreeAsync(void *ptr, hipStream_t stream) {
  (void)stream;
  ++g_count.frees;
  if (fail_now('f')) return hipErrorInvalidValue;  // the allocation stays: the runtime could not free it
  auto it = g_live.find((uintptr_t)ptr);
  if (it == g_live.end()) {
    fprintf(stderr, "stub: free of %p, which is not a live allocation\n", ptr);
    ++g_errors;
    return hipErrorInvalidValue;
  }
  g_live.erase(it);
  free(ptr);
  return hipSuccess;
}

}  // extern "C"

// The kernels' launch functions: extent checks of every scratch range.
namespace tk {

hipError_t launch_span_scan(const ScanArgs &a, int64_t rows, hipStream_t) {
  if (a.spans > 1) {
    const size_t n = (size_t)rows * (size_t)a.spans;
    check_extent(a.span_list, n * (size_t)a.k * 8, "span_scan span_list");
    check_extent(a.span_count, n * 4, "span_scan span_count");
    check_extent(a.span_flags, n * 4, "span_scan span_flags");
    if (a.row_done) check_extent(a.row_done, (size_t)rows * 4, "span_scan row_done");
    if (a.row_done && rows > kFusedMaxRows) {
      fprintf(stderr, "stub: fused launch of %lld rows\n", (long long)rows);
      ++g_errors;
    }
  }
  return launch_result("span_scan");
}

hipError_t launch_wide_scan(const ScanArgs &a, int64_t rows, hipStream_t s) { return launch_span_scan(a, rows, s); }

hipError_t launch_argmax(const ArgmaxArgs &a, int64_t rows, hipStream_t) {
  if (a.spans > 1) {
    check_extent(a.span_slot, (size_t)rows * (size_t)a.spans * 8, "argmax span_slot");
    check_extent(a.row_done, (size_t)rows * 4, "argmax row_done");
  }
  return launch_result("argmax");
}

hipError_t launch_argmax32(const ArgmaxArgs32 &a, int64_t rows, hipStream_t) {
  if (a.spans > 1) {
    check_extent(a.span_slot, (size_t)rows * (size_t)a.spans * 8, "argmax32 span_slot");
    check_extent(a.span_flag, (size_t)rows * (size_t)a.spans * 4, "argmax32 span_flag");
    check_extent(a.row_done, (size_t)rows * 4, "argmax32 row_done");
  }
  return launch_result("argmax32");
}

hipError_t launch_span_scan32(const ScanArgs32 &a, int64_t rows, hipStream_t) {
  if (a.spans > 1) {
    const size_t n = (size_t)rows * (size_t)a.spans;
    check_extent(a.span_list, n * (size_t)a.k * 8, "scan32 span_list");
    check_extent(a.span_count, n * 4, "scan32 span_count");
    check_extent(a.span_flags, n * 4, "scan32 span_flags");
    check_extent(a.row_done, (size_t)rows * 4, "scan32 row_done");
  }
  return launch_result("scan32");
}

hipError_t launch_wide_scan32(const ScanArgs32 &a, int64_t rows, hipStream_t s) {
  return launch_span_scan32(a, rows, s);
}

hipError_t launch_span_merge(const MergeArgs &a, int64_t rows, hipStream_t) {
  const size_t in = (size_t)rows * (size_t)a.lists_in;
  check_extent(a.list_in, in * (size_t)a.k * 8, "merge list_in");
  check_extent(a.count_in, in * 4, "merge count_in");
  check_extent(a.flags_in, in * 4, "merge flags_in");
  if (a.lists_out > 1) {
    const size_t out = (size_t)rows * (size_t)a.lists_out;
    check_extent(a.list_out, out * (size_t)a.k * 8, "merge list_out");
    check_extent(a.count_out, out * 4, "merge count_out");
    check_extent(a.flags_out, out * 4, "merge flags_out");
  }
  return launch_result("merge");
}

hipError_t launch_head_scan(const HeadArgs &a, hipStream_t) {
  const size_t n = (size_t)a.rows * (size_t)a.spans;
  check_extent(a.span_list, n * (size_t)a.k * 8, "head span_list");
  check_extent(a.span_count, n * 4, "head span_count");
  check_extent(a.span_flags, n * 4, "head span_flags");
  return launch_result("head");
}

hipError_t launch_shard_merge(const ShardMergeArgs &, hipStream_t) { return launch_result("shard_merge"); }
hipError_t launch_sample(const SampleArgs &, hipStream_t) { return launch_result("sample"); }
hipError_t launch_read_probe(const void *, int64_t, int32_t, uint32_t *, hipStream_t) {
  return launch_result("read_probe");
}

hipError_t launch_zero_fill(int32_t *p, int64_t n, hipStream_t) {
  check_extent(p, (size_t)n * 4, "zero_fill");
  ++g_count.fills;
  --g_count.launches;  // counted as a fill, not a kernel of the top-k
  return launch_result("zero_fill");
}

hipError_t fixed_scratch(int dev, hipStream_t, void **ptr) {
  (void)dev;
  ++g_count.fixed;
  if (fail_now('x')) return hipErrorInvalidSymbol;
  *ptr = g_fixed;
  return hipSuccess;
}

}  // namespace tk
