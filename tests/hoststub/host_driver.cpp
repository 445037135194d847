// Host-only checks of the C ABI (tk_api.cpp over the stand-in device layer of
// hip_stub.cpp) and of the CPU oracle, meant to run under AddressSanitizer
// and UndefinedBehaviorSanitizer:
//  - every fallible HIP call of every launching entry point is made to fail
//    in turn: the call returns TK_ERR_DEVICE (or TK_OK where the library
//    treats that call as optional), leaves no allocation of its own behind,
//    and later calls still work;
//  - every scratch range handed to a kernel lies inside its allocation;
//  - a failed zero fill of a fresh cached buffer is not reused unzeroed;
//  - tk_topk_bf16_noalloc never allocates or frees, and batches rows within
//    its fixed array;
//  - the oracle against a brute-force rank on small random rows.
// Test infrastructure: built and run by tests/test_host_sanitized.py.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <functional>
#include <string>
#include <vector>

#include "hip_stub.h"
#include "tk_topk.h"

extern "C" int tko_topk_bf16(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                             int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                             int32_t threads);

namespace {

int g_fail = 0;

#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                       \
      fprintf(stderr, "\n");                              \
      ++g_fail;                                           \
    }                                                     \
  } while (0)

// Fake device addresses: the guards only do arithmetic on them and the
// stand-in launches never touch them.
const uintptr_t IN = 0x100000000ull, IDX = 0x900000000ull, VAL = 0xA00000000ull, CNT = 0xB00000000ull,
                MSK = 0xC00000000ull, H = 0xD00000000ull, W = 0x1000000000ull;

template <class T>
T *fake(uintptr_t a) {
  return reinterpret_cast<T *>(a);
}

using Call = std::function<tk_status(void *stream)>;

// Runs `call` cleanly, then once more for every fallible HIP call it makes,
// failing that one -- from a fresh stream (scratch allocated and zeroed in
// the call) and from a warm one (scratch cached by a previous call).  After
// each attempt the stream's cached scratch is released and no allocation may
// remain (apart from one whose own free was the failing call), and a clean
// call still works.
void sweep_from(const char *name, Call call, void *stream, bool warm, bool noalloc, int *calls, std::string *trace) {
  stub_reset(0);
  CHECK(tk_release_stream(stream) == TK_OK, "%s: release", name);
  if (warm) {
    stub_reset(0);
    CHECK(call(stream) == TK_OK, "%s: warming call", name);
  }
  stub_reset(0);
  tk_status st = call(stream);
  const int n = stub_fallible_calls();
  const StubCounters base = stub_counters();
  *calls = n;
  *trace = stub_trace();
  CHECK(st == TK_OK, "%s: clean call gave %d", name, (int)st);
  if (noalloc)
    CHECK(base.mallocs == 0 && base.frees == 0, "%s: noalloc allocated (%d) or freed (%d)", name, base.mallocs,
          base.frees);
  for (int i = 1; i <= n + 2; ++i) {
    stub_reset(0);
    CHECK(tk_release_stream(stream) == TK_OK, "%s: release before failure %d", name, i);
    if (warm) {
      stub_reset(0);
      CHECK(call(stream) == TK_OK, "%s: warming call before failure %d", name, i);
    }
    stub_reset(i);
    st = call(stream);
    const std::string t = stub_trace();
    const char kind = i <= (int)t.size() ? t[i - 1] : '-';
    // pool setup (p, s) and the CU count (a) are optional: the library goes on without them
    const bool optional = kind == 'p' || kind == 's' || kind == 'a' || kind == '-';
    if (optional) CHECK(st == TK_OK, "%s: failing optional call %d (%c) gave %d", name, i, kind, (int)st);
    else CHECK(st == TK_ERR_DEVICE, "%s: failing call %d (%c of %s) gave %d", name, i, kind, t.c_str(), (int)st);
    if (noalloc) {
      const StubCounters c = stub_counters();
      CHECK(c.mallocs == 0 && c.frees == 0, "%s: noalloc allocated or freed at failure %d", name, i);
    }
    // the next call on the stream works, and zeroes a cached buffer if the failed one was not
    stub_reset(0);
    CHECK(call(stream) == TK_OK, "%s: clean call after failure %d (%c)", name, i, kind);
    stub_reset(0);
    CHECK(tk_release_stream(stream) == TK_OK, "%s: release after failure %d", name, i);
    const size_t left = stub_live_allocations();
    CHECK(left == 0 || kind == 'f', "%s: failure %d (%c) left %zu allocations", name, i, kind, left);
  }
}

void sweep(const char *name, Call call, bool noalloc = false) {
  static uintptr_t next_stream = 0x5000;
  void *stream = (void *)(next_stream += 0x10);
  int n_fresh = 0, n_warm = 0;
  std::string t_fresh, t_warm;
  sweep_from(name, call, stream, false, noalloc, &n_fresh, &t_fresh);
  sweep_from(name, call, stream, true, noalloc, &n_warm, &t_warm);
  stub_reset(0);
  (void)tk_release_stream(stream);
  printf("swept %-36s fresh %2d calls (%s), warm %2d (%s)\n", name, n_fresh, t_fresh.c_str(), n_warm,
         t_warm.c_str());
}

tk_status topk(void *s, int64_t rows, int64_t cols, int32_t k, int spans = 0, int exact = 0) {
  if (spans || exact) {
    tk_options o{};
    o.spans = spans;
    o.exact = exact;
    return tk_topk_bf16_ex(rows, cols, cols, k, fake<uint16_t>(IN), fake<int32_t>(IDX), fake<uint16_t>(VAL),
                           fake<int32_t>(CNT), fake<uint32_t>(MSK), s, &o);
  }
  return tk_topk_bf16(rows, cols, cols, k, fake<uint16_t>(IN), fake<int32_t>(IDX), fake<uint16_t>(VAL),
                      fake<int32_t>(CNT), fake<uint32_t>(MSK), s);
}

tk_status noalloc(void *s, int64_t rows, int64_t cols, int32_t k) {
  return tk_topk_bf16_noalloc(rows, cols, cols, k, fake<uint16_t>(IN), fake<int32_t>(IDX), fake<uint16_t>(VAL),
                              fake<int32_t>(CNT), fake<uint32_t>(MSK), s);
}

void host_api() {
  sweep("bf16 15x98592 k32 (fused fold)", [](void *s) { return topk(s, 15, 98592, 32); });
  sweep("bf16 1024x151936 k64 (one span)", [](void *s) { return topk(s, 1024, 151936, 64); });
  sweep("bf16 15x98592 k1 (argmax slots)", [](void *s) { return topk(s, 15, 98592, 1); });
  sweep("bf16 15x98592 k256 (wide lists)", [](void *s) { return topk(s, 15, 98592, 256); });
  sweep("bf16 9000x128 k4 s2 (row batches)", [](void *s) { return topk(s, 9000, 128, 4, 2); });
  sweep("bf16 3x98592 k64 s70 (merge levels)", [](void *s) { return topk(s, 3, 98592, 64, 70); });
  sweep("bf16 2x20000000 k8 (span limit)", [](void *s) { return topk(s, 2, 20000000, 8); });
  sweep("f32 15x98592 k32", [](void *s) {
    return tk_topk_f32(15, 98592, 98592, 32, fake<uint32_t>(IN), fake<int32_t>(IDX), fake<uint32_t>(VAL),
                       fake<int32_t>(CNT), fake<uint32_t>(MSK), s);
  });
  sweep("f32 15x98592 k1 (argmax slots)", [](void *s) {
    return tk_topk_f32(15, 98592, 98592, 1, fake<uint32_t>(IN), fake<int32_t>(IDX), fake<uint32_t>(VAL),
                       fake<int32_t>(CNT), fake<uint32_t>(MSK), s);
  });
  sweep("f16 64x151936 k16", [](void *s) {
    return tk_topk_f16(64, 151936, 151936, 16, fake<uint16_t>(IN), fake<int32_t>(IDX), fake<uint16_t>(VAL),
                       fake<int32_t>(CNT), fake<uint32_t>(MSK), s);
  });
  sweep("head 15x2048x98592 k32", [](void *s) {
    return tk_head_topk_bf16(15, 2048, 98592, 32, fake<uint16_t>(H), 2048, fake<uint16_t>(W), 2048,
                             fake<int32_t>(IDX), fake<uint16_t>(VAL), fake<int32_t>(CNT), fake<uint32_t>(MSK),
                             nullptr, 0, s);
  });
  sweep("shard merge 8x1024 k64", [](void *s) {
    return tk_merge_topk_bf16(1024, 8, 64, fake<int32_t>(H), fake<uint16_t>(W), fake<int32_t>(IN),
                              fake<uint32_t>(IN + 0x1000000), fake<int32_t>(IDX), fake<uint16_t>(VAL),
                              fake<int32_t>(CNT), fake<uint32_t>(MSK), s);
  });
  sweep("sample 1024 k64", [](void *s) {
    return tk_sample_topk_bf16(1024, 64, fake<int32_t>(IDX), fake<uint16_t>(VAL), fake<int32_t>(CNT), 0.7f,
                               0.95f, 1234, 0, fake<int32_t>(H), fake<int32_t>(W), s);
  });
  sweep("probe read", [](void *s) { return tk_probe_read(fake<void>(IN), 1 << 20, 64, fake<uint32_t>(H), s); });
  sweep("noalloc 15x98592 k32", [](void *s) { return noalloc(s, 15, 98592, 32); }, true);
  sweep("noalloc 15x98592 k1", [](void *s) { return noalloc(s, 15, 98592, 1); }, true);
  sweep("noalloc 17x16000000 k256 (batched)", [](void *s) { return noalloc(s, 17, 16000000, 256); }, true);
  sweep("noalloc 300x30000 k64 (one span)", [](void *s) { return noalloc(s, 300, 30000, 64); }, true);

  // noalloc: a row that cannot fit is rejected before any device call but the device query
  stub_reset(0);
  CHECK(noalloc((void *)0x77, 1, 1100000000, 64) == TK_ERR_SCRATCH, "noalloc rejection");
  CHECK(stub_counters().launches == 0 && stub_counters().mallocs == 0, "noalloc rejection launched or allocated");

  // a failed zero fill of a fresh cached buffer: the next call must zero a buffer again
  {
    void *s = (void *)0x6100;
    stub_reset(0);
    CHECK(topk(s, 15, 98592, 32) == TK_OK, "fill case warm");
    stub_reset(0);
    CHECK(tk_release_stream(s) == TK_OK, "fill case release");
    stub_reset(0);
    (void)topk(s, 15, 98592, 32);
    const std::string t = stub_trace();
    const size_t z = t.find('z');
    CHECK(z != std::string::npos, "no zero fill in %s", t.c_str());
    stub_reset(0);
    CHECK(tk_release_stream(s) == TK_OK, "fill case release 2");
    stub_reset((int)z + 1);
    CHECK(topk(s, 15, 98592, 32) == TK_ERR_DEVICE, "fill failure status");
    stub_reset(0);
    CHECK(topk(s, 15, 98592, 32) == TK_OK, "call after fill failure");
    CHECK(stub_counters().fills == 1, "the call after a failed fill zeroed %d buffers", stub_counters().fills);
    stub_reset(0);
    (void)tk_release_stream(s);
  }
  // release of a stream the library never saw
  stub_reset(0);
  CHECK(tk_release_stream((void *)0x7777) == TK_OK, "release unknown stream");
  CHECK(stub_errors() == 0, "%d scratch ranges outside their allocations", stub_errors());
  CHECK(stub_live_allocations() == 0, "%zu allocations left at the end", stub_live_allocations());
}

// ---------------------------------------------------------------------------
// The oracle against the rank definition on small random rows.

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint32_t rnd() {
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return (uint32_t)g_rng;
}

double value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

bool is_nan(uint16_t b) { return (b & 0x7FFF) > 0x7F80; }

void oracle_rows() {
  const uint16_t symbols[] = {0x7FC0, 0xFFC1, 0x7F80, 0xFF80, 0x3F80, 0xBF80, 0x0001, 0x8001, 0x0000, 0x8000};
  int cases = 0;
  for (int it = 0; it < 400; ++it) {
    const int rows = 1 + (int)(rnd() % 4), cols = (int)(rnd() % 70), pad = (int)(rnd() % 5), k = 1 + (int)(rnd() % 80);
    const int stride = cols + pad;
    std::vector<uint16_t> in((size_t)rows * stride + 1);
    for (auto &v : in) v = (rnd() & 3) ? (uint16_t)rnd() : symbols[rnd() % 10];
    std::vector<int32_t> idx((size_t)rows * k);
    std::vector<uint16_t> val((size_t)rows * k);
    std::vector<int32_t> cnt(rows);
    std::vector<uint32_t> msk(rows);
    const int threads = 1 + (int)(rnd() % 3);
    CHECK(tko_topk_bf16(rows, cols, stride, k, in.data(), idx.data(), val.data(), cnt.data(), msk.data(), threads) ==
              0,
          "oracle call");
    for (int r = 0; r < rows; ++r) {
      const uint16_t *row = in.data() + (size_t)r * stride;
      int nonnan = 0;
      uint32_t mask = 0;
      for (int c = 0; c < cols; ++c) {
        if (is_nan(row[c])) mask |= 1;
        else ++nonnan;
        if (row[c] == 0x7F80) mask |= 2;
        if (row[c] == 0xFF80) mask |= 4;
      }
      CHECK(cnt[r] == (nonnan < k ? nonnan : k), "count row %d", r);
      CHECK(msk[r] == mask, "mask row %d", r);
      for (int c = 0; c < cols; ++c) {
        if (is_nan(row[c])) continue;
        int rank = 0;  // elements that beat c: larger value, or equal value at a lower column
        for (int o = 0; o < cols; ++o)
          if (!is_nan(row[o]) && (value(row[o]) > value(row[c]) || (value(row[o]) == value(row[c]) && o < c))) ++rank;
        if (rank < k) {
          CHECK(idx[(size_t)r * k + rank] == c, "entry %d of row %d", rank, r);
          CHECK(val[(size_t)r * k + rank] == row[c], "value %d of row %d", rank, r);
        }
      }
      for (int j = cnt[r]; j < k; ++j)
        CHECK(idx[(size_t)r * k + j] == -1 && val[(size_t)r * k + j] == 0x7FC0, "fill %d of row %d", j, r);
    }
    ++cases;
  }
  printf("oracle: %d random cases equal to the rank definition\n", cases);
}

}  // namespace

int main() {
  host_api();
  oracle_rows();
  if (g_fail) {
    fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  printf("host driver: all checks passed\n");
  return 0;
}
