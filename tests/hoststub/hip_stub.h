// Control of the stand-in device layer (hip_stub.cpp) for host-only builds of
// the C ABI.  Test infrastructure only.
#pragma once

#include <stddef.h>

struct StubCounters {
  int mallocs, frees, launches, fills, fixed;
};

extern "C" {
void stub_reset(int fail_at);          // counters to zero; fail the fail_at-th fallible call (0: none)
int stub_fallible_calls(void);         // fallible calls since the reset
int stub_errors(void);                 // scratch ranges found outside every allocation, ever
size_t stub_live_allocations(void);    // "device" allocations not freed
StubCounters stub_counters(void);
const char *stub_trace(void);          // one letter per fallible call since the reset
void *stub_fixed_base(void);
}
