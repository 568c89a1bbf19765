// Measurement hook: optional HIP events around kernel launches, enabled by
// moe_profile_start().  Off by default; then each launch site pays one
// thread-local flag test.  Host code only.
#include <vector>

#include "../../include/moe.h"
#include "launch.hpp"

namespace moe {
namespace {
struct Prof {
  int mode = 0, which = 0, capacity = 0;
  int call_launch = 0;       // launches so far in the current entry-point call
  int n = 0;                 // recorded pairs
  bool open = false;         // a start event is pending its stop
  std::vector<hipEvent_t> start, stop;
  std::vector<const char*> name;
};
thread_local Prof g;

void release() {
  for (auto e : g.start) hipEventDestroy(e);
  for (auto e : g.stop) hipEventDestroy(e);
  g.start.clear();
  g.stop.clear();
  g.name.clear();
  g.mode = g.n = g.capacity = 0;
  g.open = false;
}
}  // namespace

void prof_call_begin() { g.call_launch = 0; }

bool prof_serial() { return g.mode == 1; }

void prof_before(const char* name, hipStream_t s) {
  if (g.mode == 0) return;
  const bool take = (g.mode == 1 || g.call_launch == g.which) && g.n < g.capacity;
  if (take) {
    hipEventRecord(g.start[g.n], s);
    g.name[g.n] = name;
    g.open = true;
  }
}

void prof_after(hipStream_t s) {
  if (g.mode == 0) return;
  if (g.open) {
    hipEventRecord(g.stop[g.n], s);
    ++g.n;
    g.open = false;
  }
  ++g.call_launch;
}

}  // namespace moe

extern "C" {

int moe_profile_start(int mode, int which, int capacity) {
  moe::release();
  if (mode < 1 || mode > 2 || capacity < 1 || which < 0) return MOE_ERR_INVALID_ARG;
  moe::g.start.resize(capacity);
  moe::g.stop.resize(capacity);
  moe::g.name.assign(capacity, nullptr);
  for (int i = 0; i < capacity; ++i) {
    // Timing-only events: no system-scope fence (its cache write-back and
    // invalidation would slow the launches that follow each record).
    if (hipEventCreateWithFlags(&moe::g.start[i], hipEventDisableSystemFence) != hipSuccess ||
        hipEventCreateWithFlags(&moe::g.stop[i], hipEventDisableSystemFence) != hipSuccess) {
      moe::g.start.resize(i);
      moe::g.stop.resize(i);
      moe::release();
      return MOE_ERR_HIP;
    }
  }
  moe::g.mode = mode;
  moe::g.which = which;
  moe::g.capacity = capacity;
  moe::g.n = 0;
  return MOE_OK;
}

int moe_profile_count(void) { return moe::g.n; }

int moe_profile_read(int i, float* ms, const char** name) {
  if (i < 0 || i >= moe::g.n || ms == nullptr) return MOE_ERR_INVALID_ARG;
  if (hipEventSynchronize(moe::g.stop[i]) != hipSuccess) return MOE_ERR_HIP;
  if (hipEventElapsedTime(ms, moe::g.start[i], moe::g.stop[i]) != hipSuccess) return MOE_ERR_HIP;
  if (name) *name = moe::g.name[i];
  return MOE_OK;
}

int moe_profile_stop(void) {
  moe::release();
  return MOE_OK;
}

}  // extern "C"
