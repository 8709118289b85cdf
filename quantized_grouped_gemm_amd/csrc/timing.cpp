// Measurement hook: caller-owned HIP events recorded around the library's
// kernel launches, so that a benchmark can time one kernel inside a whole call
// on the stream it runs on.  Per calling thread; off unless events are set.
#include <hip/hip_runtime.h>

#include "qgg.h"
#include "qgg_internal.hpp"

namespace qgg {
namespace {

constexpr int kMaxTimed = 4096;

struct TimingState {
  hipEvent_t const* events = nullptr;   // 2 * capacity, begin / end per launch
  int capacity = 0;
  int count = 0;
  int depth = 0;
  int32_t kinds[kMaxTimed];
};

thread_local TimingState tl;

}  // namespace

void timing_begin(int kind, hipStream_t s) {
  if (tl.depth++ > 0 || !tl.events || tl.count >= tl.capacity) return;
  if (hipEventRecord(tl.events[2 * tl.count], s) != hipSuccess) return;
  tl.kinds[tl.count] = kind;
}

void timing_end(hipStream_t s) {
  if (--tl.depth > 0 || !tl.events || tl.count >= tl.capacity) return;
  if (hipEventRecord(tl.events[2 * tl.count + 1], s) == hipSuccess) ++tl.count;
}

}  // namespace qgg

using namespace qgg;

extern "C" {

qgg_status qgg_set_timing_events(void* const* events, int capacity) {
  if (events && (capacity <= 0 || capacity > kMaxTimed)) return QGG_ERR_INVALID_ARG;
  tl.events = reinterpret_cast<hipEvent_t const*>(events);
  tl.capacity = events ? capacity : 0;
  tl.count = 0;
  tl.depth = 0;
  return QGG_OK;
}

int qgg_timing_count(void) { return tl.count; }

int qgg_timing_kind(int i) { return (i >= 0 && i < tl.count) ? tl.kinds[i] : 0; }

}  // extern "C"
