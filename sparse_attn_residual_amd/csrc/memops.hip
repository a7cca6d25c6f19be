// Runtime pieces of the C ABI layer outside the kernels: the synchronous
// host copies of the FL_CHECK validator, a device-to-device copy on the
// caller's stream (kept behind the launch layer so that the validation code
// can be exercised on the CPU against host arrays), and the opt-in kernel
// timer behind FL_LAUNCH.
#include <cstdio>
#include <vector>

#include "launch.hpp"

namespace fl {

hipError_t copy_to_host(void* dst, const void* src, size_t bytes, hipStream_t st) {
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  return hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
}

hipError_t copy_rows_to_host(void* dst, size_t dst_pitch, const void* src, size_t src_pitch, size_t width,
                             size_t rows, hipStream_t st) {
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  return hipMemcpy2D(dst, dst_pitch, src, src_pitch, width, rows, hipMemcpyDeviceToHost);
}

hipError_t copy_d2d_async(void* dst, const void* src, size_t bytes, hipStream_t st) {
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st);
}

}  // namespace fl

// ---------------------------------------------------------------- kernel timing
namespace {

struct TimingRec {
  const char* name;
  hipEvent_t e0, e1;
};
thread_local bool t_on = false;
thread_local std::vector<TimingRec> t_recs;
thread_local std::vector<hipEvent_t> t_pool;

hipEvent_t take_event() {
  if (!t_pool.empty()) {
    hipEvent_t e = t_pool.back();
    t_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace fl {

TimedLaunch::TimedLaunch(const char* name, hipStream_t s) : st(s), slot(-1) {
  if (!t_on) return;
  TimingRec r{name, take_event(), take_event()};
  if (!r.e0 || !r.e1 || hipEventRecord(r.e0, s) != hipSuccess) {
    if (r.e0) t_pool.push_back(r.e0);
    if (r.e1) t_pool.push_back(r.e1);
    return;
  }
  t_recs.push_back(r);
  slot = (int)t_recs.size() - 1;
}

TimedLaunch::~TimedLaunch() {
  if (slot >= 0) (void)hipEventRecord(t_recs[slot].e1, st);
}

}  // namespace fl

extern "C" void fl_timing_enable(int on) { t_on = on != 0; }

extern "C" int fl_timing_collect(char (*names)[FL_TIMING_NAME], float* ms, int max) {
  int n = 0;
  for (const TimingRec& r : t_recs) {
    if (n < max && names && ms && hipEventSynchronize(r.e1) == hipSuccess) {
      float t = 0.0f;
      if (hipEventElapsedTime(&t, r.e0, r.e1) != hipSuccess) t = -1.0f;
      // the launch expression's text, without the parentheses around templates
      char* out = names[n];
      int k = 0;
      for (const char* p = r.name; *p && k < FL_TIMING_NAME - 1; ++p)
        if (*p != '(' && *p != ')') out[k++] = *p;
      out[k] = 0;
      ms[n] = t;
      ++n;
    } else {
      (void)hipEventSynchronize(r.e1);
    }
    t_pool.push_back(r.e0);
    t_pool.push_back(r.e1);
  }
  t_recs.clear();
  return n;
}
