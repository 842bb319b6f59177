// Per-kernel HIP-event timing behind pkv_timing_enable / pkv_timing_collect.
#include "timing.h"

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/pkv.h"

namespace {

struct Pending {
  const char* kernel;
  hipEvent_t start;
  hipEvent_t stop;
};

struct Total {
  const char* kernel;
  int64_t launches;
  double total_ms, min_ms, max_ms;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_spare;
thread_local Pending t_open = {nullptr, nullptr, nullptr};

hipEvent_t take_event() {
  if (!g_spare.empty()) {
    hipEvent_t e = g_spare.back();
    g_spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace pkv {

void timing_begin(const char* kernel, hipStream_t stream) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &capture) != hipSuccess ||
      capture != hipStreamCaptureStatusNone)
    return;  // launches captured into a graph are not timed
  std::lock_guard<std::mutex> lk(g_mu);
  t_open = {kernel, take_event(), take_event()};
  // a pair that could not be created in full drops this launch from the timing
  if (t_open.start == nullptr || t_open.stop == nullptr) {
    if (t_open.start) g_spare.push_back(t_open.start);
    if (t_open.stop) g_spare.push_back(t_open.stop);
    t_open = {nullptr, nullptr, nullptr};
  }
}

hipEvent_t timing_start() { return t_open.start; }

hipEvent_t timing_stop() { return t_open.stop; }

void timing_end(hipStream_t stream) {
  (void)stream;
  if (t_open.kernel == nullptr) return;
  std::lock_guard<std::mutex> lk(g_mu);
  // the launch recorded both events unless it was refused
  if (hipPeekAtLastError() == hipSuccess) {
    g_pending.push_back(t_open);
  } else {
    g_spare.push_back(t_open.start);
    g_spare.push_back(t_open.stop);
  }
  t_open = {nullptr, nullptr, nullptr};
}

}  // namespace pkv

extern "C" {

pkv_status pkv_timing_enable(int32_t on) {
  g_on.store(on != 0);
  return PKV_OK;
}

}  // extern "C"

namespace {

// Waits for every recorded launch and returns (kernel, ms) in launch order; the events
// go back to the spare list.  *status is set to PKV_ERR_HIP if an event failed (that
// launch is dropped).
std::vector<std::pair<const char*, float>> drain(int32_t* status) {
  std::vector<Pending> done;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    done.swap(g_pending);
  }
  std::vector<std::pair<const char*, float>> res;
  res.reserve(done.size());
  for (const Pending& p : done) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
      *status = PKV_ERR_HIP;
      continue;
    }
    res.emplace_back(p.kernel, ms);
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (const Pending& p : done) {
      g_spare.push_back(p.start);
      g_spare.push_back(p.stop);
    }
  }
  return res;
}

}  // namespace

extern "C" {

int32_t pkv_timing_collect(pkv_kernel_timing* out, int32_t capacity) {
  int32_t status = 0;
  std::vector<Total> totals;
  for (const auto& [kernel, ms] : drain(&status)) {
    Total* t = nullptr;
    for (Total& x : totals)
      if (std::strcmp(x.kernel, kernel) == 0) t = &x;
    if (t == nullptr) {
      totals.push_back({kernel, 0, 0.0, 1e300, 0.0});
      t = &totals.back();
    }
    t->launches += 1;
    t->total_ms += ms;
    if (ms < t->min_ms) t->min_ms = ms;
    if (ms > t->max_ms) t->max_ms = ms;
  }
  if (status != 0) return status;
  const int32_t n = static_cast<int32_t>(totals.size());
  for (int32_t i = 0; i < n && i < capacity && out != nullptr; ++i) {
    std::strncpy(out[i].kernel, totals[i].kernel, sizeof(out[i].kernel) - 1);
    out[i].kernel[sizeof(out[i].kernel) - 1] = '\0';
    out[i].launches = totals[i].launches;
    out[i].total_ms = totals[i].total_ms;
    out[i].min_ms = totals[i].min_ms;
    out[i].max_ms = totals[i].max_ms;
  }
  return n;
}

int32_t pkv_timing_samples(pkv_kernel_sample* out, int32_t capacity) {
  int32_t status = 0;
  const auto res = drain(&status);
  if (status != 0) return status;
  const int32_t n = static_cast<int32_t>(res.size());
  for (int32_t i = 0; i < n && i < capacity && out != nullptr; ++i) {
    std::strncpy(out[i].kernel, res[i].first, sizeof(out[i].kernel) - 1);
    out[i].kernel[sizeof(out[i].kernel) - 1] = '\0';
    out[i].ms = res[i].second;
  }
  return n;
}

}  // extern "C"
