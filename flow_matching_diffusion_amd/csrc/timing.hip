// Opt-in kernel timing: while enabled, every kernel launch made by the library
// is bracketed by a pair of hipEvents recorded on the launch's own stream.
// flux_timing_read() waits for the recorded events and returns the summed
// duration and launch count per kernel class.  Disabled by default; when
// disabled a scope costs one relaxed atomic load.
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/flux.h"
#include "timing.h"

namespace flux {

namespace {
struct Record {
  int cls;
  double work;
  hipEvent_t start, stop;
};
std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

const char* kNames[kKcCount] = {"gemm_256_f16", "gemm_256_bf16", "gemm_128x128", "gemm_f32", "attention",
                                "ln_modulate",       "gemv",              "qk_prep",  "rf_noise_loss",
                                "misc",        "gemm_256_fp8",       "fp8_quantize",
                                "gemm_256_mxfp8", "mx_quantize", "attention_bwd", "bwd_elementwise",
                                "gemm_256_mxfp4", "mxfp4_quantize"};
}  // namespace

TimingScope::TimingScope(int cls, hipStream_t s, double work) : cls_(cls), work_(work), stream_(s), start_(nullptr) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  start_ = take_event();
  if (start_ && hipEventRecord(start_, stream_) != hipSuccess) {
    g_pool.push_back(start_);
    start_ = nullptr;
  }
}

TimingScope::~TimingScope() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t stop = take_event();
  if (!stop || hipEventRecord(stop, stream_) != hipSuccess) {
    g_pool.push_back(start_);
    if (stop) g_pool.push_back(stop);
    return;
  }
  g_records.push_back(Record{cls_, work_, start_, stop});
}

}  // namespace flux

using namespace flux;

extern "C" {

flux_status flux_timing_enable(int32_t on) {
  g_on.store(on != 0, std::memory_order_relaxed);
  return FLUX_OK;
}

int32_t flux_timing_classes(void) { return kKcCount; }

const char* flux_timing_class_name(int32_t cls) { return (cls >= 0 && cls < kKcCount) ? kNames[cls] : ""; }

flux_status flux_timing_read(double* ms, int64_t* launches, double* work, int32_t n) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (int i = 0; i < n; ++i) {
    if (ms) ms[i] = 0.0;
    if (launches) launches[i] = 0;
    if (work) work[i] = 0.0;
  }
  flux_status st = FLUX_OK;
  for (const Record& r : g_records) {
    float t = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess)
      st = FLUX_ERR_HIP;
    if (r.cls < n) {
      if (ms) ms[r.cls] += t;
      if (launches) launches[r.cls] += 1;
      if (work) work[r.cls] += r.work;
    }
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_records.clear();
  return st;
}

}  // extern "C"
