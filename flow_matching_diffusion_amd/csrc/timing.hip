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
uint4* g_flush = nullptr;       // caller-owned buffer overwritten before each timed launch
int64_t g_flush_n = 0;          // its size in 16-byte words
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
                                "gemm_256_mxfp4", "mxfp4_quantize", "hbm_copy"};

// Streaming stores over the flush buffer (grid-stride, 16 bytes per lane).
__global__ void __launch_bounds__(256) flush_kernel(uint4* p, int64_t n, uint32_t salt) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] = make_uint4(salt, (uint32_t)i, salt, (uint32_t)(i >> 32));
}

// 16 bytes per lane per step, four independent loads in flight per lane
// before the stores, grid-stride over n 16-byte words (+ a byte tail).
__global__ void __launch_bounds__(256) stream_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                          int64_t n, const uint8_t* __restrict__ src_tail,
                                                          uint8_t* __restrict__ dst_tail, int tail) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
  if (blockIdx.x == 0 && (int)threadIdx.x < tail) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}
}  // namespace

TimingScope::TimingScope(int cls, hipStream_t s, double work) : cls_(cls), work_(work), stream_(s), start_(nullptr) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_flush && g_flush_n > 0) {
    static uint32_t salt = 0;
    hipLaunchKernelGGL(flush_kernel, dim3(2048), dim3(256), 0, stream_, g_flush, g_flush_n, ++salt);
  }
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

flux_status flux_timing_flush(void* buffer, int64_t bytes) {
  if (buffer && ((reinterpret_cast<uintptr_t>(buffer) & 15u) || bytes < 16)) return FLUX_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lk(g_mu);
  g_flush = buffer ? static_cast<uint4*>(buffer) : nullptr;
  g_flush_n = buffer ? bytes / 16 : 0;
  return FLUX_OK;
}

flux_status flux_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || bytes < 1) return FLUX_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u))
    return FLUX_ERR_INVALID_ARGUMENT;
  const char* a = static_cast<const char*>(src);
  const char* b = static_cast<const char*>(dst);
  if (a < b + bytes && b < a + bytes) return FLUX_ERR_INVALID_ARGUMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t n = bytes / 16;
  const int tail = (int)(bytes - n * 16);
  TimingScope ts(kKcCopy, st, 2.0 * (double)bytes);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), n, reinterpret_cast<const uint8_t*>(a + n * 16),
                     reinterpret_cast<uint8_t*>(const_cast<char*>(b) + n * 16), tail);
  return hipGetLastError() == hipSuccess ? FLUX_OK : FLUX_ERR_HIP;
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
