// libflux device checks (off by default): a read-only pass over a tensor that
// ORs a bit into a per-device status word when a value falls outside a range.
// Timesteps outside [0, 1] ("Flux model API reference", Common issues: the
// timestep range) and non-finite activations, losses or gradients are the
// preconditions the entry points do not check on the device in normal runs.
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "api_common.h"

using namespace flux;
using namespace flux::api;

namespace {

// One word per device (each GPU holds its own copy of a __device__ variable);
// the kernels below are the only device code that touches it.
__device__ uint32_t g_debug_status;

std::atomic<int> g_debug_on{-1};   // -1: not read from the environment yet

// status |= bit if any of the n values (fp32, bf16 or fp16) is outside
// [lo, hi] or NaN.  Grid-stride, one value per thread per step.
__global__ void __launch_bounds__(256) debug_range_kernel(const void* p, int dt, int64_t n, float lo, float hi,
                                                          uint32_t bit) {
  bool bad = false;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    float v;
    if (dt == kF32) v = reinterpret_cast<const float*>(p)[i];
    else if (dt == kF16) v = (float)reinterpret_cast<const _Float16*>(p)[i];
    else v = bf16_to_f32(reinterpret_cast<const bf16_t*>(p)[i]);
    bad |= !(v >= lo && v <= hi);
  }
  // one atomic per wave that saw a bad value (every lane reaches this point)
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(&g_debug_status, bit);
}

}  // namespace

namespace flux {
namespace api {

bool debug_checks_on() {
  int v = g_debug_on.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = getenv("FLUX_DEBUG_CHECKS");
    const int want = (e && strcmp(e, "0") != 0 && e[0] != '\0') ? 1 : 0;
    int expect = -1;
    g_debug_on.compare_exchange_strong(expect, want);
    v = g_debug_on.load(std::memory_order_relaxed);
  }
  return v > 0;
}

hipError_t debug_check(const void* p, int dt, int64_t rows, int64_t cols, int64_t row_stride, float lo, float hi,
                       uint32_t bit, hipStream_t st) {
  if (!p || rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t es = dt == kF32 ? 4 : 2;
  // contiguous rows: one pass; strided rows (a per-sample residual with
  // padding): one launch per row block of the same stride
  if (row_stride == cols) {
    const int64_t n = rows * cols;
    const int64_t blocks = ceil_div(n, 256) < 1024 ? ceil_div(n, 256) : 1024;
    hipLaunchKernelGGL(debug_range_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, dt, n, lo, hi, bit);
    return hipGetLastError();
  }
  for (int64_t r = 0; r < rows; ++r) {
    const void* q = static_cast<const char*>(p) + r * row_stride * es;
    const int64_t blocks = ceil_div(cols, 256) < 1024 ? ceil_div(cols, 256) : 1024;
    hipLaunchKernelGGL(debug_range_kernel, dim3((unsigned)blocks), dim3(256), 0, st, q, dt, cols, lo, hi, bit);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace api
}  // namespace flux

extern "C" {

int32_t flux_debug_checks(int32_t on) {
  const int prev = debug_checks_on() ? 1 : 0;
  if (on >= 0) g_debug_on.store(on ? 1 : 0, std::memory_order_relaxed);
  return prev;
}

flux_status flux_debug_status(uint32_t* status, int32_t clear) {
  g_err[0] = 0;
  REQUIRE(status, "status is NULL");
  FLUX_HIP(hipDeviceSynchronize(), "device synchronize");
  uint32_t v = 0;
  FLUX_HIP(hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_status), sizeof(v), 0, hipMemcpyDeviceToHost),
           "read the status word");
  if (clear) {
    const uint32_t zero = 0;
    FLUX_HIP(hipMemcpyToSymbol(HIP_SYMBOL(g_debug_status), &zero, sizeof(zero), 0, hipMemcpyHostToDevice),
             "clear the status word");
  }
  *status = v;
  return FLUX_OK;
}

}  // extern "C"
