// Kernel classes and the RAII launch bracket used by the opt-in timing hook.
#pragma once
#include <hip/hip_runtime.h>

namespace flux {

enum KernelClass : int {
  kKcGemmPkF16 = 0,   // gemm_dl_kernel (256 x 256 persistent), fp16 activations
  kKcGemmPkBf16,      // gemm_dl_kernel, bf16 activations
  kKcGemm128,         // gemm_mfma_kernel (128 x 128 tiles)
  kKcGemmF32,
  kKcAttn,
  kKcLnMod,
  kKcGemv,
  kKcPrep,
  kKcRf,
  kKcMisc,
  kKcGemmPkFp8,       // gemm_fp8_kernel (E4M3 operands)
  kKcFp8Cast,         // fp8 quantization of a whole tensor (weight cast)
  kKcGemmPkMx,        // gemm_fp8_kernel with MXFP8 block scales
  kKcMxQuant,         // MXFP8 quantization
  kKcAttnBwd,         // attention backward (dK / dV and dQ kernels)
  kKcBwdElem,         // backward row-wise, element-wise, transpose and reduction kernels
  kKcGemmPkMx4,       // gemm_fp8_kernel on MXFP4 operands
  kKcMx4Quant,        // MXFP4 quantization
  kKcCopy,            // flux_stream_copy (the HBM streaming reference)
  kKcCount
};

// Records a start event on `s` at construction and a stop event at
// destruction when timing is enabled; does nothing otherwise.  With a flush
// buffer set (flux_timing_flush), the construction first enqueues a kernel
// that overwrites that buffer, so the timed launch starts with its data
// evicted from L2 and the Infinity Cache.  `work` is the
// launch's algorithmic work: FLOPs for the GEMM and attention classes, bytes
// that must cross HBM for the others.
class TimingScope {
 public:
  TimingScope(int cls, hipStream_t s, double work = 0.0);
  ~TimingScope();
  TimingScope(const TimingScope&) = delete;
  TimingScope& operator=(const TimingScope&) = delete;

 private:
  int cls_;
  double work_;
  hipStream_t stream_;
  hipEvent_t start_;
};

}  // namespace flux
