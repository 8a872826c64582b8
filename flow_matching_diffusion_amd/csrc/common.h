// Device helpers shared by the HIP kernels of libflux (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/flux.h"

namespace flux {

typedef uint16_t bf16_t;                                            // storage: raw bf16 bits
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));        // MFMA operand (8 x bf16)
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));       // MFMA operand (8 x fp16)
typedef float f32x16_t __attribute__((ext_vector_type(16)));        // 32x32 MFMA accumulator
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));       // 16-byte raw vector

constexpr int kWave = 64;

// ---- bf16 <-> fp32 (round to nearest even; NaN kept quiet) -------------------
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  // v_cvt_pk_bf16_f32 on gfx950: round to nearest even, NaN stays NaN
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// fp32 -> fp16 with saturation: magnitudes above fp16's largest finite value
// (65504, infinities included) become +-65504 instead of infinity, so an
// out-of-range activation cannot turn into inf and then NaN downstream.
// NaN stays NaN (the comparison is false for it).
__device__ __forceinline__ _Float16 f32_to_f16_sat(float x) {
  const float c = fabsf(x) > 65504.0f ? copysignf(65504.0f, x) : x;
  return (_Float16)c;
}

// fp32 -> fp16 (round to nearest even, saturating), two values packed low | high
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, f32_to_f16_sat(lo)) |
         ((uint32_t)__builtin_bit_cast(uint16_t, f32_to_f16_sat(hi)) << 16);
}

// Four 16-bit values (an 8-byte word, low half first) to fp32 and back:
// fp16 when f16, else bf16; the stores round to nearest even (fp16 saturating).
__device__ __forceinline__ void unpack4_16(uint2 u, bool f16, float* v) {
  const uint32_t w[2] = {u.x, u.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (f16) {
      v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
      v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    } else {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

__device__ __forceinline__ uint2 pack4_16(const float* v, bool f16) {
  uint2 u;
  u.x = f16 ? pack_f16x2(v[0], v[1]) : pack_bf16x2(v[0], v[1]);
  u.y = f16 ? pack_f16x2(v[2], v[3]) : pack_bf16x2(v[2], v[3]);
  return u;
}

// Eight bf16 (a 16-byte word) to eight fp16, rounding toward zero.  Exact for
// magnitudes in fp16's normal range [2^-14, 65504]; smaller magnitudes lose
// at most 2^-24 (the few bits fp16 subnormals cannot hold); finite magnitudes
// above 65504 become +-65504 (toward zero never rounds up to infinity).
__device__ __forceinline__ u32x4_t bf16x8_to_f16x8(u32x4_t w) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
    r[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return r;
}

// Storage-type adapters: T is float (fp32 workloads), bf16_t or _Float16.
template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }
template <> __device__ __forceinline__ float load_f32<_Float16>(const _Float16* p) { return (float)*p; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float v) { return f32_to_f16_sat(v); }

// Block barrier for LDS hand-offs that leaves global loads in flight: the
// wave's own LDS accesses are complete before it arrives (lgkmcnt(0)), but
// outstanding global loads are not waited for.  __syncthreads() would also
// wait for every one of them (its workgroup fences imply s_waitcnt
// vmcnt(0)): for loads into registers the compiler waits where the registers
// are used, and for direct-to-LDS loads the caller bounds them with a
// counted vmcnt wait first.  The asm statements keep the compiler from
// moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) leaving expcnt / lgkmcnt unconstrained (gfx9 encoding)
#define DL_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

// LDS and global address-space pointers of the direct global -> LDS loads.
// Their integer operands are passed as plain int expressions: an operand of a
// template-dependent type keeps the host compiler from emitting the kernel's
// launch stub.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// ---- wave reductions (fixed butterfly order -> deterministic) ---------------
template <int WIDTH = kWave>
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
  return v;
}
template <int WIDTH = kWave>
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WIDTH));
  return v;
}
// max of unsigned values over the wave (used on |x| bit patterns for amax)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}
// bit pattern of |x|: orders like |x| for non-negative values, NaN above all
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7fffffffu; }
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---- activations -------------------------------------------------------------
__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }
// GELU, erf form: x * Phi(x) = x (1 + erf(x / sqrt 2)) / 2.  erf by the
// rational approximation 7.1.26 of Abramowitz and Stegun, "Handbook of
// Mathematical Functions" (1964): for a >= 0, erf(a) = 1 - t (a1 + t (a2 +
// t (a3 + t (a4 + t a5)))) exp(-a^2), t = 1 / (1 + p a), |error| <= 1.5e-7;
// erf is odd.  About half the instructions of the library erff, which
// matters in the GEMM epilogues that apply it to every MLP activation.
__device__ __forceinline__ float erf_as(float x) {
  const float a = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, a, 1.0f));
  float poly = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  poly = __builtin_fmaf(poly, t, 1.421413741f);
  poly = __builtin_fmaf(poly, t, -0.284496736f);
  poly = __builtin_fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float e = __builtin_amdgcn_exp2f(-a * a * 1.4426950408889634f);
  return copysignf(__builtin_fmaf(-poly, e, 1.0f), x);
}
__device__ __forceinline__ float gelu_f(float x) { return 0.5f * x * (1.0f + erf_as(x * 0.70710678118654752f)); }

// ---- OCP E4M3FN ("FP8 training for Flux models", Configuration: fp8 e4m3) ----
// Byte of the nearest E4M3FN value to x, ties to the even code; |x| > 448
// (infinities included) saturates to +-448; NaN stays NaN (0x7F | sign).
// Written from the format: 4 exponent bits with bias 7, 3 mantissa bits,
// subnormals m * 2^-9 under 2^-6.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a > 0x7f800000u) {
    code = 0x7fu;                                           // NaN
  } else if (a > 0x43e00000u) {
    code = 0x7eu;                                           // above 448: saturate
  } else if (a >= 0x3c800000u) {
    // normal: keep 3 of fp32's 23 mantissa bits, round half to even; a carry
    // out of the mantissa moves into the exponent by itself
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);                         // exponent bias 127 -> 7
  } else {
    // subnormal range: nearest multiple of 2^-9 (the product is exact), ties to even
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return code | sign;
}

// Four values as E4M3FN bytes (x0 in the low byte), the same bytes as
// f32_to_e4m3 on each: v_med3 saturates finite and infinite values to
// +-448, then the conversion instruction rounds to nearest even (subnormals
// included).  A NaN comes out of med3 as a number, so a group holding one
// takes the bit-level path.  Checked equal to f32_to_e4m3 over all 2^32 fp32
// patterns in every byte position.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float x0, float x1, float x2, float x3) {
  const float c0 = __builtin_amdgcn_fmed3f(x0, -448.0f, 448.0f);
  const float c1 = __builtin_amdgcn_fmed3f(x1, -448.0f, 448.0f);
  const float c2 = __builtin_amdgcn_fmed3f(x2, -448.0f, 448.0f);
  const float c3 = __builtin_amdgcn_fmed3f(x3, -448.0f, 448.0f);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, (int)w, true);
  if (__builtin_isnan(x0) || __builtin_isnan(x1) || __builtin_isnan(x2) || __builtin_isnan(x3))
    w = f32_to_e4m3(x0) | (f32_to_e4m3(x1) << 8) | (f32_to_e4m3(x2) << 16) | (f32_to_e4m3(x3) << 24);
  return w;
}

__device__ __forceinline__ float fp8_scale(const flux_fp8_tensor* r) {
  return (r->flags & FLUX_FP8_SCALE_SET) ? r->scale : 1.0f;
}
__device__ __forceinline__ float fp8_scale_inv(const flux_fp8_tensor* r) {
  return (r->flags & FLUX_FP8_SCALE_SET) ? r->scale_inv : 1.0f;
}
// Raise the record's amax to m (m >= 0 or NaN): fp32 bit patterns of
// non-negative values order like unsigned integers, and a NaN's pattern is
// above every finite one, so the update sees it.  Vector-memory atomic.
__device__ __forceinline__ void fp8_amax_raise(flux_fp8_tensor* r, float m) {
  atomicMax(&r->amax_bits, __float_as_uint(m) & 0x7fffffffu);
}

// Eight E4M3 bytes to eight fp16 (exact: every E4M3 value is an fp16 value).
// Placing the byte's exponent and mantissa fields at fp16's exponent and
// mantissa positions gives the value times 2^-8 (for subnormals too), so one
// multiply by 256 restores it.  NaN bytes are not expected here.
__device__ __forceinline__ u32x4_t e4m3x8_to_f16x8(uint2 w) {
  u32x4_t r;
  const uint32_t in[2] = {w.x, w.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t b0 = (in[i] >> (16 * j)) & 0xffu, b1 = (in[i] >> (16 * j + 8)) & 0xffu;
      const uint16_t h0 = (uint16_t)(((b0 & 0x7fu) << 7) | ((b0 & 0x80u) << 8));
      const uint16_t h1 = (uint16_t)(((b1 & 0x7fu) << 7) | ((b1 & 0x80u) << 8));
      const _Float16 f0 = __builtin_bit_cast(_Float16, h0) * (_Float16)256.0f;
      const _Float16 f1 = __builtin_bit_cast(_Float16, h1) * (_Float16)256.0f;
      r[2 * i + j] = (uint32_t)__builtin_bit_cast(uint16_t, f0) | ((uint32_t)__builtin_bit_cast(uint16_t, f1) << 16);
    }
  }
  return r;
}

// ---- integer helpers ---------------------------------------------------------
__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace flux
