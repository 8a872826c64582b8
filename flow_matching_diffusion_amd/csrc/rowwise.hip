// Row-wise and elementwise kernels of the Flux block forward (gfx950, wave64):
// rectified-flow noising and loss, timestep sinusoid, 3D RoPE table,
// patchify, LayerNorm + adaLN modulate, modulation GEMV, q/k RMSNorm + RoPE.
#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace flux {

// ===========================================================================
// Rectified flow ("Flux architecture deep dive", Flow matching framework and
// Mathematical formulation / Flow matching objective).
// ===========================================================================
// z_t = (1 - t) z0 + t z1 as two rounded products and one rounded sum;
// v* = z1 - z0.  Contraction into an FMA is switched off for this kernel, so
// the result is the same rounding sequence on every build.
__global__ void __launch_bounds__(256) rf_noise_kernel(int64_t n, const float* __restrict__ z0,
                                                       const float* __restrict__ z1, const float* __restrict__ t,
                                                       float* __restrict__ zt, float* __restrict__ vt) {
#pragma clang fp contract(off)
  const int b = blockIdx.y;
  const float tb = t[b];
  const float omt = 1.0f - tb;
  const int64_t base = (int64_t)b * n;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const bool vec4 = ((n & 3) == 0);
  if (vec4) {
    const int64_t n4 = n >> 2;
    const float4* a4 = reinterpret_cast<const float4*>(z0 + base);
    const float4* b4 = reinterpret_cast<const float4*>(z1 + base);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
      float4 a = a4[i], c = b4[i];
      if (zt) {
        float4 r;
        r.x = omt * a.x + tb * c.x;
        r.y = omt * a.y + tb * c.y;
        r.z = omt * a.z + tb * c.z;
        r.w = omt * a.w + tb * c.w;
        reinterpret_cast<float4*>(zt + base)[i] = r;
      }
      if (vt) {
        float4 v;
        v.x = c.x - a.x; v.y = c.y - a.y;
        v.z = c.z - a.z; v.w = c.w - a.w;
        reinterpret_cast<float4*>(vt + base)[i] = v;
      }
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
      const float a = z0[base + i], c = z1[base + i];
      if (zt) zt[base + i] = omt * a + tb * c;
      if (vt) vt[base + i] = c - a;
    }
  }
}

hipError_t launch_rf_noise(int batch, int64_t n, const float* z0, const float* z1, const float* t, float* zt,
                           float* vt, hipStream_t stream) {
  const int64_t work = (n & 3) == 0 ? n / 4 : n;
  int gx = (int)ceil_div(work, 256);
  if (gx > 1024) gx = 1024;
  TimingScope ts(kKcRf, stream, (double)batch * n * (8.0 + (zt ? 4.0 : 0.0) + (vt ? 4.0 : 0.0)));
  hipLaunchKernelGGL(rf_noise_kernel, dim3(gx, batch), dim3(256), 0, stream, n, z0, z1, t, zt, vt);
  return hipGetLastError();
}

// ===========================================================================
// Sampling ("Flux architecture deep dive", Sampling (inference) / Euler
// integration and Classifier-free guidance): one Euler step of dz/dt = v from
// t_cur down to t_next, z <- z - dt * g, with g = v_u + w (v_c - v_u) under
// guidance (model output rows 0..B-1 conditional, B..2B-1 unconditional) or
// g = v.  Each operation is rounded in the order written (contraction off),
// so the result is the same bits on every build.  The new z is also written
// into each of `copies` halves of the next forward's input, and t_next into
// its timestep vector.
// ===========================================================================
__global__ void __launch_bounds__(256) euler_step_kernel(int batch, int64_t n, const float* __restrict__ v, int cfg,
                                                         float w, float dt, float* __restrict__ z,
                                                         float* __restrict__ zm, int copies, float t_next,
                                                         float* __restrict__ tm, int tm_n) {
#pragma clang fp contract(off)
  const int b = blockIdx.y;
  const float* vc = v + (int64_t)b * n;
  const float* vu = v + (int64_t)(batch + b) * n;
  float* zb = z + (int64_t)b * n;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  auto step = [&](float zc, float c, float u) -> float {
    float g = c;
    if (cfg) {
      const float d = c - u;
      const float wd = w * d;
      g = u + wd;
    }
    const float s = dt * g;
    return zc - s;
  };
  if ((n & 3) == 0) {
    const int64_t n4 = n >> 2;
    for (int64_t i = i0; i < n4; i += stride) {
      const float4 c = reinterpret_cast<const float4*>(vc)[i];
      const float4 u = cfg ? reinterpret_cast<const float4*>(vu)[i] : c;
      const float4 zc = reinterpret_cast<const float4*>(zb)[i];
      const float4 r = make_float4(step(zc.x, c.x, u.x), step(zc.y, c.y, u.y), step(zc.z, c.z, u.z),
                                   step(zc.w, c.w, u.w));
      reinterpret_cast<float4*>(zb)[i] = r;
      for (int k = 0; k < copies; ++k) reinterpret_cast<float4*>(zm + ((int64_t)k * batch + b) * n)[i] = r;
    }
  } else {
    for (int64_t i = i0; i < n; i += stride) {
      const float r = step(zb[i], vc[i], cfg ? vu[i] : vc[i]);
      zb[i] = r;
      for (int k = 0; k < copies; ++k) zm[((int64_t)k * batch + b) * n + i] = r;
    }
  }
  if (tm && b == 0 && blockIdx.x == 0)
    for (int i = threadIdx.x; i < tm_n; i += blockDim.x) tm[i] = t_next;
}

hipError_t launch_euler_step(int batch, int64_t n, const float* v, int cfg, float w, float dt, float* z, float* zm,
                             int copies, float t_next, float* tm, int tm_n, hipStream_t stream) {
  const int64_t work = (n & 3) == 0 ? n / 4 : n;
  int gx = (int)ceil_div(work, 256);
  if (gx > 1024) gx = 1024;
  TimingScope ts(kKcRf, stream, (double)batch * n * ((cfg ? 12.0 : 8.0) + 4.0 + 4.0 * copies));
  hipLaunchKernelGGL(euler_step_kernel, dim3(gx, batch), dim3(256), 0, stream, batch, n, v, cfg, w, dt, z, zm,
                     copies, t_next, tm, tm_n);
  return hipGetLastError();
}

// Guidance embedding ("Flux architecture deep dive", Conditioning: the
// optional guidance scale g enters the combined vector through a Linear):
// vec[b, j] += g[b] * W[j] + bias[j], W the [D, 1] weight.
template <typename T>
__global__ void __launch_bounds__(256) guidance_embed_kernel(int batch, int dim, const float* __restrict__ g,
                                                             const T* __restrict__ w, const T* __restrict__ bias,
                                                             float* __restrict__ vec) {
  const int b = blockIdx.y;
  const float gb = g[b];
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < dim; j += gridDim.x * blockDim.x)
    vec[(int64_t)b * dim + j] += gb * load_f32<T>(w + j) + load_f32<T>(bias + j);
}

hipError_t launch_guidance_embed(int batch, int dim, const float* g, const void* w, const void* bias, int dtype,
                                 float* vec, hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(dim, 256), batch);
  TimingScope ts(kKcMisc, stream);
  if (dtype == kBF16)
    hipLaunchKernelGGL(guidance_embed_kernel<bf16_t>, grid, dim3(256), 0, stream, batch, dim, g,
                       static_cast<const bf16_t*>(w), static_cast<const bf16_t*>(bias), vec);
  else
    hipLaunchKernelGGL(guidance_embed_kernel<float>, grid, dim3(256), 0, stream, batch, dim, g,
                       static_cast<const float*>(w), static_cast<const float*>(bias), vec);
  return hipGetLastError();
}

// Velocity MSE, stage 1: block (g, b) sums (v_pred - (z1 - z0))^2 over its
// slice of sample b in fp64.  Each thread walks a fixed strided set, then a
// fixed butterfly/tree -> the same bits on every run.
constexpr int kRfLossThreads = 256;
int rf_parts_per_sample(int64_t n) {
  int64_t p = ceil_div(n, (int64_t)kRfLossThreads * 16);
  if (p < 1) p = 1;
  if (p > 256) p = 256;
  return (int)p;
}

__global__ void __launch_bounds__(kRfLossThreads) rf_loss_partial_kernel(int64_t n, const float* __restrict__ z0,
                                                                         const float* __restrict__ z1,
                                                                         const float* __restrict__ vp,
                                                                         double* __restrict__ partials) {
  const int b = blockIdx.y, g = blockIdx.x, parts = gridDim.x;
  const int64_t per = round_up(ceil_div(n, parts), 4);   // a multiple of 4: whole float4 words per part
  const int64_t lo = (int64_t)g * per;
  const int64_t hi = lo + per < n ? lo + per : n;
  const int64_t base = (int64_t)b * n;
  double acc = 0.0;
  auto sq = [&](float z0v, float z1v, float pv) {
    const float d = __fsub_rn(pv, __fsub_rn(z1v, z0v));
    acc += (double)d * (double)d;
  };
  // 16-byte path: the part's float4 words, four strides of the block at a
  // time so 12 loads per thread are in flight; each thread adds its values in
  // one fixed order, so the sum has the same bits on every run
  const bool vec4 = (n & 3) == 0 && (per & 3) == 0 &&
                    ((reinterpret_cast<uintptr_t>(z0) | reinterpret_cast<uintptr_t>(z1) |
                      reinterpret_cast<uintptr_t>(vp)) & 15) == 0;
  if (vec4) {
    const float4* a4 = reinterpret_cast<const float4*>(z0 + base);
    const float4* c4 = reinterpret_cast<const float4*>(z1 + base);
    const float4* p4 = reinterpret_cast<const float4*>(vp + base);
    const int64_t lo4 = lo >> 2, hi4 = hi >> 2;
    constexpr int S = kRfLossThreads;
    int64_t i = lo4 + threadIdx.x;
    for (; i + 3 * S < hi4; i += 4 * S) {
      float4 a[4], c[4], q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = a4[i + j * S];
        c[j] = c4[i + j * S];
        q[j] = p4[i + j * S];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sq(a[j].x, c[j].x, q[j].x);
        sq(a[j].y, c[j].y, q[j].y);
        sq(a[j].z, c[j].z, q[j].z);
        sq(a[j].w, c[j].w, q[j].w);
      }
    }
    for (; i < hi4; i += S) {
      const float4 a = a4[i], c = c4[i], q = p4[i];
      sq(a.x, c.x, q.x);
      sq(a.y, c.y, q.y);
      sq(a.z, c.z, q.z);
      sq(a.w, c.w, q.w);
    }
  } else {
    for (int64_t i = lo + threadIdx.x; i < hi; i += kRfLossThreads) sq(z0[base + i], z1[base + i], vp[base + i]);
  }
  acc = wave_sum_f64(acc);
  __shared__ double red[kRfLossThreads / kWave];
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int i = 0; i < kRfLossThreads / kWave; ++i) s += red[i];
    partials[(int64_t)b * parts + g] = s;
  }
}

// Stage 2: one block; per-sample sums in fixed order, then the total.
__global__ void __launch_bounds__(256) rf_loss_final_kernel(int batch, int64_t n, int parts,
                                                            const double* __restrict__ partials,
                                                            float* __restrict__ loss, float* __restrict__ loss_ps) {
  __shared__ double ps[256];
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    double s = 0.0;
    for (int g = 0; g < parts; ++g) s += partials[(int64_t)b * parts + g];
    if (b < 256) ps[b] = s;
    if (loss_ps) loss_ps[b] = (float)(s / (double)n);
  }
  __syncthreads();
  if (threadIdx.x == 0 && loss) {
    double s = 0.0;
    if (batch <= 256) {
      for (int b = 0; b < batch; ++b) s += ps[b];
    } else {
      for (int b = 0; b < batch; ++b)
        for (int g = 0; g < parts; ++g) s += partials[(int64_t)b * parts + g];
    }
    *loss = (float)(s / ((double)n * (double)batch));
  }
}

hipError_t launch_rf_loss(int batch, int64_t n, const float* z0, const float* z1, const float* vpred, float* loss,
                          float* loss_ps, double* partials, int parts, hipStream_t stream) {
  TimingScope ts(kKcRf, stream, (double)batch * n * 12.0);
  hipLaunchKernelGGL(rf_loss_partial_kernel, dim3(parts, batch), dim3(kRfLossThreads), 0, stream, n, z0, z1, vpred,
                     partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rf_loss_final_kernel, dim3(1), dim3(256), 0, stream, batch, n, parts, partials, loss, loss_ps);
  return hipGetLastError();
}

// ===========================================================================
// Timestep sinusoid ("Flux architecture deep dive", Conditioning; "Flux model
// API reference", TimeStepEmbedder): tau = time_factor * t,
// out = [cos(tau f_j) | sin(tau f_j)], f_j = max_period^(-j/half).  fp64.
// ===========================================================================
__global__ void timestep_embed_kernel(const float* __restrict__ t, int batch, int dim, double time_factor,
                                      double log_max_period, float* __restrict__ out) {
  const int half = dim / 2;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= batch * half) return;
  const int b = i / half, j = i % half;
  const double tau = time_factor * (double)t[b];
  const double f = exp(-log_max_period * (double)j / (double)half);
  double s, c;
  sincos(tau * f, &s, &c);
  out[(int64_t)b * dim + j] = (float)c;
  out[(int64_t)b * dim + half + j] = (float)s;
}

hipError_t launch_timestep_embed(const float* t, int batch, int dim, float time_factor, float max_period, float* out,
                                 hipStream_t stream) {
  const int n = batch * (dim / 2);
  TimingScope ts(kKcMisc, stream);
  hipLaunchKernelGGL(timestep_embed_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, t, batch, dim,
                     (double)time_factor, log((double)max_period), out);
  return hipGetLastError();
}

// ===========================================================================
// 3D RoPE table ("Flux architecture deep dive", 3D RoPE mathematics; "Flux
// model API reference", EmbedND).  Pair m of the head belongs to axis a with
// local index j; angle = p_a * theta^(-2j/d_a) in fp64; stored (cos, sin).
// ===========================================================================
__global__ void rope_table_kernel(const float* __restrict__ ids, int n_tok, int a0, int a1, int a2, double log_theta,
                                  float2* __restrict__ table) {
  const int pairs = (a0 + a1 + a2) / 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)n_tok * pairs) return;
  const int64_t tok = i / pairs;
  int m = (int)(i % pairs);
  int axis, d;
  if (m < a0 / 2) { axis = 0; d = a0; }
  else if (m < (a0 + a1) / 2) { axis = 1; d = a1; m -= a0 / 2; }
  else { axis = 2; d = a2; m -= (a0 + a1) / 2; }
  const double p = (double)ids[tok * 3 + axis];
  const double ang = p * exp(-log_theta * (2.0 * (double)m) / (double)d);
  double s, c;
  sincos(ang, &s, &c);
  table[i] = make_float2((float)c, (float)s);
}

hipError_t launch_rope_table(const float* ids, int batch, int seq, const int32_t axes[3], float theta, float* table,
                             hipStream_t stream) {
  const int n_tok = batch * seq;
  const int pairs = (axes[0] + axes[1] + axes[2]) / 2;
  const int64_t n = (int64_t)n_tok * pairs;
  TimingScope ts(kKcMisc, stream);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, ids, n_tok, axes[0],
                     axes[1], axes[2], log((double)theta), reinterpret_cast<float2*>(table));
  return hipGetLastError();
}

// ===========================================================================
// patchify ("Flux architecture deep dive", Implementation details / Memory
// layout): [B, C, H*W] float -> [B, H*W, C] operand type.
// ===========================================================================
template <typename T>
__global__ void patchify_kernel(const float* __restrict__ z, int channels, int hw, T* __restrict__ out) {
  const int b = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // over hw * C, channel fastest
  if (i >= (int64_t)hw * channels) return;
  const int c = (int)(i % channels);
  const int64_t l = i / channels;
  out[(int64_t)b * hw * channels + i] = from_f32<T>(z[((int64_t)b * channels + c) * hw + l]);
}

hipError_t launch_patchify(const float* z, int batch, int channels, int hw, void* out, int dtype,
                           hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div((int64_t)hw * channels, 256), batch);
  TimingScope ts(kKcMisc, stream);
  if (dtype == kBF16)
    hipLaunchKernelGGL(patchify_kernel<bf16_t>, grid, dim3(256), 0, stream, z, channels, hw, (bf16_t*)out);
  else
    hipLaunchKernelGGL(patchify_kernel<float>, grid, dim3(256), 0, stream, z, channels, hw, (float*)out);
  return hipGetLastError();
}

// Text tokens that enter the joint sequence at the hidden width (no context
// projection): sample b of src ([batch, rows, width] contiguous, element T)
// into fp32 rows at dst + b * dst_bstride.  Four elements per thread (width
// is a multiple of 4).
template <typename T>
__global__ void __launch_bounds__(256) rows_to_f32_kernel(const T* __restrict__ src, int64_t n, float* __restrict__ dst,
                                                          int64_t dst_bstride) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;   // element of the sample
  if (i >= n) return;
  const T* s = src + blockIdx.y * n + i;
  float4 v;
  if constexpr (sizeof(T) == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(s);
    v = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                    __uint_as_float(u.y & 0xffff0000u));
  } else {
    v = *reinterpret_cast<const float4*>(s);
  }
  *reinterpret_cast<float4*>(dst + blockIdx.y * dst_bstride + i) = v;
}

hipError_t launch_rows_to_f32(const void* src, int batch, int rows, int width, int dtype, float* dst,
                              int64_t dst_bstride, hipStream_t stream) {
  const int64_t n = (int64_t)rows * width;
  const dim3 grid((unsigned)ceil_div(n / 4, 256), batch);
  TimingScope ts(kKcMisc, stream);
  if (dtype == kBF16)
    hipLaunchKernelGGL(rows_to_f32_kernel<bf16_t>, grid, dim3(256), 0, stream, static_cast<const bf16_t*>(src), n,
                       dst, dst_bstride);
  else
    hipLaunchKernelGGL(rows_to_f32_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(src), n, dst,
                       dst_bstride);
  return hipGetLastError();
}

// ===========================================================================
// LayerNorm (no affine, biased variance) + adaLN modulate ("Flux architecture
// deep dive", Implementation details / Adaptive layer normalization):
// h = (x - mean) / sqrt(var + eps) * (1 + scale[b]) + shift[b].
// One wave per token row, the row in registers (two-pass variance).  A block
// of 4 waves owns a contiguous range of rows (at most kLnBlocks blocks, two
// per CU); wave w takes rows w, w+4, ... of the range and loads its next row
// while it normalizes the current one.  (1 + scale) and shift of the sample
// of the block's first row are staged in LDS once (a row of another sample
// reads them from global memory, where L2 serves them).
// E4M3 output: the amax of each segment is reduced over the block and raises
// the segment's record with one atomic per block.  Atomics on one address are
// serialized by the memory system (about 11 ns each, measured), so one per
// row would cost more than the whole kernel.
// ===========================================================================
constexpr int kLnMaxVec = 16;   // float4 per lane: D <= 64 * 4 * 16 = 4096
constexpr int kLnBlocks = 512;  // grid cap

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  uint2 v;
  v.x = pack_bf16x2(a, b);
  v.y = pack_bf16x2(c, d);
  *reinterpret_cast<uint2*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<_Float16>(_Float16* p, float a, float b, float c, float d) {
  uint2 v;
  v.x = pack_f16x2(a, b);
  v.y = pack_f16x2(c, d);
  *reinterpret_cast<uint2*>(p) = v;
}

template <typename T, int NV>
__global__ void __launch_bounds__(256) ln_mod_kernel(LnArgs a, int64_t rows_per_block) {
  __shared__ float4 msc[NV * 64], msh[NV * 64];   // (1 + scale), shift of the block's first sample
  __shared__ uint32_t red[2][4];                  // per-wave amax of each segment (E4M3 output)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t total = a.s[0].rows + (a.count > 1 ? (int64_t)a.s[1].rows : 0);
  const int64_t b0 = (int64_t)blockIdx.x * 4;     // one row per wave
  if (b0 >= total) return;   // block-uniform
  const int D = a.dim;
  // global rows run over segment 0 then segment 1 (g < total)
  auto locate = [&](int64_t g, int& si, int64_t& r) {
    si = g >= a.s[0].rows ? 1 : 0;
    r = si ? g - a.s[0].rows : g;
  };
  // 1. the wave's row, all NV loads in flight before anything else
  const int64_t g = b0 + wave;
  const bool has_row = g < total;   // wave-uniform
  int si = 0;
  int64_t r = 0;
  float4 v[NV];
  if (has_row) {
    locate(g, si, r);
    const LnSeg& sg = a.s[si];
    const int64_t bb = r / sg.xmap.seg, ll = r % sg.xmap.seg;
    const float* x = sg.x + bb * sg.xmap.bstride + ll * sg.xmap.ld;
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = reinterpret_cast<const float4*>(x)[lane + 64 * i];
  }
  // 2. (1 + scale) and shift of the block's first row's sample, staged while
  // the rows are in flight
  int bsi;
  int64_t brow;
  locate(b0, bsi, brow);
  const int64_t bsam = brow / a.s[bsi].xmap.seg;
  {
    const float* scp = a.s[bsi].scale + bsam * a.s[bsi].mod_bstride;
    const float* shp = a.s[bsi].shift + bsam * a.s[bsi].mod_bstride;
    for (int i = threadIdx.x; i < NV * 64; i += 256) {
      const float4 t = reinterpret_cast<const float4*>(scp)[i];
      msc[i] = make_float4(1.f + t.x, 1.f + t.y, 1.f + t.z, 1.f + t.w);
      msh[i] = reinterpret_cast<const float4*>(shp)[i];
    }
  }
  __syncthreads();
  uint32_t mx = 0;
  if (has_row) {
    const LnSeg& sg = a.s[si];
    const int64_t bb = r / sg.xmap.seg, ll = r % sg.xmap.seg;
    const bool staged = si == bsi && bb == bsam;   // wave-uniform
    const float4* gsc = reinterpret_cast<const float4*>(sg.scale + bb * sg.mod_bstride);
    const float4* gsh = reinterpret_cast<const float4*>(sg.shift + bb * sg.mod_bstride);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    const float mean = wave_sum(sum) / (float)D;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float dx = v[i].x - mean, dy = v[i].y - mean, dz = v[i].z - mean, dw = v[i].w - mean;
      sq += (dx * dx + dy * dy) + (dz * dz + dw * dw);
    }
    const float var = wave_sum(sq) / (float)D;
    const float rstd = 1.0f / sqrtf(var + a.eps);
    T* out = reinterpret_cast<T*>(sg.out) + bb * sg.omap.bstride + ll * sg.omap.ld;
    float qs = 1.0f;   // E4M3 output: the record's delayed scale
    if constexpr (sizeof(T) == 1) qs = fp8_scale(sg.q);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = (lane + 64 * i) * 4;
      float4 s1, h4;
      if (staged) {
        s1 = msc[lane + 64 * i];
        h4 = msh[lane + 64 * i];
      } else {
        const float4 t = gsc[lane + 64 * i];
        s1 = make_float4(1.f + t.x, 1.f + t.y, 1.f + t.z, 1.f + t.w);
        h4 = gsh[lane + 64 * i];
      }
      const float y0 = (v[i].x - mean) * rstd * s1.x + h4.x;
      const float y1 = (v[i].y - mean) * rstd * s1.y + h4.y;
      const float y2 = (v[i].z - mean) * rstd * s1.z + h4.z;
      const float y3 = (v[i].w - mean) * rstd * s1.w + h4.w;
      if constexpr (sizeof(T) == 1) {
        // E4M3 output with the record's delayed scale; amax of the unscaled values
        mx = max(mx, max(max(abs_bits(y0), abs_bits(y1)), max(abs_bits(y2), abs_bits(y3))));
        *reinterpret_cast<uint32_t*>(out + c) = f32x4_to_e4m3(y0 * qs, y1 * qs, y2 * qs, y3 * qs);
      } else {
        store4<T>(out + c, y0, y1, y2, y3);
      }
    }
  }
  if constexpr (sizeof(T) == 1) {
    const uint32_t m = wave_max_u32(mx);
    if (lane == 0) {
      red[0][wave] = has_row && si == 0 ? m : 0u;
      red[1][wave] = has_row && si == 1 ? m : 0u;
    }
    __syncthreads();
    if (threadIdx.x < 2 && threadIdx.x < a.count) {
      const uint32_t mm = max(max(red[threadIdx.x][0], red[threadIdx.x][1]), max(red[threadIdx.x][2], red[threadIdx.x][3]));
      if (mm) fp8_amax_raise(a.s[threadIdx.x].q, __uint_as_float(mm));
    }
  }
}

// E4M3 output: the kernel above keeps one amax atomic per block of 4 rows;
// this one walks a contiguous row range per block (at most kLnBlocks blocks),
// so the amax atomics stay few.
template <typename T, int NV>
__global__ void __launch_bounds__(256) ln_mod_rows_kernel(LnArgs a, int64_t rows_per_block) {
  __shared__ float4 msc[NV * 64], msh[NV * 64];   // (1 + scale), shift of the block's first sample
  __shared__ uint32_t red[2][4];                  // per-wave amax of each segment (E4M3 output)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t total = a.s[0].rows + (a.count > 1 ? (int64_t)a.s[1].rows : 0);
  const int64_t b0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t b1 = b0 + rows_per_block < total ? b0 + rows_per_block : total;
  if (b0 >= total) return;   // block-uniform
  const int D = a.dim;
  // global rows run over segment 0 then segment 1 (g < total)
  auto locate = [&](int64_t g, int& si, int64_t& r) {
    si = g >= a.s[0].rows ? 1 : 0;
    r = si ? g - a.s[0].rows : g;
  };
  int bsi;
  int64_t brow;
  locate(b0, bsi, brow);
  const int64_t bsam = brow / a.s[bsi].xmap.seg;
  {
    const float* scp = a.s[bsi].scale + bsam * a.s[bsi].mod_bstride;
    const float* shp = a.s[bsi].shift + bsam * a.s[bsi].mod_bstride;
    for (int i = threadIdx.x; i < NV * 64; i += 256) {
      const float4 t = reinterpret_cast<const float4*>(scp)[i];
      msc[i] = make_float4(1.f + t.x, 1.f + t.y, 1.f + t.z, 1.f + t.w);
      msh[i] = reinterpret_cast<const float4*>(shp)[i];
    }
  }
  __syncthreads();

  auto load_row = [&](int64_t g, float4* dst) {
    int sidx;
    int64_t row;
    locate(g, sidx, row);
    const LnSeg& sg = a.s[sidx];
    const int64_t bb = row / sg.xmap.seg, ll = row % sg.xmap.seg;
    const float* x = sg.x + bb * sg.xmap.bstride + ll * sg.xmap.ld;
#pragma unroll
    for (int i = 0; i < NV; ++i) dst[i] = reinterpret_cast<const float4*>(x)[lane + 64 * i];
  };
  uint32_t mxs[2] = {0u, 0u};
  float qsc[2] = {1.0f, 1.0f};   // E4M3 output: delayed scales, read once (stores may alias the records)
  if constexpr (sizeof(T) == 1) {
    qsc[0] = fp8_scale(a.s[0].q);
    if (a.count > 1) qsc[1] = fp8_scale(a.s[1].q);
  }
  float4 v[NV], vn[NV];
  int64_t g = b0 + wave;
  if (g < b1) load_row(g, v);
#pragma unroll 1
  for (; g < b1; g += 4) {
    const bool has_next = g + 4 < b1;   // wave-uniform
    if (has_next) load_row(g + 4, vn);
    int si;
    int64_t r;
    locate(g, si, r);
    const LnSeg& sg = a.s[si];
    const int64_t bb = r / sg.xmap.seg, ll = r % sg.xmap.seg;
    const bool staged = si == bsi && bb == bsam;   // wave-uniform
    const float4* gsc = reinterpret_cast<const float4*>(sg.scale + bb * sg.mod_bstride);
    const float4* gsh = reinterpret_cast<const float4*>(sg.shift + bb * sg.mod_bstride);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    const float mean = wave_sum(sum) / (float)D;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float dx = v[i].x - mean, dy = v[i].y - mean, dz = v[i].z - mean, dw = v[i].w - mean;
      sq += (dx * dx + dy * dy) + (dz * dz + dw * dw);
    }
    const float var = wave_sum(sq) / (float)D;
    const float rstd = 1.0f / sqrtf(var + a.eps);
    T* out = reinterpret_cast<T*>(sg.out) + bb * sg.omap.bstride + ll * sg.omap.ld;
    uint32_t mx = 0;
    const float qs = qsc[si];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = (lane + 64 * i) * 4;
      float4 s1, h4;
      if (staged) {
        s1 = msc[lane + 64 * i];
        h4 = msh[lane + 64 * i];
      } else {
        const float4 t = gsc[lane + 64 * i];
        s1 = make_float4(1.f + t.x, 1.f + t.y, 1.f + t.z, 1.f + t.w);
        h4 = gsh[lane + 64 * i];
      }
      const float y0 = (v[i].x - mean) * rstd * s1.x + h4.x;
      const float y1 = (v[i].y - mean) * rstd * s1.y + h4.y;
      const float y2 = (v[i].z - mean) * rstd * s1.z + h4.z;
      const float y3 = (v[i].w - mean) * rstd * s1.w + h4.w;
      if constexpr (sizeof(T) == 1) {
        // E4M3 output with the record's delayed scale; amax of the unscaled values
        mx = max(mx, max(max(abs_bits(y0), abs_bits(y1)), max(abs_bits(y2), abs_bits(y3))));
        *reinterpret_cast<uint32_t*>(out + c) = f32x4_to_e4m3(y0 * qs, y1 * qs, y2 * qs, y3 * qs);
      } else {
        store4<T>(out + c, y0, y1, y2, y3);
      }
    }
    if constexpr (sizeof(T) == 1) {
      if (si) mxs[1] = max(mxs[1], mx);
      else mxs[0] = max(mxs[0], mx);
    }
    if (has_next) {
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i] = vn[i];
    }
  }
  if constexpr (sizeof(T) == 1) {
    const uint32_t m0 = wave_max_u32(mxs[0]), m1 = wave_max_u32(mxs[1]);
    if (lane == 0) {
      red[0][wave] = m0;
      red[1][wave] = m1;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
      const uint32_t m = max(max(red[threadIdx.x][0], red[threadIdx.x][1]), max(red[threadIdx.x][2], red[threadIdx.x][3]));
      if (m) fp8_amax_raise(a.s[threadIdx.x].q, __uint_as_float(m));
    }
  }
}

template <typename T>
static void launch_ln_mod_t(const LnArgs& a, dim3 grid, int64_t rpb, hipStream_t stream) {
  // D is a multiple of 256, at most 4096 (checked by the API): NV float4 per lane
#define FLUX_LN_CASE(nv)                                                                             \
  case nv:                                                                                           \
    if constexpr (sizeof(T) == 1)                                                                    \
      hipLaunchKernelGGL((ln_mod_rows_kernel<T, nv>), grid, dim3(256), 0, stream, a, rpb);           \
    else                                                                                             \
      hipLaunchKernelGGL((ln_mod_kernel<T, nv>), grid, dim3(256), 0, stream, a, rpb);                \
    break;
  switch (a.dim / 256) {
    FLUX_LN_CASE(1) FLUX_LN_CASE(2) FLUX_LN_CASE(3) FLUX_LN_CASE(4) FLUX_LN_CASE(5) FLUX_LN_CASE(6)
    FLUX_LN_CASE(7) FLUX_LN_CASE(8) FLUX_LN_CASE(9) FLUX_LN_CASE(10) FLUX_LN_CASE(11) FLUX_LN_CASE(12)
    FLUX_LN_CASE(13) FLUX_LN_CASE(14) FLUX_LN_CASE(15) default: FLUX_LN_CASE(16)
  }
#undef FLUX_LN_CASE
}

hipError_t launch_ln_mod(const LnArgs& a, int dtype, hipStream_t stream) {  // dtype: output element type
  if (a.dim % 256 != 0 || a.dim < 256 || a.dim > 256 * kLnMaxVec) return hipErrorInvalidValue;
  const int64_t rows = a.s[0].rows + (a.count > 1 ? a.s[1].rows : 0);
  if (rows <= 0) return hipSuccess;
  // 16/32-bit output: one row per wave, every row's loads in flight at once;
  // E4M3 output: contiguous row ranges, at most kLnBlocks blocks
  int64_t blocks = ceil_div(rows, 4);
  if (dtype == kFP8 && blocks > kLnBlocks) blocks = kLnBlocks;
  const int64_t rpb = ceil_div(rows, blocks);
  const dim3 grid((unsigned)ceil_div(rows, rpb));
  TimingScope ts(kKcLnMod, stream, (double)rows * a.dim * (4.0 + (dtype == kF32 ? 4.0 : dtype == kFP8 ? 1.0 : 2.0)));
  if (dtype == kFP8)
    launch_ln_mod_t<uint8_t>(a, grid, rpb, stream);
  else if (dtype == kBF16)
    launch_ln_mod_t<bf16_t>(a, grid, rpb, stream);
  else if (dtype == kF16)
    launch_ln_mod_t<_Float16>(a, grid, rpb, stream);
  else
    launch_ln_mod_t<float>(a, grid, rpb, stream);
  return hipGetLastError();
}

// ===========================================================================
// Modulation GEMV (M = batch <= 4 per launch): y[b, n] (+)= sum_k W[n, k]
// act(x[b, k]) + bias[n] ("Flux model API reference", AdaLN: Linear over
// SiLU(vec); also the timestep / pooled-vector embedders).  Weight-bandwidth
// bound: each wave streams kGemvRows whole W rows at a time with 16-byte
// loads, kGemvLoads per lane and row in flight; act(x) is staged in LDS once
// per block and each LDS read of it serves all rows of the group.
// ===========================================================================
constexpr int kGemvMaxB = 4;
constexpr int kGemvLoads = 4;   // 16-byte loads per lane and row in flight
constexpr int kGemvRows = 4;    // W rows a wave reduces at once (act(x) read from LDS once for all)

template <typename T>
struct Vec16;  // 16 bytes of operand elements
template <>
struct Vec16<bf16_t> { static constexpr int n = 8; };
template <>
struct Vec16<float> { static constexpr int n = 4; };

template <typename T>
__device__ __forceinline__ void unpack16(const u32x4_t& r, float* w);
template <>
__device__ __forceinline__ void unpack16<bf16_t>(const u32x4_t& r, float* w) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[2 * i] = __uint_as_float(r[i] << 16);
    w[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void unpack16<float>(const u32x4_t& r, float* w) {
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = __uint_as_float(r[i]);
}

template <typename T>
__global__ void __launch_bounds__(256) gemv_kernel(GemvBatch a) {
  extern __shared__ float xs[];   // [batch][K]
  const GemvProblem& p = a.p[blockIdx.y];
  const int K = p.K, B = a.batch;
  if ((K & 3) == 0 && (p.x_bstride & 3) == 0 && (reinterpret_cast<uintptr_t>(p.x) & 15) == 0) {
    // float4 staging, all of a thread's loads in flight before the first SiLU
    constexpr int SU = 4;
    const int K4 = K >> 2, n4 = B * K4;
    for (int i0 = threadIdx.x; i0 < n4; i0 += 256 * SU) {
      float4 v[SU];
#pragma unroll
      for (int j = 0; j < SU; ++j) {
        const int i = i0 + 256 * j;
        if (i < n4) v[j] = reinterpret_cast<const float4*>(p.x + (int64_t)(i / K4) * p.x_bstride)[i % K4];
      }
#pragma unroll
      for (int j = 0; j < SU; ++j) {
        const int i = i0 + 256 * j;
        if (i < n4) {
          if (p.act_silu) v[j] = make_float4(silu_f(v[j].x), silu_f(v[j].y), silu_f(v[j].z), silu_f(v[j].w));
          reinterpret_cast<float4*>(xs)[i] = v[j];
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < B * K; i += blockDim.x) {
      const int b = i / K, k = i % K;
      const float v = p.x[(int64_t)b * p.x_bstride + k];
      xs[i] = p.act_silu ? silu_f(v) : v;
    }
  }
  __syncthreads();
  constexpr int E = Vec16<T>::n;
  constexpr int U = kGemvLoads;
  constexpr int R = kGemvRows;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const T* W = reinterpret_cast<const T*>(p.W);
  const T* bias = reinterpret_cast<const T*>(p.bias);
  for (int n0 = (blockIdx.x * 4 + wave) * R; n0 < p.N; n0 += gridDim.x * 4 * R) {
    float acc[R][kGemvMaxB];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < kGemvMaxB; ++b) acc[r][b] = 0.f;
    for (int kc = 0; kc < K; kc += 64 * E * U) {
      // R x U 16-byte loads issued before the first use
      u32x4_t raw[R][U];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int k0 = kc + (u * 64 + lane) * E;
          if (k0 < K && n0 + r < p.N) raw[r][u] = *reinterpret_cast<const u32x4_t*>(W + (int64_t)(n0 + r) * K + k0);
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k0 = kc + (u * 64 + lane) * E;
        if (k0 < K) {
          // act(x) for these E columns, read from LDS once for all R rows
          float xv[kGemvMaxB][E];
#pragma unroll
          for (int b = 0; b < kGemvMaxB; ++b)
#pragma unroll
            for (int e = 0; e < E; ++e) xv[b][e] = b < B ? xs[b * K + k0 + e] : 0.f;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            if (n0 + r < p.N) {
              float w[E];
              unpack16<T>(raw[r][u], w);
#pragma unroll
              for (int b = 0; b < kGemvMaxB; ++b) {
                if (b < B) {
#pragma unroll
                  for (int e = 0; e < E; ++e) acc[r][b] += w[e] * xv[b][e];
                }
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = n0 + r;
#pragma unroll
      for (int b = 0; b < kGemvMaxB; ++b) {
        if (b < B && n < p.N) {
          const float s = wave_sum(acc[r][b]);
          if (lane == 0) {
            float v = s + (bias ? load_f32<T>(bias + n) : 0.f);
            float* y = p.y + (int64_t)b * p.y_bstride + n;
            *y = p.accumulate ? *y + v : v;
          }
        }
      }
    }
  }
}

hipError_t launch_gemv(const GemvBatch& a, int dtype, hipStream_t stream) {
  int maxn = 0, maxk = 0;
  for (int i = 0; i < a.count; ++i) {
    maxn = a.p[i].N > maxn ? a.p[i].N : maxn;
    maxk = a.p[i].K > maxk ? a.p[i].K : maxk;
  }
  // about three blocks per CU over all problems: each wave keeps kGemvLoads
  // 16-byte loads per lane in flight
  int gx = (int)ceil_div(maxn, 4 * kGemvRows);
  const int cap = 768 / (a.count > 0 ? a.count : 1);
  if (gx > cap) gx = cap;
  const size_t lds = (size_t)a.batch * maxk * sizeof(float);
  const dim3 grid(gx, a.count);
  double wbytes = 0.0;
  for (int i = 0; i < a.count; ++i) wbytes += (double)a.p[i].N * a.p[i].K * (dtype == kBF16 ? 2.0 : 4.0);
  TimingScope ts(kKcGemv, stream, wbytes);
  if (dtype == kBF16)
    hipLaunchKernelGGL(gemv_kernel<bf16_t>, grid, dim3(256), lds, stream, a);
  else
    hipLaunchKernelGGL(gemv_kernel<float>, grid, dim3(256), lds, stream, a);
  return hipGetLastError();
}

// ===========================================================================
// q/k preparation for attention: per token and head, RMSNorm over head_dim
// with the stream's scale ("Flux model API reference", RMSNorm), then the 3D
// RoPE rotation of interleaved pairs ("Flux architecture deep dive", 3D RoPE
// mathematics), written head-major [B, H, seq_pad, Dh]; v is written
// transposed [B, H, Dh, seq_pad] so that attention reads it K-contiguous.
// Rows seq .. seq_pad-1 are written as zeros.
// ===========================================================================
template <typename T>
__device__ __forceinline__ void load_pair(const T* p, float& u, float& w);
template <>
__device__ __forceinline__ void load_pair<float>(const float* p, float& u, float& w) {
  const float2 v = *reinterpret_cast<const float2*>(p);
  u = v.x;
  w = v.y;
}
template <>
__device__ __forceinline__ void load_pair<bf16_t>(const bf16_t* p, float& u, float& w) {
  const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
  u = __uint_as_float(v << 16);
  w = __uint_as_float(v & 0xffff0000u);
}
template <typename T>
__device__ __forceinline__ void store_pair(T* p, float u, float w);
template <>
__device__ __forceinline__ void store_pair<float>(float* p, float u, float w) {
  *reinterpret_cast<float2*>(p) = make_float2(u, w);
}
template <>
__device__ __forceinline__ void store_pair<bf16_t>(bf16_t* p, float u, float w) {
  *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(u, w);
}

// One block per (64 tokens, head, batch): q and k rows of the head get
// RMSNorm + RoPE and go to their head-major rows; v goes through LDS and out
// transposed.  Every global access is 16 bytes per lane: a chunk holds E =
// 16 / sizeof(T) consecutive head dims, and the DH / E lanes of one
// (token, head) row form an aligned group of the wave, so the RMSNorm sum is
// a shuffle reduction within the group.  A lane's chunk position inside the
// head is the same for every row it handles, so its RoPE pairs and norm
// scales are loaded once per row from the per-token table and once per block.
template <typename T, int DH>
__global__ void __launch_bounds__(256) prep_kernel(PrepArgs a) {
  constexpr int E = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int G = DH / E;                  // lanes per (token, head) row
  constexpr int TOK = 64;                    // tokens per block
  constexpr int PER = TOK * G / 256;         // chunks per thread per matrix
  static_assert(PER >= 1 && (TOK * G) % 256 == 0, "tile shape");
  typedef uint32_t chunk_t __attribute__((ext_vector_type(4)));
  __shared__ T tile[TOK][DH + E];            // v tile, rows padded by one chunk
  const int j0 = blockIdx.x * TOK, h = blockIdx.y, b = blockIdx.z;
  const int H = a.heads;
  const int tid = threadIdx.x;
  const int g = tid % G;                     // chunk position inside the head
  const int d0 = g * E;
  const int64_t head_row0 = ((int64_t)b * H + h) * a.seq_pad;
  // q and k
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const T* src = reinterpret_cast<const T*>(which == 0 ? a.src_q : a.src_k) + (int64_t)b * a.src_bstride + h * DH;
    T* dst = reinterpret_cast<T*>(which == 0 ? a.qh : a.kh);
    chunk_t raw[PER];
    int jj[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int r = (tid + 256 * i) / G;     // token within the tile
      jj[i] = j0 + r;
      if (jj[i] < a.seq) raw[i] = *reinterpret_cast<const chunk_t*>(src + (int64_t)jj[i] * a.src_ld + d0);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = jj[i];
      float x[E];
      if (j < a.seq) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < E / 2; ++e) {
            x[2 * e] = __uint_as_float(raw[i][e] << 16);
            x[2 * e + 1] = __uint_as_float(raw[i][e] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) x[e] = __uint_as_float(raw[i][e]);
        }
        const bool txt = j >= a.l_img;
        const float* gm = which == 0 ? (txt ? a.gq_txt : a.gq_img) : (txt ? a.gk_txt : a.gk_img);
        if (gm) {
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) ss += x[e] * x[e];
          const float ms = wave_sum<G>(ss) / (float)DH;
          const float rs = 1.0f / sqrtf(ms + a.eps);
#pragma unroll
          for (int e = 0; e < E; ++e) x[e] = x[e] * rs * gm[d0 + e];
        }
        if (a.rope) {
          const float2* cs = reinterpret_cast<const float2*>(a.rope) + ((int64_t)b * a.seq + j) * (DH / 2) + d0 / 2;
#pragma unroll
          for (int e = 0; e < E / 2; ++e) {
            const float2 t = cs[e];
            const float u = x[2 * e], w = x[2 * e + 1];
            x[2 * e] = u * t.x - w * t.y;
            x[2 * e + 1] = u * t.y + w * t.x;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = 0.f;
      }
      chunk_t o;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < E / 2; ++e) o[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = __float_as_uint(x[e]);
      }
      *reinterpret_cast<chunk_t*>(dst + (head_row0 + j) * DH + d0) = o;
    }
  }
  // v: rows into LDS, columns out
  {
    const T* src = reinterpret_cast<const T*>(a.src_v) + (int64_t)b * a.src_bstride + h * DH;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int r = (tid + 256 * i) / G, j = j0 + r;
      chunk_t c = {0u, 0u, 0u, 0u};
      if (j < a.seq) c = *reinterpret_cast<const chunk_t*>(src + (int64_t)j * a.src_ld + d0);
      *reinterpret_cast<chunk_t*>(&tile[r][d0]) = c;
    }
  }
  __syncthreads();
  {
    // output row d of vt holds the tile's 64 tokens: TOK / E chunks per row
    constexpr int CPR = TOK / E;
    T* dst = reinterpret_cast<T*>(a.vt) + ((int64_t)b * H + h) * DH * a.seq_pad + j0;
#pragma unroll
    for (int i = 0; i < DH * CPR / 256; ++i) {
      const int c = tid + 256 * i, d = c / CPR, r0 = (c % CPR) * E;
      T vals[E];
#pragma unroll
      for (int e = 0; e < E; ++e) vals[e] = tile[r0 + e][d];
      *reinterpret_cast<chunk_t*>(dst + (int64_t)d * a.seq_pad + r0) = __builtin_bit_cast(chunk_t, vals);
    }
  }
}

template <typename T>
static hipError_t launch_prep_t(const PrepArgs& a, hipStream_t stream) {
  const dim3 grid(a.seq_pad / 64, a.heads, a.batch);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((prep_kernel<T, 128>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((prep_kernel<T, 64>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs& a, int dtype, hipStream_t stream) {
  const double es = dtype == kBF16 ? 2.0 : 4.0, D = (double)a.heads * a.head_dim;
  TimingScope ts(kKcPrep, stream, es * a.batch * D * (3.0 * a.seq + 3.0 * a.seq_pad));
  return dtype == kBF16 ? launch_prep_t<bf16_t>(a, stream) : launch_prep_t<float>(a, stream);
}

// ===========================================================================
// One-time bf16 -> fp16 conversion of static weights.  Rounds toward zero,
// the same rule as the conversion inside the GEMM (bf16x8_to_f16x8): exact in
// fp16's normal range, at most 2^-24 lost below 2^-14, magnitudes above 65504
// saturate to +-65504.
// ===========================================================================
__global__ void __launch_bounds__(256) convert_bf16_f16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                               int64_t n8, const bf16_t* __restrict__ src_tail,
                                                               _Float16* __restrict__ dst_tail, int tail) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint4 v = src[i];
    const u32x4_t o = bf16x8_to_f16x8(u32x4_t{v.x, v.y, v.z, v.w});
    dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < tail)
    dst_tail[threadIdx.x] = __builtin_amdgcn_cvt_pkrtz(bf16_to_f32(src_tail[threadIdx.x]), 0.0f)[0];
}

hipError_t launch_convert_bf16_f16(const void* src, void* dst, int64_t n, hipStream_t stream) {
  const int64_t n8 = n / 8;
  const int tail = (int)(n - n8 * 8);
  int64_t blocks = ceil_div(n8 > 0 ? n8 : 1, 256);
  if (blocks > 4096) blocks = 4096;
  TimingScope ts(kKcMisc, stream, 4.0 * (double)n);
  hipLaunchKernelGGL(convert_bf16_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), n8,
                     reinterpret_cast<const bf16_t*>(src) + n8 * 8, reinterpret_cast<_Float16*>(dst) + n8 * 8, tail);
  return hipGetLastError();
}

// ===========================================================================
// FP8 (E4M3) delayed scaling ("FP8 training for Flux models", Configuration).
// ===========================================================================
// MXFP8 quantization (the "mxfp8" recipe of "FP8 training for Flux models",
// Configuration; block-scaled E4M3 in the OCP MX format): every 32 values of
// a row share the scale 2^X, X = floor(log2 max|v|) - 8 clamped to [-127, 127]
// (-127 for an all-zero block, NaN byte 0xFF and unscaled elements for a
// block holding a non-finite value); the elements are E4M3 of v * 2^-X, a
// product that is exact.  Four lanes own a block, 8 values each; the block
// maximum is two lane exchanges.  Scale bytes go to the GEMM layout of
// mx_scale_bytes; rows past `rows` up to the 256-row padding get zero codes
// and the all-zero scale.
// ===========================================================================
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* v) {
  const u32x4_t r = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(r[i] << 16);
    v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename T>
__global__ void __launch_bounds__(256) mx_quantize_kernel(const T* __restrict__ src, int rows, int k, int rows_pad,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int per_row = k / 8;   // a multiple of 8: groups of 4 lanes never straddle rows
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (int64_t)rows_pad * per_row) return;   // whole groups of 4 lanes leave together
  const int row = (int)(g / per_row), c8 = (int)(g % per_row);
  float v[8];
  if (row < rows) {
    load8<T>(src + (int64_t)row * k + c8 * 8, v);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, abs_bits(v[i]));   // NaN patterns sort above infinity
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2));
  uint32_t sbyte;
  float inv = 1.0f;
  if (m >= 0x7f800000u) {
    sbyte = 0xFFu;   // non-finite block: NaN scale, elements unscaled
  } else {
    // floor(log2 m) for a normal m; any subnormal m gives X = -127 anyway
    const int e = m >= 0x00800000u ? (int)(m >> 23) - 127 : -127;
    int X = m == 0u ? -127 : e - 8;
    X = X < -127 ? -127 : X;
    sbyte = (uint32_t)(X + 127);
    inv = __uint_as_float((uint32_t)(127 - X) << 23);   // 2^-X, a normal float for X in [-127, 119]
  }
  if (row < rows) {
    uint2 o;
    o.x = f32x4_to_e4m3(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    o.y = f32x4_to_e4m3(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    *reinterpret_cast<uint2*>(codes + (int64_t)row * k + c8 * 8) = o;
  }
  if ((c8 & 3) == 0) {
    const int kb = c8 >> 2, kt = kb >> 1, h = kb & 1;
    const int64_t idx = (((int64_t)(row >> 7) * (k >> 6) + kt) * 2 + h) * 128 + (row & 31) * 4 + ((row >> 5) & 3);
    scales[idx] = (uint8_t)sbyte;
  }
}

hipError_t launch_mx_quantize(const void* src, int src_dtype, int rows, int k, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  const int rows_pad = ((rows + 255) / 256) * 256;
  const int64_t threads = (int64_t)rows_pad * (k / 8);
  const dim3 grid((unsigned)ceil_div(threads, 256));
  TimingScope ts(kKcMxQuant, stream, (double)rows * k * ((src_dtype == kBF16 ? 2.0 : 4.0) + 1.0 + 1.0 / 32));
  if (src_dtype == kBF16)
    hipLaunchKernelGGL(mx_quantize_kernel<bf16_t>, grid, dim3(256), 0, stream, static_cast<const bf16_t*>(src), rows,
                       k, rows_pad, codes, scales);
  else
    hipLaunchKernelGGL(mx_quantize_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(src), rows,
                       k, rows_pad, codes, scales);
  return hipGetLastError();
}

// MXFP4 quantization (OCP MX v1.0 with E2M1 elements, the fp4 sibling of
// the recipe above): the block exponent is X = floor(log2 max|v|) - 2, 2 being
// the exponent of E2M1's largest value 6 = 1.5 * 2^2, clamped to [-127, 127]
// (-127 for an all-zero block; NaN byte 0xFF and unscaled elements for a block
// holding a non-finite value).  v * 2^-X is exact and lies below 8; it rounds
// to the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even code (the
// one whose mantissa bit is 0), and saturates at 6.
// ===========================================================================
// E2M1 code of a finite float: the magnitude code counts the grid midpoints
// below |v|.  A midpoint between code 2c and 2c + 1 goes down (to the even
// code), one between 2c + 1 and 2c + 2 goes up; bit 3 is the sign.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
                     (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

template <typename T>
__global__ void __launch_bounds__(256) mxfp4_quantize_kernel(const T* __restrict__ src, int rows, int k, int rows_pad,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int per_row = k / 8;   // k is a multiple of 128: groups of 4 lanes never straddle rows
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (int64_t)rows_pad * per_row) return;   // whole groups of 4 lanes leave together
  const int row = (int)(g / per_row), c8 = (int)(g % per_row);
  float v[8];
  if (row < rows) {
    load8<T>(src + (int64_t)row * k + c8 * 8, v);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, abs_bits(v[i]));   // NaN patterns sort above infinity
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2));
  uint32_t sbyte;
  float inv = 1.0f;
  if (m >= 0x7f800000u) {
    sbyte = 0xFFu;   // non-finite block: NaN scale, elements unscaled
  } else {
    // floor(log2 m) for a normal m; any subnormal m gives X = -127 anyway
    const int e = m >= 0x00800000u ? (int)(m >> 23) - 127 : -127;
    int X = m == 0u ? -127 : e - 2;
    X = X < -127 ? -127 : X;
    sbyte = (uint32_t)(X + 127);
    inv = __uint_as_float((uint32_t)(127 - X) << 23);   // 2^-X, a normal float for X in [-127, 125]
  }
  if (row < rows) {
    uint32_t o = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) o |= e2m1_code(v[i] * inv) << (4 * i);
    *reinterpret_cast<uint32_t*>(codes + (int64_t)row * (k / 2) + c8 * 4) = o;
  }
  if ((c8 & 3) == 0) {
    const int kb = c8 >> 2, q = kb & 3;
    const int64_t idx = ((int64_t)(row >> 7) * (k >> 7) + (kb >> 2)) * 512 + (q & 1) * 256 + (row & 31) * 8 +
                        (q >> 1) * 4 + ((row >> 5) & 3);
    scales[idx] = (uint8_t)sbyte;
  }
}

hipError_t launch_mxfp4_quantize(const void* src, int src_dtype, int rows, int k, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream) {
  const int rows_pad = ((rows + 255) / 256) * 256;
  const int64_t threads = (int64_t)rows_pad * (k / 8);
  const dim3 grid((unsigned)ceil_div(threads, 256));
  TimingScope ts(kKcMx4Quant, stream, (double)rows * k * ((src_dtype == kBF16 ? 2.0 : 4.0) + 0.5 + 1.0 / 32));
  if (src_dtype == kBF16)
    hipLaunchKernelGGL(mxfp4_quantize_kernel<bf16_t>, grid, dim3(256), 0, stream, static_cast<const bf16_t*>(src),
                       rows, k, rows_pad, codes, scales);
  else
    hipLaunchKernelGGL(mxfp4_quantize_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(src), rows,
                       k, rows_pad, codes, scales);
  return hipGetLastError();
}

// ===========================================================================
// Blockwise E4M3 quantization (the "blockwise" recipe of "FP8 training for
// Flux models", Configuration): one power-of-two scale 2^e per tile along K,
// tiles of 1 x 128 values (activations) or 128 x 128 (weights), e the largest
// integer with amax * 2^e <= 448, clamped to [-127, 127] (0 for an all-zero
// tile; a tile holding a non-finite value gets the NaN byte 0xFF and its
// elements are encoded unscaled).  With a power-of-two scale the dequantized
// product of a 128-wide k block is 2^-(e_x + e_w) times the code product, so
// the scales are written as E8M0 bytes 127 - e, replicated over the four
// 32-value blocks of the tile, into the layout of mx_quantize_kernel: the
// MXFP8 GEMM consumes the operands unchanged.
//
// One 256-thread block per 128 x 128 tile: thread t covers columns
// 8 (t % 16) .. + 7 of tile rows t / 16 + 16 j, j < 8, so sixteen lanes read
// one row's 256 contiguous bytes (bf16) per load.
// ===========================================================================
__device__ __forceinline__ int block_scale_exp(uint32_t m) {
  if (m == 0u) return 0;
  if (m < 0x00800000u) return 127;   // subnormal amax: e >= 135 before the clamp
  const int ex = (int)(m >> 23) - 127;   // amax = 1.f * 2^ex
  // amax * 2^e <= 448 = 1.75 * 2^8: e = 8 - ex when 1.f <= 1.75, else 7 - ex
  const int e = (m & 0x7fffffu) <= 0x600000u ? 8 - ex : 7 - ex;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

template <typename T>
__global__ void __launch_bounds__(256) fp8_block_quantize_kernel(const T* __restrict__ src, int rows, int k,
                                                                 int tile_rows, uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales) {
  __shared__ uint32_t red[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int col = blockIdx.x * 128 + (t & 15) * 8;
  const int row0 = blockIdx.y * 128 + (t >> 4);
  float v[8][8];
  uint32_t rm[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = row0 + 16 * j;
    if (row < rows) {
      load8<T>(src + (int64_t)row * k + col, v[j]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] = 0.f;
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, abs_bits(v[j][i]));   // NaN patterns sort above infinity
    rm[j] = m;
  }
  if (tile_rows == 1) {   // block-uniform: the row's amax over its sixteen lanes
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t m = rm[j];
      m = max(m, (uint32_t)__shfl_xor((int)m, 1));
      m = max(m, (uint32_t)__shfl_xor((int)m, 2));
      m = max(m, (uint32_t)__shfl_xor((int)m, 4));
      m = max(m, (uint32_t)__shfl_xor((int)m, 8));
      rm[j] = m;
    }
  } else {                // the whole tile's amax
    uint32_t m = rm[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) m = max(m, rm[j]);
    m = wave_max_u32(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
#pragma unroll
    for (int j = 0; j < 8; ++j) rm[j] = m;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = row0 + 16 * j;
    uint32_t sbyte;
    float mul = 1.0f;
    if (rm[j] >= 0x7f800000u) {
      sbyte = 0xFFu;
    } else {
      const int e = block_scale_exp(rm[j]);
      sbyte = (uint32_t)(127 - e);
      mul = __uint_as_float((uint32_t)(127 + e) << 23);   // 2^e, normal: a finite amax gives e >= -120
    }
    if (row < rows) {
      uint2 o;
      o.x = f32x4_to_e4m3(v[j][0] * mul, v[j][1] * mul, v[j][2] * mul, v[j][3] * mul);
      o.y = f32x4_to_e4m3(v[j][4] * mul, v[j][5] * mul, v[j][6] * mul, v[j][7] * mul);
      *reinterpret_cast<uint2*>(codes + (int64_t)row * k + col) = o;
    }
    if ((t & 3) == 0) {   // the first lane of each 32-value block writes its byte (pad rows too)
      const int kb = col >> 5, kt = kb >> 1, h = kb & 1;
      const int64_t idx = (((int64_t)(row >> 7) * (k >> 6) + kt) * 2 + h) * 128 + (row & 31) * 4 + ((row >> 5) & 3);
      scales[idx] = (uint8_t)sbyte;
    }
  }
}

hipError_t launch_fp8_block_quantize(const void* src, int src_dtype, int rows, int k, int tile_rows, uint8_t* codes,
                                     uint8_t* scales, hipStream_t stream) {
  const int rows_pad = ((rows + 255) / 256) * 256;
  const dim3 grid((unsigned)(k / 128), (unsigned)(rows_pad / 128));
  TimingScope ts(kKcMxQuant, stream, (double)rows * k * ((src_dtype == kBF16 ? 2.0 : 4.0) + 1.0 + 1.0 / 32));
  if (src_dtype == kBF16)
    hipLaunchKernelGGL(fp8_block_quantize_kernel<bf16_t>, grid, dim3(256), 0, stream, static_cast<const bf16_t*>(src),
                       rows, k, tile_rows, codes, scales);
  else
    hipLaunchKernelGGL(fp8_block_quantize_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(src),
                       rows, k, tile_rows, codes, scales);
  return hipGetLastError();
}

// ===========================================================================
// dst = e4m3(src * scale(rec)) over a whole tensor (the weight cast of a
// forward); each thread converts 16 consecutive elements per step, and one
// atomic per block raises the record's amax (atomics on one address
// serialize, so the grid is kept to at most 1024 blocks).
template <typename T>
__global__ void __launch_bounds__(256) fp8_quantize_kernel(const T* __restrict__ src, int64_t n,
                                                           flux_fp8_tensor* rec, uint8_t* __restrict__ dst) {
  __shared__ uint32_t red[4];
  const float qs = fp8_scale(rec);
  const int64_t n16 = n / 16;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t mx = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    float v[16];
    if constexpr (sizeof(T) == 4) {
      const float4* p = reinterpret_cast<const float4*>(src) + 4 * i;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 f = p[j];
        v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
      }
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(src) + 2 * i;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 w = p[j];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[8 * j + 2 * e] = __uint_as_float(ws[e] << 16);
          v[8 * j + 2 * e + 1] = __uint_as_float(ws[e] & 0xffff0000u);
        }
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = max(mx, abs_bits(v[4 * j + e]));
      o[j] = f32x4_to_e4m3(v[4 * j] * qs, v[4 * j + 1] * qs, v[4 * j + 2] * qs, v[4 * j + 3] * qs);
    }
    reinterpret_cast<uint4*>(dst)[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (blockIdx.x == 0 && (int64_t)threadIdx.x < n - n16 * 16) {
    const int64_t k = n16 * 16 + threadIdx.x;
    const float x = load_f32<T>(src + k);
    mx = max(mx, abs_bits(x));
    dst[k] = (uint8_t)f32_to_e4m3(x * qs);
  }
  mx = wave_max_u32(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t b = max(max(red[0], red[1]), max(red[2], red[3]));
    if (b) fp8_amax_raise(rec, __uint_as_float(b));
  }
}

hipError_t launch_fp8_quantize(const void* src, int src_dtype, int64_t n, flux_fp8_tensor* rec, uint8_t* dst,
                               hipStream_t stream) {
  int64_t blocks = ceil_div(n / 16 > 0 ? n / 16 : 1, 256);
  if (blocks > 1024) blocks = 1024;
  TimingScope ts(kKcFp8Cast, stream, (double)n * ((src_dtype == kF32 ? 4.0 : 2.0) + 1.0));
  if (src_dtype == kF32)
    hipLaunchKernelGGL(fp8_quantize_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const float*>(src), n, rec, dst);
  else
    hipLaunchKernelGGL(fp8_quantize_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(src), n, rec, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Current ("tensorwise") scaling, the alternative recipe the FP8 page names:
// the scale comes from the amax of the tensor being quantized, not from
// earlier forwards.  Three launches ahead of the quantization: clear the
// record's amax, reduce max |src| into it (one atomic per block), set
// scale = fp32(448 / amax) and scale_inv = 1 / scale when the amax is finite
// and positive (else keep the scale; a non-finite amax sets the sticky flag).
// ---------------------------------------------------------------------------
__global__ void fp8_amax_clear_kernel(flux_fp8_tensor* rec) {
  if (threadIdx.x == 0) rec->amax_bits = 0u;
}

template <typename T>
__global__ void __launch_bounds__(256) fp8_amax_kernel(const T* __restrict__ src, int64_t n, flux_fp8_tensor* rec) {
  __shared__ uint32_t red[4];
  uint32_t m = 0;
  // 16-byte loads over the whole vectors, then the tail element by element
  constexpr int V = 16 / sizeof(T);
  const int64_t nv = n / V, stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nv; i += stride) {
    const uint4 w = reinterpret_cast<const uint4*>(src)[i];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (sizeof(T) == 4) {
        m = max(m, ws[e] & 0x7fffffffu);   // NaN patterns sort above every finite one
      } else {
        m = max(m, abs_bits(__uint_as_float(ws[e] << 16)));
        m = max(m, abs_bits(__uint_as_float(ws[e] & 0xffff0000u)));
      }
    }
  }
  for (int64_t i = nv * V + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    m = max(m, abs_bits(load_f32<T>(src + i)));
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t b = max(max(red[0], red[1]), max(red[2], red[3]));
    if (b) fp8_amax_raise(rec, __uint_as_float(b));
  }
}

__global__ void fp8_current_scale_kernel(flux_fp8_tensor* rec) {
  if (threadIdx.x != 0) return;
  const float a = __uint_as_float(rec->amax_bits);
  uint32_t flags = rec->flags;
  if (!__builtin_isfinite(a)) flags |= FLUX_FP8_NONFINITE;
  if (__builtin_isfinite(a) && a > 0.f) {
    const float sc = 448.0f / a;
    const float inv = 1.0f / sc;
    // an amax so small that 448 / amax overflows keeps the old scale
    if (__builtin_isfinite(sc) && __builtin_isfinite(inv) && inv > 0.f) {
      rec->scale = sc;
      rec->scale_inv = inv;
      flags |= FLUX_FP8_SCALE_SET;
    }
  }
  rec->flags = flags;
}

hipError_t launch_fp8_current_scale(const void* src, int src_dtype, int64_t n, flux_fp8_tensor* rec,
                                    hipStream_t stream) {
  TimingScope ts(kKcFp8Cast, stream, (double)n * (src_dtype == kF32 ? 4.0 : 2.0));
  hipLaunchKernelGGL(fp8_amax_clear_kernel, dim3(1), dim3(64), 0, stream, rec);
  int64_t blocks = ceil_div(n, 256 * 64);
  if (blocks > 512) blocks = 512;
  if (blocks < 1) blocks = 1;
  if (src_dtype == kF32)
    hipLaunchKernelGGL(fp8_amax_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const float*>(src), n, rec);
  else
    hipLaunchKernelGGL(fp8_amax_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(src), n, rec);
  hipLaunchKernelGGL(fp8_current_scale_kernel, dim3(1), dim3(64), 0, stream, rec);
  return hipGetLastError();
}


// One thread per record: the amax recorded since the last update enters the
// history ring, the selected amax (newest entry, or the history maximum with
// NaN propagating) gives scale = (448 / amax) * 2^-margin when the amax is
// finite and positive and the scale and its reciprocal are finite and
// non-zero; the amax is then cleared for the next forward.
__global__ void fp8_update_kernel(flux_fp8_tensor* recs, int n, int algo, int margin) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  flux_fp8_tensor* t = recs + i;
  const float a = __uint_as_float(t->amax_bits);
  const uint32_t pos = t->hist_pos % FLUX_FP8_HISTORY;
  t->amax_history[pos] = a;
  t->hist_pos = (pos + 1) % FLUX_FP8_HISTORY;
  const uint32_t len = t->hist_len < FLUX_FP8_HISTORY ? t->hist_len + 1 : FLUX_FP8_HISTORY;
  t->hist_len = len;
  float sel = a;
  if (algo == 1) {
    bool nan = false;
    float m = 0.f;
    for (uint32_t j = 0; j < len; ++j) {
      const float h = t->amax_history[j];
      nan = nan || (h != h);
      m = h > m ? h : m;
    }
    sel = nan ? __uint_as_float(0x7fc00000u) : m;
  }
  uint32_t flags = t->flags;
  if (!(__builtin_isfinite(a))) flags |= FLUX_FP8_NONFINITE;
  if (__builtin_isfinite(sel) && sel > 0.f) {
    const float s = ldexpf(448.0f / sel, -margin);
    const float inv = 1.0f / s;
    // a scale that overflows (or underflows) fp32 is not taken: the old one stays
    if (__builtin_isfinite(s) && s > 0.f && __builtin_isfinite(inv)) {
      t->scale = s;
      t->scale_inv = inv;
      flags |= FLUX_FP8_SCALE_SET;
    }
  }
  t->flags = flags;
  t->amax_bits = 0u;
}

hipError_t launch_fp8_update(flux_fp8_tensor* rec, int n, int algo, int margin, hipStream_t stream) {
  TimingScope ts(kKcMisc, stream);
  hipLaunchKernelGGL(fp8_update_kernel, dim3((unsigned)ceil_div(n, 64)), dim3(64), 0, stream, rec, n, algo, margin);
  return hipGetLastError();
}

}  // namespace flux
