// Backward pass of the Flux blocks under the rectified-flow objective ("Flux
// architecture deep dive", Flow matching framework: the training step
// backpropagates the velocity MSE through the network).  The chain rule of
// each forward step, as kernels:
//   * batched transposes (operands of the weight-gradient and data-gradient
//     GEMMs, which reuse the forward's GEMM C = A W^T);
//   * column sums in a fixed order (bias, gate, shift and scale gradients);
//   * gate, GELU and LayerNorm-modulate backward, RMSNorm + RoPE backward;
//   * attention backward, flash style: P is recomputed from the scores and
//     the forward's log-sum-exp, never stored; one kernel accumulates dK and
//     dV per key block over all queries, another dQ per query block over all
//     keys;
//   * adaLN modulation backward (weight outer product, transposed GEMV).
// Every reduction runs in a fixed order, so results are bitwise repeatable.
#include <math.h>

#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace flux {

__device__ __forceinline__ int swap23b(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ __forceinline__ int64_t row_off(const RowMap& m, int64_t r) {
  return (r / m.seg) * m.bstride + (r % m.seg) * m.ld;
}

// d/dx of x Phi(x) = Phi(x) + x phi(x)
__device__ __forceinline__ float gelu_grad_f(float x) {
  const float cdf = 0.5f * (1.0f + erf_as(x * 0.70710678118654752f));
  const float pdf = 0.3989422804014327f * __builtin_amdgcn_exp2f(-0.5f * x * x * 1.4426950408889634f);
  return __builtin_fmaf(x, pdf, cdf);
}
__device__ __forceinline__ float silu_grad_f(float x) {
  const float s = 1.0f / (1.0f + __expf(-x));
  return s * (1.0f + x * (1.0f - s));
}

// ===========================================================================
// Batched transpose to bf16: dst[z][c][r] = src[z][r][c] (r < R, c < C) from
// fp32, bf16 or fp16 sources;
// columns r in [R, R_fill) of dst are zero (padding of a GEMM's K).
// 64 x 64 tiles through LDS; 4 consecutive elements per thread on both sides.
// ===========================================================================
template <typename TS> constexpr bool kBf16Src = false;
template <> constexpr bool kBf16Src<bf16_t> = true;

template <typename TS>
__global__ void __launch_bounds__(256) transpose_kernel(TransposeArgs a) {
  __shared__ float tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64, z = blockIdx.z;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const TS* src = reinterpret_cast<const TS*>(a.src) + (int64_t)z * a.src_zstride;   // rows through smap
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + ty + 16 * i, c = c0 + 4 * tx;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (r < a.R && c < a.C) {
      if constexpr (sizeof(TS) == 4) {
        const float4 f = *reinterpret_cast<const float4*>(src + row_off(a.smap, r) + c);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
      } else {
        unpack4_16(*reinterpret_cast<const uint2*>(src + row_off(a.smap, r) + c), sizeof(TS) == 2 && !kBf16Src<TS>, v);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[ty + 16 * i][4 * tx + e] = v[e];
  }
  __syncthreads();
  bf16_t* dst = reinterpret_cast<bf16_t*>(a.dst) + (int64_t)z * a.dst_zstride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = c0 + ty + 16 * i, r = r0 + 4 * tx;
    if (c < a.C && r < a.R_fill) {
      uint2 o;
      o.x = pack_bf16x2(tile[4 * tx][ty + 16 * i], tile[4 * tx + 1][ty + 16 * i]);
      o.y = pack_bf16x2(tile[4 * tx + 2][ty + 16 * i], tile[4 * tx + 3][ty + 16 * i]);
      *reinterpret_cast<uint2*>(dst + (int64_t)c * a.dst_ld + r) = o;
    }
  }
}

hipError_t launch_transpose(const TransposeArgs& a, int src_dtype, hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(a.C, 64), (unsigned)ceil_div(a.R_fill, 64), (unsigned)a.Z);
  TimingScope ts(kKcBwdElem, stream, (double)a.Z * ((double)a.R * a.C * (src_dtype == kF32 ? 4 : 2) +
                                                    (double)a.R_fill * a.C * 2));
  if (src_dtype == kF32)
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, stream, a);
  else if (src_dtype == kF16)
    hipLaunchKernelGGL(transpose_kernel<_Float16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ===========================================================================
// Column sums.  Stage 1: part[(z * nrb + rb) * C + c] = sum over the rows
// [rb * rpb, min((rb + 1) * rpb, R)) of sample z of A (* Bm); stage 2 sums the
// nrb partials of every (z, c) in index order.
// ===========================================================================
template <typename TA>
__global__ void __launch_bounds__(256) colsum_partial_kernel(ColsumArgs a) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int rb = blockIdx.y, z = blockIdx.z;
  if (c >= a.C) return;
  const int r_begin = rb * a.rpb, r_end = min(a.R, r_begin + a.rpb);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const TA* A = reinterpret_cast<const TA*>(a.A);
  for (int r = r_begin; r < r_end; ++r) {
    const int64_t g = (int64_t)z * a.R + r;
    float v[4];
    if constexpr (sizeof(TA) == 4) {
      const float4 f = *reinterpret_cast<const float4*>(A + row_off(a.amap, g) + c);
      v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(A + row_off(a.amap, g) + c);
      v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
      v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
    }
    if (a.Bm) {
      const float4 f = *reinterpret_cast<const float4*>(a.Bm + row_off(a.bmap, g) + c);
      v[0] *= f.x; v[1] *= f.y; v[2] *= f.z; v[3] *= f.w;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
  *reinterpret_cast<float4*>(a.part + ((int64_t)z * a.nrb + rb) * a.C + c) = make_float4(acc[0], acc[1], acc[2], acc[3]);
}

// Partials of sample z sit at part + z * zs + i * ps (i < np).  The sum runs
// as a fixed tree: chunks of kRedChunk partials are summed in place (into the
// chunk's first slot) until at most kRedChunk remain, then the last pass
// writes out[z * out_zstride + c] (=, += or += silu'(aux[z][c]) *) the sum.
constexpr int kRedChunk = 16;

__global__ void __launch_bounds__(256) reduce_chunks_kernel(float* part, int np, int64_t ps, int64_t zs, int C) {
  const int c = blockIdx.x * 256 + threadIdx.x, k = blockIdx.y, z = blockIdx.z;
  if (c >= C) return;
  float* base = part + (int64_t)z * zs + c;
  const int i0 = k * kRedChunk, i1 = min(np, i0 + kRedChunk);
  float s = 0.f;
  for (int i = i0; i < i1; ++i) s += base[(int64_t)i * ps];
  base[(int64_t)i0 * ps] = s;
}

__global__ void __launch_bounds__(256) reduce_parts_kernel(ReduceArgs a, int np, int64_t ps, int64_t zs) {
  const int c = blockIdx.x * 256 + threadIdx.x, z = blockIdx.y;
  if (c >= a.C) return;
  float s = 0.f;
  const float* p = a.part + (int64_t)z * zs + c;
  for (int i = 0; i < np; ++i) s += p[(int64_t)i * ps];
  float* o = a.out + (int64_t)z * a.out_zstride + c;
  if (a.mode == 0) *o = s;
  else if (a.mode == 1) *o += s;
  else if (a.mode == 2) *o += s * silu_grad_f(a.aux[(int64_t)z * a.aux_zstride + c]);
  else *o = s * silu_grad_f(a.aux[(int64_t)z * a.aux_zstride + c]);
}

// note: overwrites the partials (scratch)
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream) {
  TimingScope ts(kKcBwdElem, stream, 4.0 * a.Z * (double)a.C * (a.np + 1));
  int np = a.np;
  int64_t ps = a.pstride ? a.pstride : a.C;
  const int64_t zs = (int64_t)a.np * ps;
  float* part = const_cast<float*>(a.part);
  while (np > kRedChunk) {
    const int nch = (int)ceil_div(np, kRedChunk);
    hipLaunchKernelGGL(reduce_chunks_kernel, dim3((unsigned)ceil_div(a.C, 256), (unsigned)nch, (unsigned)a.Z),
                       dim3(256), 0, stream, part, np, ps, zs, a.C);
    np = nch;
    ps *= kRedChunk;
  }
  hipLaunchKernelGGL(reduce_parts_kernel, dim3((unsigned)ceil_div(a.C, 256), (unsigned)a.Z), dim3(256), 0, stream, a,
                     np, ps, zs);
  return hipGetLastError();
}

hipError_t launch_colsum(ColsumArgs a, int a_dtype, float* out, int64_t out_zstride, int mode, hipStream_t stream) {
  {
    TimingScope ts(kKcBwdElem, stream, (double)a.Z * a.R * a.C * ((a_dtype == kF32 ? 4 : 2) + (a.Bm ? 4 : 0)));
    const dim3 grid((unsigned)ceil_div(a.C, 1024), (unsigned)a.nrb, (unsigned)a.Z);
    if (a_dtype == kF32)
      hipLaunchKernelGGL(colsum_partial_kernel<float>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(colsum_partial_kernel<bf16_t>, grid, dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ReduceArgs r{};
  r.part = a.part; r.np = a.nrb; r.C = a.C; r.Z = a.Z;
  r.out = out; r.out_zstride = out_zstride; r.mode = mode;
  return launch_reduce(r, stream);
}

// ===========================================================================
// Elementwise steps, 4 columns per thread, rows through RowMaps
// ===========================================================================
// kEwGateBwd:  out (bf16) = gate[b][c] * x (float)        dy of x += gate * y
// kEwGeluBwd:  out (16-bit) = x (16-bit) * GELU'(y (16-bit))   d(pre-activation) of u = GELU(a)
// kEwGelu:     out (16-bit) = GELU(x (16-bit))
// (16-bit: bf16, or fp16 where the f16 mask bit of that operand is set)
// kEwGateAdd:  out (float) += gate[b][c] * x (float)      the forward's gated residual
__global__ void __launch_bounds__(256) elementwise_kernel(EwArgs a) {
  const int64_t n4 = (int64_t)a.rows * (a.C / 4);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / (a.C / 4);
    const int c = (int)(i % (a.C / 4)) * 4;
    float x[4], y[4] = {0.f, 0.f, 0.f, 0.f}, o[4];
    if (a.op == kEwGateBwd || a.op == kEwGateAdd) {
      const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + row_off(a.xmap, r) + c);
      x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
      const float4 g = *reinterpret_cast<const float4*>(a.gate + (r / a.xmap.seg) * a.gate_bstride + c);
      y[0] = g.x; y[1] = g.y; y[2] = g.z; y[3] = g.w;
    } else {
      unpack4_16(*reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(a.x) + row_off(a.xmap, r) + c),
                 a.f16 & 1, x);
      if (a.op == kEwGeluBwd)
        unpack4_16(*reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(a.y) + row_off(a.ymap, r) + c),
                   a.f16 & 2, y);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (a.op == kEwGateBwd || a.op == kEwGateAdd) o[e] = y[e] * x[e];
      else if (a.op == kEwGeluBwd) o[e] = x[e] * gelu_grad_f(y[e]);
      else o[e] = gelu_f(x[e]);
    }
    if (a.op == kEwGateAdd) {
      float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + row_off(a.omap, r) + c);
      float4 v = *p;
      v.x += o[0]; v.y += o[1]; v.z += o[2]; v.w += o[3];
      *p = v;
    } else {
      *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(a.out) + row_off(a.omap, r) + c) = pack4_16(o, a.f16 & 4);
    }
  }
}

hipError_t launch_elementwise(const EwArgs& a, hipStream_t stream) {
  const int64_t n4 = (int64_t)a.rows * (a.C / 4);
  int64_t blocks = ceil_div(n4 > 0 ? n4 : 1, 256);
  if (blocks > 8192) blocks = 8192;
  const double bytes = (double)a.rows * a.C * (a.op == kEwGateAdd ? 12.0 : a.op == kEwGateBwd ? 6.0 :
                                               a.op == kEwGeluBwd ? 6.0 : 4.0);
  TimingScope ts(kKcBwdElem, stream, bytes);
  hipLaunchKernelGGL(elementwise_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ===========================================================================
// LayerNorm-modulate backward.  h = xhat (1 + scale) + shift, xhat = (x - mu)
// rstd: dxhat = dh (1 + scale); dx = rstd (dxhat - mean(dxhat) - xhat
// mean(dxhat xhat)), added to the residual gradient; per-wave partial column
// sums of dh (-> dshift) and dh xhat (-> dscale).  One wave per row, the row
// in registers (NV float4 per lane); blocks never span two samples.
// ===========================================================================
template <int NV>
__global__ void __launch_bounds__(256) ln_mod_bwd_kernel(LnBwdArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int blk = blockIdx.x, z = blockIdx.y;
  const int D = NV * 256;
  float opsc[NV][4];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const float4 s = *reinterpret_cast<const float4*>(a.scale + (int64_t)z * a.mod_bstride + v * 256 + lane * 4);
    opsc[v][0] = 1.f + s.x; opsc[v][1] = 1.f + s.y; opsc[v][2] = 1.f + s.z; opsc[v][3] = 1.f + s.w;
  }
  float acc_sh[NV][4], acc_sc[NV][4];
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc_sh[v][e] = acc_sc[v][e] = 0.f;
  const int r_begin = blk * a.rpb, r_end = min(a.seg, r_begin + a.rpb);
  for (int r = r_begin + wave; r < r_end; r += 4) {
    const int64_t g = (int64_t)z * a.seg + r;
    const float* xr = a.x + row_off(a.xmap, g);
    const float* dr = a.dh + row_off(a.dhmap, g);
    float x[NV][4], dh[NV][4];
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const float4 f = *reinterpret_cast<const float4*>(xr + v * 256 + lane * 4);
      const float4 d = *reinterpret_cast<const float4*>(dr + v * 256 + lane * 4);
      x[v][0] = f.x; x[v][1] = f.y; x[v][2] = f.z; x[v][3] = f.w;
      dh[v][0] = d.x; dh[v][1] = d.y; dh[v][2] = d.z; dh[v][3] = d.w;
      s += (f.x + f.y) + (f.z + f.w);
    }
    const float mu = wave_sum(s) / (float)D;
    float q = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[v][e] -= mu;
        q += x[v][e] * x[v][e];
      }
    const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)D + a.eps);
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[v][e] *= rstd;                       // xhat
        acc_sh[v][e] += dh[v][e];
        acc_sc[v][e] += dh[v][e] * x[v][e];
        dh[v][e] *= opsc[v][e];                // dxhat
        s1 += dh[v][e];
        s2 += dh[v][e] * x[v][e];
      }
    const float m1 = wave_sum(s1) / (float)D, m2 = wave_sum(s2) / (float)D;
    float* o = a.dx + row_off(a.dxmap, g);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      float4* p = reinterpret_cast<float4*>(o + v * 256 + lane * 4);
      float4 t = *p;
      t.x += rstd * (dh[v][0] - m1 - x[v][0] * m2);
      t.y += rstd * (dh[v][1] - m1 - x[v][1] * m2);
      t.z += rstd * (dh[v][2] - m1 - x[v][2] * m2);
      t.w += rstd * (dh[v][3] - m1 - x[v][3] * m2);
      *p = t;
    }
  }
  const int64_t pi = ((int64_t)z * gridDim.x + blk) * 4 + wave;   // partial index within sample z
  float* psh = a.part_sh + pi * D;
  float* psc = a.part_sc + pi * D;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    *reinterpret_cast<float4*>(psh + v * 256 + lane * 4) = make_float4(acc_sh[v][0], acc_sh[v][1], acc_sh[v][2], acc_sh[v][3]);
    *reinterpret_cast<float4*>(psc + v * 256 + lane * 4) = make_float4(acc_sc[v][0], acc_sc[v][1], acc_sc[v][2], acc_sc[v][3]);
  }
}

int ln_bwd_blocks(int seg, int batch) {
  int nb = (int)ceil_div(256, batch > 0 ? batch : 1);
  const int by_rows = (int)ceil_div(seg, 8);        // at least 8 rows per block (2 per wave)
  if (nb > by_rows) nb = by_rows;
  return nb < 1 ? 1 : nb;
}

hipError_t launch_ln_mod_bwd(LnBwdArgs a, int dim, hipStream_t stream) {
  const int nb = ln_bwd_blocks(a.seg, a.batch);
  a.rpb = (int)ceil_div(a.seg, nb);
  const dim3 grid((unsigned)nb, (unsigned)a.batch);
  {
    TimingScope ts(kKcBwdElem, stream, (double)a.batch * a.seg * dim * 16.0);
    switch (dim / 256) {
      case 1: hipLaunchKernelGGL(ln_mod_bwd_kernel<1>, grid, dim3(256), 0, stream, a); break;
      case 2: hipLaunchKernelGGL(ln_mod_bwd_kernel<2>, grid, dim3(256), 0, stream, a); break;
      case 3: hipLaunchKernelGGL(ln_mod_bwd_kernel<3>, grid, dim3(256), 0, stream, a); break;
      case 4: hipLaunchKernelGGL(ln_mod_bwd_kernel<4>, grid, dim3(256), 0, stream, a); break;
      case 6: hipLaunchKernelGGL(ln_mod_bwd_kernel<6>, grid, dim3(256), 0, stream, a); break;
      case 8: hipLaunchKernelGGL(ln_mod_bwd_kernel<8>, grid, dim3(256), 0, stream, a); break;
      case 12: hipLaunchKernelGGL(ln_mod_bwd_kernel<12>, grid, dim3(256), 0, stream, a); break;
      default: hipLaunchKernelGGL(ln_mod_bwd_kernel<16>, grid, dim3(256), 0, stream, a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ReduceArgs r{};
  r.np = nb * 4; r.C = dim; r.Z = a.batch; r.mode = 0;
  r.part = a.part_sh; r.out = a.dshift; r.out_zstride = a.mod_bstride;
  hipError_t e = launch_reduce(r, stream);
  if (e != hipSuccess) return e;
  r.part = a.part_sc; r.out = a.dscale;
  return launch_reduce(r, stream);
}

// ===========================================================================
// q/k RMSNorm + RoPE backward and the v passthrough: dQ, dK, dV (fp32,
// head-major [B, H, Lp, 128]) -> d(q|k|v) (bf16 token rows); per-block
// partial sums of dgamma = sum d(normed) * n for the image and text streams.
// One block per (64 tokens, head, sample); 16 lanes of 8 elements per row.
// ===========================================================================
__global__ void __launch_bounds__(256) prep_bwd_kernel(PrepBwdArgs a) {
  constexpr int DH = 128, E = 8, TOK = 64;
  __shared__ float red[16][2][2][DH];          // [token group][stream][q / k][d]
  const int j0 = blockIdx.x * TOK, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, g = tid & 15, rg = tid >> 4, d0 = g * E;
  const int64_t head_row0 = ((int64_t)b * a.heads + h) * a.seq_pad;
  const int D = a.heads * DH;
  float acc[2][2][E];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[s][w][e] = 0.f;
  for (int i = 0; i < TOK / 16; ++i) {
    const int j = j0 + rg + 16 * i;
    const bool in = j < a.seq;                  // uniform over the 16-lane row group
    const int st = j >= a.l_img ? 1 : 0;
#pragma unroll
    for (int which = 0; which < 3; ++which) {
      const float* src = which == 0 ? a.dq : which == 1 ? a.dk : a.dv;
      float d[E];
      if (in) {
        const float4 f0 = *reinterpret_cast<const float4*>(src + (head_row0 + j) * DH + d0);
        const float4 f1 = *reinterpret_cast<const float4*>(src + (head_row0 + j) * DH + d0 + 4);
        d[0] = f0.x; d[1] = f0.y; d[2] = f0.z; d[3] = f0.w; d[4] = f1.x; d[5] = f1.y; d[6] = f1.z; d[7] = f1.w;
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) d[e] = 0.f;
      }
      if (which < 2) {
        if (a.rope && in) {   // the rotation's transpose: turn each pair back by its angle
          const float2* cs = reinterpret_cast<const float2*>(a.rope) + ((int64_t)b * a.seq + j) * (DH / 2) + d0 / 2;
#pragma unroll
          for (int e = 0; e < E / 2; ++e) {
            const float2 t = cs[e];
            const float u = d[2 * e], w = d[2 * e + 1];
            d[2 * e] = u * t.x + w * t.y;
            d[2 * e + 1] = w * t.x - u * t.y;
          }
        }
        const float* gm = which == 0 ? (st ? a.gq_txt : a.gq_img) : (st ? a.gk_txt : a.gk_img);
        if (gm) {
          float x[E];
          if (in) {
            const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.src) +
                                                              (int64_t)b * a.src_bstride + (int64_t)j * a.src_ld +
                                                              which * D + h * DH + d0);
            x[0] = __uint_as_float(raw.x << 16); x[1] = __uint_as_float(raw.x & 0xffff0000u);
            x[2] = __uint_as_float(raw.y << 16); x[3] = __uint_as_float(raw.y & 0xffff0000u);
            x[4] = __uint_as_float(raw.z << 16); x[5] = __uint_as_float(raw.z & 0xffff0000u);
            x[6] = __uint_as_float(raw.w << 16); x[7] = __uint_as_float(raw.w & 0xffff0000u);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) x[e] = 0.f;
          }
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) ss += x[e] * x[e];
          const float rstd = 1.0f / sqrtf(wave_sum<16>(ss) / (float)DH + a.eps);
          float dn[E], n[E], dot = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            n[e] = x[e] * rstd;
            dn[e] = d[e] * gm[d0 + e];
            dot += dn[e] * n[e];
            acc[st][which][e] += d[e] * n[e];
          }
          const float m = wave_sum<16>(dot) / (float)DH;
#pragma unroll
          for (int e = 0; e < E; ++e) d[e] = rstd * (dn[e] - n[e] * m);
        }
      }
      if (in) {
        uint4 o;
        o.x = pack_bf16x2(d[0], d[1]); o.y = pack_bf16x2(d[2], d[3]);
        o.z = pack_bf16x2(d[4], d[5]); o.w = pack_bf16x2(d[6], d[7]);
        *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(a.dst) + (int64_t)b * a.dst_bstride +
                                  (int64_t)j * a.dst_ld + which * D + h * DH + d0) = o;
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
      for (int e = 0; e < E; ++e) red[rg][s][w][d0 + e] = acc[s][w][e];
  __syncthreads();
  // 512 sums of 16 partials, two per thread, in token-group order
  const int64_t blk = ((int64_t)b * gridDim.y + h) * gridDim.x + blockIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = tid + 256 * k;             // (stream, which, d)
    const int s = idx >> 8, w = (idx >> 7) & 1, d = idx & 127;
    float t = 0.f;
    for (int r = 0; r < 16; ++r) t += red[r][s][w][d];
    a.part[blk * 512 + idx] = t;
  }
}

hipError_t launch_prep_bwd(const PrepBwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(a.seq, 64), (unsigned)a.heads, (unsigned)a.batch);
  TimingScope ts(kKcBwdElem, stream, (double)a.batch * a.seq * a.heads * 128.0 * (12.0 + 4.0 + 6.0));
  hipLaunchKernelGGL(prep_bwd_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

int prep_bwd_parts(int batch, int seq, int heads) { return (int)ceil_div(seq, 64) * heads * batch; }

// ===========================================================================
// Attention backward, step 0: from the output gradient dO and the output O
// (token rows, head h at column h * 128; dO bf16, O bf16 or fp16): dOh [B, H, Lp, 128], its
// transpose dOt [B, H, 128, Lp] (zero beyond seq) and Dv[q] = dO[q] . O[q]
// per head (0 beyond seq).  One block per (64 tokens, head, sample).
// ===========================================================================
__global__ void __launch_bounds__(256) attn_bwd_pre_kernel(AttnBwdArgs a) {
  constexpr int DH = 128, E = 8, TOK = 64;
  __shared__ bf16_t tile[TOK][DH + 8];
  const int j0 = blockIdx.x * TOK, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, g = tid & 15, rg = tid >> 4, d0 = g * E;
  const int64_t bh = (int64_t)b * a.heads + h;
  for (int i = 0; i < TOK / 16; ++i) {
    const int r = rg + 16 * i, j = j0 + r;
    uint4 dov = {0u, 0u, 0u, 0u};
    float dot = 0.f;
    if (j < a.seq) {
      dov = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.dout) + (int64_t)b * a.dout_bstride +
                                             (int64_t)j * a.dout_ld + h * DH + d0);
      const uint4 ov = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.o) + (int64_t)b * a.o_bstride +
                                                        (int64_t)j * a.o_ld + h * DH + d0);
      float fd[8], fo[8];
      unpack4_16(make_uint2(dov.x, dov.y), false, fd); unpack4_16(make_uint2(dov.z, dov.w), false, fd + 4);
      unpack4_16(make_uint2(ov.x, ov.y), a.o_f16, fo); unpack4_16(make_uint2(ov.z, ov.w), a.o_f16, fo + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) dot += fd[2 * e] * fo[2 * e] + fd[2 * e + 1] * fo[2 * e + 1];
    }
    dot = wave_sum<16>(dot);
    *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(a.doh) + (bh * a.seq_pad + j) * DH + d0) = dov;
    *reinterpret_cast<uint4*>(&tile[r][d0]) = dov;
    if (g == 0) a.dd[bh * a.seq_pad + j] = dot;
  }
  __syncthreads();
  // dOt row d holds the tile's 64 tokens: 8 chunks of 8 per row, 1024 chunks
  bf16_t* dst = reinterpret_cast<bf16_t*>(a.dot) + bh * DH * a.seq_pad + j0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i, d = idx >> 3, c = (idx & 7) * 8;
    uint4 o;
    uint32_t* po = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
    for (int e = 0; e < 4; ++e) po[e] = (uint32_t)tile[c + 2 * e][d] | ((uint32_t)tile[c + 2 * e + 1][d] << 16);
    *reinterpret_cast<uint4*>(dst + (int64_t)d * a.seq_pad + c) = o;
  }
}

// ===========================================================================
// Attention backward, dK and dV.  A block owns 128 keys of one (batch, head),
// 32 per wave; each wave keeps its K and V rows as MFMA operands in registers
// and walks all queries in tiles of 32, staged in LDS (Q and dO rows with bits
// 2 and 3 of the row index swapped, so that the accumulator registers of S and
// dP hold 8 consecutive queries per 16-query step; Q^T and dO^T in natural
// order).  Per tile: S = Q K^T, dP = dO V^T, P = exp2(S sc - lse),
// dS = P (dP - Dv); dV^T += dO^T P, dK^T += Q^T dS (scaled by 1/sqrt(Dh) at
// the store).  Scores of padded queries vanish (lse = +inf there).
// ===========================================================================
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_bwd_dkdv_kernel(AttnBwdArgs a) {
  constexpr int DH = 128, KS = DH / 16, DT = DH / 32, QT = 32;
  constexpr int RLD = DH + 8, TLD = QT + 8;
  __shared__ __attribute__((aligned(16))) bf16_t Qs[2][QT * RLD];
  __shared__ __attribute__((aligned(16))) bf16_t dOs[2][QT * RLD];
  __shared__ __attribute__((aligned(16))) bf16_t Qts[2][DH * TLD];
  __shared__ __attribute__((aligned(16))) bf16_t dOts[2][DH * TLD];
  __shared__ __attribute__((aligned(16))) float lse_s[2][QT];
  __shared__ __attribute__((aligned(16))) float dd_s[2][QT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.heads + h;
  const int key = blockIdx.x * 128 + wave * 32 + l32;
  const bf16_t* Qh = reinterpret_cast<const bf16_t*>(a.qh) + bh * a.seq_pad * DH;
  const bf16_t* Qt = reinterpret_cast<const bf16_t*>(a.qt) + bh * DH * a.seq_pad;
  const bf16_t* dOh = reinterpret_cast<const bf16_t*>(a.doh) + bh * a.seq_pad * DH;
  const bf16_t* dOt = reinterpret_cast<const bf16_t*>(a.dot) + bh * DH * a.seq_pad;
  const float* lse = a.lse + bh * a.seq_pad;
  const float* dd = a.dd + bh * a.seq_pad;
  bf16x8_t kf[KS], vf[KS];
  {
    const bf16_t* Kr = reinterpret_cast<const bf16_t*>(a.kh) + (bh * a.seq_pad + key) * DH;
    const bf16_t* Vr = reinterpret_cast<const bf16_t*>(a.vh) + (bh * a.seq_pad + key) * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = *reinterpret_cast<const bf16x8_t*>(Kr + ks * 16 + half * 8);
      vf[ks] = *reinterpret_cast<const bf16x8_t*>(Vr + ks * 16 + half * 8);
    }
  }
  f32x16_t acc_dv[DT], acc_dk[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc_dv[i][e] = acc_dk[i][e] = 0.f;
  const float sc = a.scale_log2;
  // staging of one query tile: 2 chunks each of Q rows, dO rows, Q^T, dO^T
  u32x4_t rq[2], rdo[2], rqt[2], rdot[2];
  float4 rl = make_float4(0.f, 0.f, 0.f, 0.f);
  auto gload = [&](int t) {
    const int q0 = t * QT;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 4, c = (idx & 15) * 8;        // row tiles: 32 rows x 16 chunks
      rq[i] = *reinterpret_cast<const u32x4_t*>(Qh + (int64_t)(q0 + r) * DH + c);
      rdo[i] = *reinterpret_cast<const u32x4_t*>(dOh + (int64_t)(q0 + r) * DH + c);
      const int d = idx >> 2, cq = (idx & 3) * 8;         // transposed tiles: 128 rows x 4 chunks
      rqt[i] = *reinterpret_cast<const u32x4_t*>(Qt + (int64_t)d * a.seq_pad + q0 + cq);
      rdot[i] = *reinterpret_cast<const u32x4_t*>(dOt + (int64_t)d * a.seq_pad + q0 + cq);
    }
    if (tid < 8) rl = *reinterpret_cast<const float4*>(lse + q0 + tid * 4);
    else if (tid < 16) rl = *reinterpret_cast<const float4*>(dd + q0 + (tid - 8) * 4);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 4, c = (idx & 15) * 8;
      const int rho = swap23b(r);
      *reinterpret_cast<u32x4_t*>(&Qs[buf][rho * RLD + c]) = rq[i];
      *reinterpret_cast<u32x4_t*>(&dOs[buf][rho * RLD + c]) = rdo[i];
      const int d = idx >> 2, cq = (idx & 3) * 8;
      *reinterpret_cast<u32x4_t*>(&Qts[buf][d * TLD + cq]) = rqt[i];
      *reinterpret_cast<u32x4_t*>(&dOts[buf][d * TLD + cq]) = rdot[i];
    }
    if (tid < 8) *reinterpret_cast<float4*>(&lse_s[buf][tid * 4]) = rl;
    else if (tid < 16) *reinterpret_cast<float4*>(&dd_s[buf][(tid - 8) * 4]) = rl;
  };
  const int ntiles = (a.seq + QT - 1) / QT;
  gload(0);
  lstore(0);
  if (ntiles > 1) gload(1);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    f32x16_t s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(&Qs[buf][l32 * RLD + ks * 16 + half * 8]);
      const bf16x8_t da = *reinterpret_cast<const bf16x8_t*>(&dOs[buf][l32 * RLD + ks * 16 + half * 8]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[ks], dp, 0, 0, 0);
    }
    // element e of S / dP is query 16 (e / 8) + 8 half + e % 8 of the tile
    bf16x8_t pb[2], dsb[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const float4 l0 = *reinterpret_cast<const float4*>(&lse_s[buf][16 * st + 8 * half]);
      const float4 l1 = *reinterpret_cast<const float4*>(&lse_s[buf][16 * st + 8 * half + 4]);
      const float4 d0 = *reinterpret_cast<const float4*>(&dd_s[buf][16 * st + 8 * half]);
      const float4 d1 = *reinterpret_cast<const float4*>(&dd_s[buf][16 * st + 8 * half + 4]);
      const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
      const float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
      uint32_t wp[4], wd[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int e = 8 * st + 2 * e2;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], sc, -lv[2 * e2]));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e + 1], sc, -lv[2 * e2 + 1]));
        wp[e2] = pack_bf16x2(p0, p1);
        wd[e2] = pack_bf16x2(p0 * (dp[e] - dv[2 * e2]), p1 * (dp[e + 1] - dv[2 * e2 + 1]));
      }
      const u32x4_t vp = {wp[0], wp[1], wp[2], wp[3]}, vd = {wd[0], wd[1], wd[2], wd[3]};
      pb[st] = __builtin_bit_cast(bf16x8_t, vp);
      dsb[st] = __builtin_bit_cast(bf16x8_t, vd);
    }
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8_t ot = *reinterpret_cast<const bf16x8_t*>(&dOts[buf][(i * 32 + l32) * TLD + st * 16 + half * 8]);
        const bf16x8_t qt = *reinterpret_cast<const bf16x8_t*>(&Qts[buf][(i * 32 + l32) * TLD + st * 16 + half * 8]);
        acc_dv[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ot, pb[st], acc_dv[i], 0, 0, 0);
        acc_dk[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt, dsb[st], acc_dk[i], 0, 0, 0);
      }
    if (t + 1 < ntiles) lstore(buf ^ 1);
    if (t + 2 < ntiles) gload(t + 2);
    __syncthreads();
  }
  if (key < a.seq) {
    const float scale = a.scale;
    float* dK = a.dk + (bh * a.seq_pad + key) * DH;
    float* dV = a.dv + (bh * a.seq_pad + key) * DH;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = i * 32 + 8 * j + 4 * half;
        *reinterpret_cast<float4*>(dV + d) =
            make_float4(acc_dv[i][4 * j], acc_dv[i][4 * j + 1], acc_dv[i][4 * j + 2], acc_dv[i][4 * j + 3]);
        *reinterpret_cast<float4*>(dK + d) = make_float4(acc_dk[i][4 * j] * scale, acc_dk[i][4 * j + 1] * scale,
                                                         acc_dk[i][4 * j + 2] * scale, acc_dk[i][4 * j + 3] * scale);
      }
  }
}

// ===========================================================================
// Attention backward, dQ.  A block owns 128 queries of one (batch, head), 32
// per wave (Q and dO rows of the wave's queries as MFMA operands in
// registers), and walks all keys in tiles of 64 staged in LDS: K and V rows
// with bits 2 and 3 of the row index swapped within each 32-row half, K^T in
// natural order.  Per tile: S^T = K Q^T, dP^T = V dO^T, P^T = exp2(S^T sc -
// lse[q]) (zero for keys beyond seq), dS^T = P^T (dP^T - Dv[q]);
// dQ^T += K^T dS^T, scaled by 1/sqrt(Dh) at the store.
// ===========================================================================
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_bwd_dq_kernel(AttnBwdArgs a) {
  constexpr int DH = 128, KS = DH / 16, DT = DH / 32, KT = 64;
  constexpr int RLD = DH + 8, TLD = KT + 8;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][KT * RLD];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][KT * RLD];
  __shared__ __attribute__((aligned(16))) bf16_t Kts[2][DH * TLD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.heads + h;
  const int q = blockIdx.x * 128 + wave * 32 + l32;
  const bf16_t* Kh = reinterpret_cast<const bf16_t*>(a.kh) + bh * a.seq_pad * DH;
  const bf16_t* Vh = reinterpret_cast<const bf16_t*>(a.vh) + bh * a.seq_pad * DH;
  const bf16_t* Kt = reinterpret_cast<const bf16_t*>(a.kt) + bh * DH * a.seq_pad;
  bf16x8_t qf[KS], df[KS];
  {
    const bf16_t* Qr = reinterpret_cast<const bf16_t*>(a.qh) + (bh * a.seq_pad + q) * DH;
    const bf16_t* Dr = reinterpret_cast<const bf16_t*>(a.doh) + (bh * a.seq_pad + q) * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(Qr + ks * 16 + half * 8);
      df[ks] = *reinterpret_cast<const bf16x8_t*>(Dr + ks * 16 + half * 8);
    }
  }
  const float lq = a.lse[bh * a.seq_pad + q], dq_ = a.dd[bh * a.seq_pad + q];
  f32x16_t acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  const float sc = a.scale_log2;
  u32x4_t rk[4], rv[4], rt[4];
  auto gload = [&](int t) {
    const int k0 = t * KT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 4, c = (idx & 15) * 8;         // 64 rows x 16 chunks
      rk[i] = *reinterpret_cast<const u32x4_t*>(Kh + (int64_t)(k0 + r) * DH + c);
      rv[i] = *reinterpret_cast<const u32x4_t*>(Vh + (int64_t)(k0 + r) * DH + c);
      const int d = idx >> 3, ck = (idx & 7) * 8;         // 128 rows x 8 chunks
      rt[i] = *reinterpret_cast<const u32x4_t*>(Kt + (int64_t)d * a.seq_pad + k0 + ck);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 4, c = (idx & 15) * 8;
      const int rho = (r & 32) | swap23b(r & 31);
      *reinterpret_cast<u32x4_t*>(&Ks[buf][rho * RLD + c]) = rk[i];
      *reinterpret_cast<u32x4_t*>(&Vs[buf][rho * RLD + c]) = rv[i];
      const int d = idx >> 3, ck = (idx & 7) * 8;
      *reinterpret_cast<u32x4_t*>(&Kts[buf][d * TLD + ck]) = rt[i];
    }
  };
  const int ntiles = (a.seq + KT - 1) / KT;
  gload(0);
  lstore(0);
  if (ntiles > 1) gload(1);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    f32x16_t s[2] = {}, dp[2] = {};
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(&Ks[buf][(u * 32 + l32) * RLD + ks * 16 + half * 8]);
        const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(&Vs[buf][(u * 32 + l32) * RLD + ks * 16 + half * 8]);
        s[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[u], 0, 0, 0);
        dp[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[ks], dp[u], 0, 0, 0);
      }
    // element e of tile u is key t*64 + 16 (2u + e/8) + 8 half + e%8
    bf16x8_t dsb[4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t w[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int e = 8 * hh + 2 * e2;
          const int k = t * KT + 16 * (2 * u + hh) + 8 * half + 2 * e2;
          float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][e], sc, -lq));
          float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][e + 1], sc, -lq));
          if (k >= a.seq) p0 = 0.f;
          if (k + 1 >= a.seq) p1 = 0.f;
          w[e2] = pack_bf16x2(p0 * (dp[u][e] - dq_), p1 * (dp[u][e + 1] - dq_));
        }
        const u32x4_t v = {w[0], w[1], w[2], w[3]};
        dsb[2 * u + hh] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8_t kt = *reinterpret_cast<const bf16x8_t*>(&Kts[buf][(i * 32 + l32) * TLD + st * 16 + half * 8]);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, dsb[st], acc[i], 0, 0, 0);
      }
    if (t + 1 < ntiles) lstore(buf ^ 1);
    if (t + 2 < ntiles) gload(t + 2);
    __syncthreads();
  }
  if (q < a.seq) {
    const float scale = a.scale;
    float* dQ = a.dq + (bh * a.seq_pad + q) * DH;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(dQ + i * 32 + 8 * j + 4 * half) =
            make_float4(acc[i][4 * j] * scale, acc[i][4 * j + 1] * scale, acc[i][4 * j + 2] * scale,
                        acc[i][4 * j + 3] * scale);
  }
}

hipError_t launch_attention_bwd(const AttnBwdArgs& a, hipStream_t stream) {
  const double L = a.seq, work = 4.0 * a.batch * a.heads * L * L * 128.0;   // two products of L x L x Dh
  {
    TimingScope ts(kKcBwdElem, stream, (double)a.batch * a.seq * a.heads * 128.0 * 8.0);
    hipLaunchKernelGGL(attn_bwd_pre_kernel, dim3((unsigned)(a.seq_pad / 64), (unsigned)a.heads, (unsigned)a.batch),
                       dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(a.seq_pad / 128), (unsigned)a.heads, (unsigned)a.batch);
  // algorithmic work: five L x L x Dh products (S recomputed, dP, dV, dK, dQ),
  // 2.5 times the forward's two; the dQ kernel's second S and dP are overhead
  {
    TimingScope ts(kKcAttnBwd, stream, 2.0 * work);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel, grid, dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  TimingScope ts(kKcAttnBwd, stream, 0.5 * work);
  hipLaunchKernelGGL(attn_bwd_dq_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ===========================================================================
// adaLN modulation backward: m = W SiLU(vec) + b.  dW[r][c] = sum_b dm[b][r]
// SiLU(vec[b][c]), db[r] = sum_b dm[b][r] (fp32 outputs); the vec gradient's
// transposed GEMV W^T dm in row chunks (partials, reduced in order and
// multiplied by SiLU'(vec) into dvec).
// ===========================================================================
template <typename TW>
__global__ void __launch_bounds__(256) mod_dw_kernel(ModBwdArgs a) {
  const int64_t n4 = (int64_t)a.N * (a.K / 4);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const int r = (int)(i / (a.K / 4)), c = (int)(i % (a.K / 4)) * 4;
    float s[4] = {0.f, 0.f, 0.f, 0.f}, sb = 0.f;
    for (int b = 0; b < a.batch; ++b) {
      const float g = a.dm[(int64_t)b * a.dm_bstride + r];
      const float4 v = *reinterpret_cast<const float4*>(a.vec + (int64_t)b * a.K + c);
      if (a.silu_in) {
        s[0] += g * silu_f(v.x); s[1] += g * silu_f(v.y); s[2] += g * silu_f(v.z); s[3] += g * silu_f(v.w);
      } else {
        s[0] += g * v.x; s[1] += g * v.y; s[2] += g * v.z; s[3] += g * v.w;
      }
      sb += g;
    }
    *reinterpret_cast<float4*>(a.dw + (int64_t)r * a.K + c) = make_float4(s[0], s[1], s[2], s[3]);
    if (c == 0) a.db[r] = sb;
  }
}

template <typename TW>
__global__ void __launch_bounds__(256) mod_dvec_partial_kernel(ModBwdArgs a) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4, rc = blockIdx.y;
  if (c >= a.K) return;
  const int r0 = rc * a.rpc, r1 = min(a.N, r0 + a.rpc);
  const TW* W = reinterpret_cast<const TW*>(a.w);
  for (int b = 0; b < a.batch; ++b) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    const float* g = a.dm + (int64_t)b * a.dm_bstride;
    for (int r = r0; r < r1; ++r) {
      const float gr = g[r];
      if constexpr (sizeof(TW) == 4) {
        const float4 w = *reinterpret_cast<const float4*>(W + (int64_t)r * a.K + c);
        s[0] += w.x * gr; s[1] += w.y * gr; s[2] += w.z * gr; s[3] += w.w * gr;
      } else {
        const uint2 w = *reinterpret_cast<const uint2*>(W + (int64_t)r * a.K + c);
        s[0] += __uint_as_float(w.x << 16) * gr; s[1] += __uint_as_float(w.x & 0xffff0000u) * gr;
        s[2] += __uint_as_float(w.y << 16) * gr; s[3] += __uint_as_float(w.y & 0xffff0000u) * gr;
      }
    }
    *reinterpret_cast<float4*>(a.part + ((int64_t)b * gridDim.y + rc) * a.K + c) = make_float4(s[0], s[1], s[2], s[3]);
  }
}

hipError_t launch_mod_bwd(ModBwdArgs a, int w_dtype, hipStream_t stream) {
  {
    const int64_t n4 = (int64_t)a.N * (a.K / 4);
    int64_t blocks = ceil_div(n4, 256);
    if (blocks > 8192) blocks = 8192;
    TimingScope ts(kKcBwdElem, stream, 4.0 * (double)a.N * a.K);
    if (w_dtype == kF32) hipLaunchKernelGGL(mod_dw_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(mod_dw_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!a.dvec) return hipSuccess;   // no input gradient wanted
  const int nrc = a.nrc;
  a.rpc = (int)ceil_div(a.N, nrc);
  {
    TimingScope ts(kKcBwdElem, stream, (double)a.batch * a.N * a.K * (w_dtype == kF32 ? 4.0 : 2.0));
    const dim3 grid((unsigned)ceil_div(a.K, 1024), (unsigned)nrc);
    if (w_dtype == kF32) hipLaunchKernelGGL(mod_dvec_partial_kernel<float>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(mod_dvec_partial_kernel<bf16_t>, grid, dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ReduceArgs r{};
  r.part = a.part; r.np = nrc; r.C = a.K; r.Z = a.batch;
  r.out = a.dvec; r.out_zstride = a.K; r.mode = a.dvec_store ? 3 : 2; r.aux = a.vec; r.aux_zstride = a.K;
  return launch_reduce(r, stream);
}

// ===========================================================================
// Gradient of the velocity MSE J = mean((v_pred - (z1 - z0))^2) over all
// n elements: dv = (2 / n) (v_pred - v*), v* = z1 - z0 rounded to fp32 as
// the forward's target.
// ===========================================================================
__global__ void __launch_bounds__(256) rf_loss_grad_kernel(const float* v, const float* z0, const float* z1, float* dv,
                                                           int64_t n, float c) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float tgt = z1[i] - z0[i];
    dv[i] = c * (v[i] - tgt);
  }
}

hipError_t launch_rf_loss_grad(const float* v, const float* z0, const float* z1, float* dv, int64_t n,
                               hipStream_t stream) {
  int64_t blocks = ceil_div(n > 0 ? n : 1, 256);
  if (blocks > 4096) blocks = 4096;
  TimingScope ts(kKcRf, stream, 16.0 * (double)n);
  hipLaunchKernelGGL(rf_loss_grad_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, v, z0, z1, dv, n,
                     (float)(2.0 / (double)n));
  return hipGetLastError();
}

// Gradient of the guidance embedding, a Linear 1 -> D of the guidance value
// g_b added to vec ("Flux architecture deep dive", Conditioning):
// dW[d] = sum_b g_b dvec[b, d], db[d] = sum_b dvec[b, d], summed over b in
// order (one thread per d).
__global__ void __launch_bounds__(256) guidance_bwd_kernel(const float* __restrict__ dvec,
                                                           const float* __restrict__ g, int batch, int D,
                                                           float* __restrict__ dw, float* __restrict__ db) {
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= D) return;
  float sw = 0.f, sb = 0.f;
  for (int b = 0; b < batch; ++b) {
    const float v = dvec[(int64_t)b * D + d];
    sw = fmaf(g[b], v, sw);
    sb += v;
  }
  dw[d] = sw;
  db[d] = sb;
}

hipError_t launch_guidance_bwd(const float* dvec, const float* g, int batch, int D, float* dw, float* db,
                               hipStream_t stream) {
  TimingScope ts(kKcBwdElem, stream, (double)batch * D * 4.0 + D * 8.0);
  hipLaunchKernelGGL(guidance_bwd_kernel, dim3((unsigned)ceil_div(D, 256)), dim3(256), 0, stream, dvec, g, batch, D,
                     dw, db);
  return hipGetLastError();
}

}  // namespace flux
