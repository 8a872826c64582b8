// GEMM C = A W^T (+ bias, fused epilogues) for the Flux block linears
// ("Flux architecture deep dive", MMDiT layer / Flux single block: the qkv,
// output-projection and MLP linears; "Flux model API reference", add_qkv_bias).
//
// 16-bit operand paths, fp32 accumulation on 32x32x16 MFMA; operands bf16 x
// bf16, fp16 activations x bf16 weights converted to fp16 in the kernel (exact
// in fp16's normal range), or fp16 x fp16.  E4M3 x E4M3 operands run on the
// 32x32x64 fp8 MFMA (gemm_fp8r_kernel; the MX formats on gemm_fp8_kernel),
// small E4M3 problems on the 128 x 128 kernel after an exact widening to fp16.  A and W are both K-contiguous (torch
// Linear layout).  Several problems (the image and text streams of a double
// block) share one grid; the tile order keeps each XCD on a contiguous tile
// range and walks tiles in groups of 4 tile rows so A and W panels are reused
// from L2.
//  * large problems: gemm_dl_kernel, persistent (one 256-thread block per CU),
//    256 x 256 tiles; operands loaded global -> LDS directly in k = 64
//    super-stages (a ring of five 32 KB operand halves), MFMA fragment reads
//    and loads interleaved one-by-one with the MFMAs; the next tile's first
//    loads overlap the current epilogue;
//  * small problems: gemm_mfma_kernel, 128 x 128 tiles, register-staged
//    double buffer.
// fp32 path (fp32 workloads only): LDS-tiled FMA kernel with the same epilogues.
#include <type_traits>

#include <atomic>

#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace flux {

// ---------------------------------------------------------------------------
// epilogue
// ---------------------------------------------------------------------------
struct EpiRow {
  char* o0;
  char* o1;
  const float* gate;
  bool valid;
};

__device__ __forceinline__ EpiRow epi_row(const GemmProblem& p, int row, int elem_bytes) {
  EpiRow r;
  r.valid = row < p.M;
  const int rr = r.valid ? row : 0;
  const int64_t b = rr / p.omap0.seg, l = rr % p.omap0.seg;
  const int ob = (p.epi == kEpiResid || p.epi == kEpiStoreF32) ? 4 : elem_bytes;
  r.o0 = reinterpret_cast<char*>(p.out0) + (b * p.omap0.bstride + l * p.omap0.ld) * ob;
  r.gate = p.gate ? p.gate + b * p.gate_bstride : nullptr;
  r.o1 = nullptr;
  if (p.epi == kEpiSplitGelu) {
    const int64_t b1 = rr / p.omap1.seg, l1 = rr % p.omap1.seg;
    r.o1 = reinterpret_cast<char*>(p.out1) + (b1 * p.omap1.bstride + l1 * p.omap1.ld) * elem_bytes;
  }
  return r;
}

template <typename T>
__device__ __forceinline__ void epi_apply(const GemmProblem& p, const EpiRow& r, int col, float v) {
  switch (p.epi) {
    case kEpiStore:
      reinterpret_cast<T*>(r.o0)[col] = from_f32<T>(v);
      break;
    case kEpiGelu:
      reinterpret_cast<T*>(r.o0)[col] = from_f32<T>(gelu_f(v));
      break;
    case kEpiResid: {
      float* x = reinterpret_cast<float*>(r.o0) + col;
      *x = *x + r.gate[col] * v;
      break;
    }
    case kEpiStoreF32:
      reinterpret_cast<float*>(r.o0)[(int64_t)col * p.col_stride0] = v;
      break;
    case kEpiSplitGelu:
      if (col < p.n_split)
        reinterpret_cast<T*>(r.o0)[col] = from_f32<T>(v);
      else
        reinterpret_cast<T*>(r.o1)[col - p.n_split] = from_f32<T>(gelu_f(v));
      break;
    default:
      break;
  }
}

// Four values as 16-bit elements of type dt (kBF16 or kF16), packed.
__device__ __forceinline__ uint2 pack4(float4 v, int dt) {
  uint2 o;
  if (dt == kF16) {
    o.x = pack_f16x2(v.x, v.y);
    o.y = pack_f16x2(v.z, v.w);
  } else {
    o.x = pack_bf16x2(v.x, v.y);
    o.y = pack_bf16x2(v.z, v.w);
  }
  return o;
}

// Four values as E4M3 bytes (scale qs), and their largest magnitude into mx.
__device__ __forceinline__ uint32_t pack4_e4m3(float4 v, float qs, uint32_t& mx) {
  mx = max(mx, max(max(abs_bits(v.x), abs_bits(v.y)), max(abs_bits(v.z), abs_bits(v.w))));
  return f32x4_to_e4m3(v.x * qs, v.y * qs, v.z * qs, v.w * qs);
}

// Store four values of a 16-bit or E4M3 output whose element offset is off.
__device__ __forceinline__ void store4_dt(void* base, int64_t off, int dt, float4 v, float qs, uint32_t& mx) {
  if (dt == kFP8)
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(base) + off) = pack4_e4m3(v, qs, mx);
  else
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(base) + off) = pack4(v, dt);
}

// Four consecutive columns col..col+3 of one row (MFMA kernels).  N is a
// multiple of 4, so the four columns are all in range together; for the
// split epilogue n_split is a multiple of 4, so they fall on one side.
// dq multiplies the accumulator first (the product of the two operand
// scale_inv for E4M3 operands, else 1); qs is the E4M3 output scale and mx
// collects the largest magnitude written as E4M3.  EPI is the epilogue kind,
// fixed at compile time so a kernel carries the code of one kind only.
template <int EPI>
__device__ __forceinline__ void epi_apply4(const GemmProblem& p, int row, int col, float4 v, float dq, float qs,
                                           uint32_t& mx) {
  v.x *= dq; v.y *= dq; v.z *= dq; v.w *= dq;
  if (p.bias) {
    const uint2 bb = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(p.bias) + col);
    v.x += __uint_as_float(bb.x << 16);
    v.y += __uint_as_float(bb.x & 0xffff0000u);
    v.z += __uint_as_float(bb.y << 16);
    v.w += __uint_as_float(bb.y & 0xffff0000u);
  }
  const int64_t b = row / p.omap0.seg, l = row % p.omap0.seg;
  const int64_t off0 = b * p.omap0.bstride + l * p.omap0.ld;
  if constexpr (EPI == kEpiStore || EPI == kEpiGelu) {
    if constexpr (EPI == kEpiGelu) {
      v.x = gelu_f(v.x); v.y = gelu_f(v.y); v.z = gelu_f(v.z); v.w = gelu_f(v.w);
    }
    store4_dt(p.out0, off0 + col, p.out0_dt, v, qs, mx);
  } else if constexpr (EPI == kEpiResid) {
    float4* x = reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out0) + off0 + col);
    const float4 g = *reinterpret_cast<const float4*>(p.gate + b * p.gate_bstride + col);
    float4 r = *x;
    r.x += g.x * v.x; r.y += g.y * v.y; r.z += g.z * v.z; r.w += g.w * v.w;
    *x = r;
  } else if constexpr (EPI == kEpiStoreF32) {
    float* o = reinterpret_cast<float*>(p.out0) + off0;
    if (p.col_stride0 == 1) {
      *reinterpret_cast<float4*>(o + col) = v;
    } else {
      o[(int64_t)col * p.col_stride0] = v.x;
      o[(int64_t)(col + 1) * p.col_stride0] = v.y;
      o[(int64_t)(col + 2) * p.col_stride0] = v.z;
      o[(int64_t)(col + 3) * p.col_stride0] = v.w;
    }
  } else if constexpr (EPI == kEpiSplitGelu) {
    if (col < p.n_split) {
      store4_dt(p.out0, off0 + col, p.out0_dt, v, qs, mx);
    } else {
      const int64_t b1 = row / p.omap1.seg, l1 = row % p.omap1.seg;
      v.x = gelu_f(v.x); v.y = gelu_f(v.y); v.z = gelu_f(v.z); v.w = gelu_f(v.w);
      store4_dt(p.out1, b1 * p.omap1.bstride + l1 * p.omap1.ld + (col - p.n_split), p.out1_dt, v, qs, mx);
    }
  }
}

// The same with the kind read at run time (the small-problem kernel).
__device__ __forceinline__ void epi_apply4_any(const GemmProblem& p, int row, int col, float4 v, float dq, float qs,
                                               uint32_t& mx) {
  switch (p.epi) {
    case kEpiStore: epi_apply4<kEpiStore>(p, row, col, v, dq, qs, mx); break;
    case kEpiGelu: epi_apply4<kEpiGelu>(p, row, col, v, dq, qs, mx); break;
    case kEpiResid: epi_apply4<kEpiResid>(p, row, col, v, dq, qs, mx); break;
    case kEpiStoreF32: epi_apply4<kEpiStoreF32>(p, row, col, v, dq, qs, mx); break;
    case kEpiSplitGelu: epi_apply4<kEpiSplitGelu>(p, row, col, v, dq, qs, mx); break;
    default: break;
  }
}

// ---------------------------------------------------------------------------
// tile scheduling shared by both paths
// ---------------------------------------------------------------------------
struct TileCoord {
  int prob, tm, tn;
};

// Tile coordinates of tile id (problem, then groups of kGroupM tile rows
// walked column by column, so consecutive ids share operand panels).
__device__ __forceinline__ TileCoord tile_coord(const GemmBatch& bt, int id, int BM, int BN) {
  TileCoord c;
  c.prob = (bt.count > 1 && id >= bt.p[1].tile_begin) ? 1 : 0;
  const int local = id - (c.prob ? bt.p[1].tile_begin : bt.p[0].tile_begin);
  const int tiles_m = (int)ceil_div(c.prob ? bt.p[1].M : bt.p[0].M, BM);
  const int tiles_n = c.prob ? bt.p[1].tiles_n : bt.p[0].tiles_n;
  constexpr int kGroupM = 4;
  const int group = kGroupM * tiles_n;
  const int g = local / group;
  const int first_m = g * kGroupM;
  const int gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int in = local % group;
  c.tm = first_m + in % gm;
  c.tn = in / gm;
  return c;
}

// Blocks are dispatched round-robin over the 8 XCDs (block i -> XCD i % 8);
// XCD x gets the contiguous tile-id range [x*q + min(x, r), ...) of
// xcd_tiles(x) ids, walked by its blocks i = bid / 8 in order.
__device__ __forceinline__ int xcd_first(int total, int x) {
  const int q = total / 8, rem = total % 8;
  return x * q + (x < rem ? x : rem);
}
__device__ __forceinline__ int xcd_tiles(int total, int x) { return total / 8 + (x < total % 8 ? 1 : 0); }

__device__ __forceinline__ TileCoord decode_tile_id(const GemmBatch& bt, int bid, int BM, int BN) {
  return tile_coord(bt, xcd_first(bt.total_tiles, bid % 8) + bid / 8, BM, BN);
}

__device__ __forceinline__ TileCoord decode_tile(const GemmBatch& bt, int BM, int BN) {
  return decode_tile_id(bt, blockIdx.x, BM, BN);
}

// Accumulator multiplier of a problem: scale_inv of both E4M3 operand records,
// 1 for 16-bit operands.
__device__ __forceinline__ float epi_dequant(const GemmProblem& p) {
  return p.qa ? fp8_scale_inv(p.qa) * fp8_scale_inv(p.qw) : 1.0f;
}
__device__ __forceinline__ float epi_out_scale(const GemmProblem& p) { return p.qo ? fp8_scale(p.qo) : 1.0f; }
// Raise the output record's amax once per wave (every lane calls).
__device__ __forceinline__ void epi_amax_flush(const GemmProblem& p, uint32_t mx) {
  mx = wave_max_u32(mx);
  if (p.qo && (threadIdx.x & 63) == 0 && mx) fp8_amax_raise(p.qo, __uint_as_float(mx));
}

// ---------------------------------------------------------------------------
// 16-bit MFMA kernel (also the small-problem path of E4M3 operands, widened
// exactly to fp16 on their way into LDS)
// ---------------------------------------------------------------------------
constexpr int kBK = 64;   // K per stage: 64 bf16 = 128 bytes = 8 chunks of 16 bytes per row
// LDS rows padded to 144 bytes: 16 consecutive rows read at one chunk hit 16
// distinct 4-bank groups (conflict-free for 32 or 64 banks) and all fragment
// addresses are a per-lane base plus immediates.
constexpr int kLdsLd = kBK + 8;

// LDS element offset of chunk `c` (0..7) of tile row `row`.
__device__ __forceinline__ int lds_off(int row, int c) { return row * kLdsLd + (c << 3); }

template <int BM, int BN, int OP>
__global__ void __launch_bounds__(256, 1) gemm_mfma_kernel(GemmBatch bt) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int LA = BM / 32, LB = BN / 32;      // 16-byte loads per thread per stage
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * kLdsLd];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * kLdsLd];

  const TileCoord tc = decode_tile(bt, BM, BN);
  // select by value: a dynamically indexed kernel-argument array would be
  // copied to scratch memory
  GemmProblem p = bt.p[0];
  if (tc.prob) p = bt.p[1];
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // split-K: blockIdx.y takes k range [split * K / ksplit, ...) and writes an
  // fp32 partial tile; gemm_splitk_reduce_kernel sums them in order
  const int split = blockIdx.y;
  const int kspan = p.K / bt.ksplit;

  // global row pointers of this thread's loads (rows clamped into range);
  // each thread moves 8 elements (one 16-byte LDS chunk) per row and stage
  constexpr int ES = OP == kFP8 ? 1 : 2;          // operand bytes per element in memory
  const char* arow[LA];
  const char* brow[LB];
  const int lrow = tid >> 3, lchunk = tid & 7;
  {
    const char* A = reinterpret_cast<const char*>(p.A);
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      int r = m0 + i * 32 + lrow;
      r = r < p.M ? r : p.M - 1;
      arow[i] = A + ((int64_t)(r / p.amap.seg) * p.amap.bstride + (int64_t)(r % p.amap.seg) * p.amap.ld + lchunk * 8 +
                     (int64_t)split * kspan) * ES;
    }
    const char* W = reinterpret_cast<const char*>(p.W);
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      int r = n0 + i * 32 + lrow;
      r = r < p.N ? r : p.N - 1;
      brow[i] = W + ((int64_t)r * p.ldw + lchunk * 8 + (int64_t)split * kspan) * ES;
    }
  }
  u32x4_t ra[LA], rb[LB];
  auto gload = [&](int k0) {
    if constexpr (OP == kFP8) {
#pragma unroll
      for (int i = 0; i < LA; ++i) ra[i] = e4m3x8_to_f16x8(*reinterpret_cast<const uint2*>(arow[i] + k0));
#pragma unroll
      for (int i = 0; i < LB; ++i) rb[i] = e4m3x8_to_f16x8(*reinterpret_cast<const uint2*>(brow[i] + k0));
    } else {
#pragma unroll
      for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(arow[i] + (int64_t)k0 * 2);
#pragma unroll
      for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(brow[i] + (int64_t)k0 * 2);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4_t*>(&As[buf][lds_off(i * 32 + lrow, lchunk)]) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i)
      *reinterpret_cast<u32x4_t*>(&Bs[buf][lds_off(i * 32 + lrow, lchunk)]) =
          OP == kF16 ? bf16x8_to_f16x8(rb[i]) : rb[i];   // kF16W, kFP8: already fp16
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Pipeline: tile k+1 sits in registers (loaded during iteration k-1) and is
  // written to the idle LDS buffer at the start of iteration k, then the
  // global loads of tile k+2 are issued; the MFMAs of tile k read the other
  // buffer with their 16-wide k slices double-buffered in registers, so the
  // LDS reads of slice kk+1 overlap the MFMAs of slice kk.  One barrier per
  // iteration separates the buffer swap.
  const int KT = kspan / kBK;
  const int frow = lane & 31, fhalf = lane >> 5;
  gload(0);
  lstore(0);
  if (KT > 1) gload(kBK);
  __syncthreads();
  u32x4_t af[2][TM], bfr[2][TN];
  auto lfrag = [&](int buf, int s, int kk) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af[s][i] = *reinterpret_cast<const u32x4_t*>(&As[buf][lds_off(wm * WM + i * 32 + frow, kk * 2 + fhalf)]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bfr[s][j] = *reinterpret_cast<const u32x4_t*>(&Bs[buf][lds_off(wn * WN + j * 32 + frow, kk * 2 + fhalf)]);
  };
  auto mma = [&](int s) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (OP == kF16 || OP == kF16W || OP == kFP8)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, af[s][i]),
                                                            __builtin_bit_cast(f16x8_t, bfr[s][j]), acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[s][i]),
                                                             __builtin_bit_cast(bf16x8_t, bfr[s][j]), acc[i][j], 0, 0, 0);
      }
  };
  // sched_barrier(0) fences keep the compiler from sinking the fragment
  // prefetches back next to their MFMAs
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) lstore(cur ^ 1);
    if (kt + 2 < KT) gload((kt + 2) * kBK);
    lfrag(cur, 0, 0);
    lfrag(cur, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    lfrag(cur, 0, 2);
    __builtin_amdgcn_sched_barrier(0);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
    lfrag(cur, 1, 3);
    __builtin_amdgcn_sched_barrier(0);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    mma(1);
    __syncthreads();
  }

  // Epilogue.  Accumulator element e of lane l sits at row 8*(e/4) + 4*(l/32)
  // + e%4, column l%32 of its 32 x 32 tile.  Each 32-row slab of a wave's
  // tile goes through LDS (reusing the operand buffers) so the fused epilogue
  // then runs on 4 consecutive columns per lane with vector loads and stores.
  constexpr int CLD = WN + 4;
  float* cs = reinterpret_cast<float*>(&As[0][0]) + wave * 32 * CLD;
  const float dq = epi_dequant(p), qs = epi_out_scale(p);
  uint32_t mx = 0;
  static_assert(4 * 32 * CLD * 4 <= 2 * BM * kLdsLd * 2, "epilogue staging must fit in the A buffers");
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) cs[(8 * (e >> 2) + 4 * fhalf + (e & 3)) * CLD + j * 32 + frow] = acc[i][j][e];
    __syncthreads();
    constexpr int LPR = WN / 4;              // lanes per slab row
    constexpr int RPI = 64 / LPR;            // slab rows per wave step
    const int c4 = (lane % LPR) * 4;
    const int col = n0 + wn * WN + c4;
#pragma unroll 2
    for (int rr = lane / LPR; rr < 32; rr += RPI) {
      const int row = m0 + wm * WM + i * 32 + rr;
      if (row < p.M && col < p.N) {
        float4 v = *reinterpret_cast<const float4*>(&cs[rr * CLD + c4]);
        if (bt.ksplit > 1) {
          v.x *= dq; v.y *= dq; v.z *= dq; v.w *= dq;
          *reinterpret_cast<float4*>(bt.partials + ((int64_t)split * p.M + row) * p.N + col) = v;
        } else {
          epi_apply4_any(p, row, col, v, dq, qs, mx);
        }
      }
    }
    __syncthreads();
  }
  epi_amax_flush(p, mx);
}

// ---------------------------------------------------------------------------
// 256 x 256 tile, 4-stage LDS ring fed by direct global->LDS loads
// ---------------------------------------------------------------------------
constexpr int kDlBK = 32;                 // k per stage
constexpr int kDlStages = 5;
constexpr int kDlRows = 256;              // BM = BN
constexpr int kDlStageBytes = 2 * kDlRows * kDlBK * 2;   // A + B, 32 KB

// Stage layout: rows of 64 bytes (4 chunks of 16 B), A rows 0..255 then B rows
// 0..255.  Logical chunk c of row r sits at physical chunk c ^ ((r >> 2) & 3).
// gfx950 serves a 16-byte-per-lane LDS read in four cycles of 16 lanes each
// (64 banks of 4 bytes); measured on MI355X with the LDS bank-conflict
// counter, the lanes of one cycle are those with equal lane bit 5 and equal
// (bit 4 xor bit 2).  A fragment read (lane l -> row l % 32, chunk c or c+1)
// then hits 16 distinct 4-bank groups in every cycle: rows r and r + 16 of one
// cycle differ in (r >> 2) & 3 or in r % 4.  The global->LDS fill (lane l ->
// row l / 4, a whole 64-byte row per 4 lanes) is conflict-free for any
// in-row permutation.
__device__ __forceinline__ int dl_swz(int r) { return (r >> 2) & 3; }

// Epilogue of one 256 x 256 tile of the persistent kernels.  Each wave owns a
// 128 x 128 block of 4 x 4 accumulator tiles; its 8 quarters (32 rows x 64
// columns) pass one at a time through the wave's 8 KB of LDS staging
// (accumulator element e of lane l in a 32x32 tile is row 8*(e/4) +
// 4*(l/32) + e%4, column l%32), then 4 consecutive columns per lane go
// through the fused epilogue.  The quarter loop is not unrolled: only the
// staging (constant register indices) is replicated, so the kernel's code
// stays small enough for the instruction cache.
template <int Q>
__device__ __forceinline__ void stage_quarter(const f32x16_t (&acc)[4][4], float* cs, int frow, int fhalf) {
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int e = 0; e < 16; ++e) cs[(8 * (e >> 2) + 4 * fhalf + (e & 3)) * 64 + jj * 32 + frow] = acc[Q >> 1][2 * (Q & 1) + jj][e];
}

// Stream-K hand-over at the staged-quarter level (the wave's quarters Q =
// 0..7 as stage_quarter lays them out, 2048 floats each, at wave region + Q *
// 2048 of a block's slot).  A contributor (out set) copies each staged quarter
// to its slot and writes no output; an owner (nin > 0) adds, in block order,
// the staged quarters of the contributors whose bit is set in mask, before
// the epilogue reads them.  Returns true when the quarter's outputs are to be
// skipped.
struct SkIo {
  float* out;          // contributor: this wave's region of the block's slot
  const float* in;     // owner: this wave's region of the first contributor's slot
  int nin;             // owner: contributors (consecutive blocks, kGemmSkSlotFloats apart)
  uint32_t mask;       // owner: contributors whose sums arrived (the others were recomputed here)
};

// Partial sums cross compute units (and XCDs) through device-coherent
// accesses: 16-byte buffer stores and loads with the sc1 cache policy (coherent
// at device scope, so no L2 write-back or invalidate is needed); a
// contributor's stores have completed (vmcnt) before its flag is raised.
constexpr int kCpolDevice = 16;   // sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_rsrc(const float* region) {
  // a wave's 16384-float region of a slot
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(region), 0, 16384 * 4, 0x00020000);
}

__device__ __forceinline__ bool sk_quarter(float* cs, const SkIo& sk, int Q, int lane) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  float4* c4p = reinterpret_cast<float4*>(cs);
  if (sk.out) {
    const __amdgpu_buffer_rsrc_t r = sk_rsrc(sk.out);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, c4p[k * 64 + lane]), r,
                                             (Q * 512 + k * 64 + lane) * 16, 0, kCpolDevice);
    return true;
  }
  for (int c = 0; c < sk.nin; ++c) {
    if (!((sk.mask >> c) & 1u)) continue;
    const __amdgpu_buffer_rsrc_t r = sk_rsrc(sk.in + (int64_t)c * kGemmSkSlotFloats);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 v = __builtin_bit_cast(
          float4, __builtin_amdgcn_raw_buffer_load_b128(r, (Q * 512 + k * 64 + lane) * 16, 0, kCpolDevice));
      float4 w = c4p[k * 64 + lane];
      w.x += v.x; w.y += v.y; w.z += v.z; w.w += v.w;
      c4p[k * 64 + lane] = w;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the staged quarter is final
  return false;
}

// The residual rows (kEpiResid) of the lane's 8 rows rbase + 4u and four
// columns col..col+3 of a quarter, all loads issued together.
// Sample b and position l (row = b seg + l) of the rows rbase + 4u, u = 0..7,
// for segments of seg >= 32 rows: one division, then at most one wrap, since
// the eight rows span 29 consecutive rows.
__device__ __forceinline__ void seg_rows(int rbase, int seg, int (&b)[8], int (&l)[8]) {
  int bb = rbase / seg, ll = rbase - bb * seg;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    b[u] = bb;
    l[u] = ll;
    ll += 4;
    if (ll >= seg) {
      ll -= seg;
      ++bb;
    }
  }
}

__device__ __forceinline__ void load_resid(const GemmProblem& pc, int rbase, int col, float4 (&xr)[8]) {
  int sb[8], sl[8];
  seg_rows(rbase, pc.omap0.seg, sb, sl);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = rbase + 4 * u;
    xr[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < pc.M && col < pc.N)
      xr[u] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(pc.out0) +
                                               (int64_t)sb[u] * pc.omap0.bstride + (int64_t)sl[u] * pc.omap0.ld + col);
  }
}

// The fused epilogue of one staged quarter (32 rows x 64 columns, read from
// the wave's LDS staging cs) for the lane's 8 rows rbase + 4u and four
// columns col..col+3, whose bias bq and gate gq come in as values; xr holds
// the residual rows for kEpiResid (loaded a quarter ahead by the caller, so
// their latency overlaps the previous quarter).
template <int EPI>
__device__ __forceinline__ void apply_quarter(const GemmProblem& pc, const float* cs, int lrow, int c4, int rbase,
                                              int col, float4 bq, float4 gq, bool uniform, float dq, float qs,
                                              uint32_t& mx, const float4 (&xr)[8]) {
  const bool col_ok = col < pc.N;
  int sb[8], sl[8], sb1[8], sl1[8];
  seg_rows(rbase, pc.omap0.seg, sb, sl);
  if constexpr (EPI == kEpiSplitGelu) seg_rows(rbase, pc.omap1.seg, sb1, sl1);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = rbase + 4 * u;
    if (row < pc.M && col_ok) {
      const int64_t b = sb[u];
      const int64_t off0 = b * pc.omap0.bstride + (int64_t)sl[u] * pc.omap0.ld;
      float4 w = *reinterpret_cast<const float4*>(&cs[(lrow + 4 * u) * 64 + c4]);
      w.x = w.x * dq + bq.x; w.y = w.y * dq + bq.y;
      w.z = w.z * dq + bq.z; w.w = w.w * dq + bq.w;
      if constexpr (EPI == kEpiResid) {
        float4 g = gq;   // assigned in a branch: a conditional lvalue would put gq in scratch memory
        if (!uniform) g = *reinterpret_cast<const float4*>(pc.gate + b * pc.gate_bstride + col);
        float4 r = xr[u];
        r.x += g.x * w.x; r.y += g.y * w.y; r.z += g.z * w.z; r.w += g.w * w.w;
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(pc.out0) + off0 + col) = r;
      } else if constexpr (EPI == kEpiStore || EPI == kEpiGelu) {
        if constexpr (EPI == kEpiGelu) {
          w.x = gelu_f(w.x); w.y = gelu_f(w.y); w.z = gelu_f(w.z); w.w = gelu_f(w.w);
        }
        store4_dt(pc.out0, off0 + col, pc.out0_dt, w, qs, mx);
      } else if constexpr (EPI == kEpiStoreF32) {
        float* o = reinterpret_cast<float*>(pc.out0) + off0;
        if (pc.col_stride0 == 1) {
          *reinterpret_cast<float4*>(o + col) = w;
        } else {
          o[(int64_t)col * pc.col_stride0] = w.x;
          o[(int64_t)(col + 1) * pc.col_stride0] = w.y;
          o[(int64_t)(col + 2) * pc.col_stride0] = w.z;
          o[(int64_t)(col + 3) * pc.col_stride0] = w.w;
        }
      } else if constexpr (EPI == kEpiSplitGelu) {
        if (col < pc.n_split) {
          store4_dt(pc.out0, off0 + col, pc.out0_dt, w, qs, mx);
        } else {
          w.x = gelu_f(w.x); w.y = gelu_f(w.y); w.z = gelu_f(w.z); w.w = gelu_f(w.w);
          store4_dt(pc.out1, (int64_t)sb1[u] * pc.omap1.bstride + (int64_t)sl1[u] * pc.omap1.ld + (col - pc.n_split),
                    pc.out1_dt, w, qs, mx);
        }
      }
    }
  }
}

// The q|k|v projection straight into the attention layouts ("Flux model API
// reference", RMSNorm and EmbedND; "Flux architecture deep dive", 3D RoPE
// mathematics).  A wave's 128 columns are exactly one head of q, k or v.  Each
// 32-row strip is staged as its two 64-column halves; a lane then holds
// columns c4..c4+3 of both halves for 8 rows, so the RMSNorm sum over the
// head's 128 values is a 16-lane butterfly (fixed order), and the
// interleaved RoPE pairs (2m, 2m+1) are lane-local.  q and k rows are written
// head-major, v transposed, all in bf16.
__device__ __forceinline__ void qkv_epilogue(const GemmProblem& pc, const f32x16_t (&acc)[4][4], float* cs,
                                             int row0, int col0, int lane, float dq, const SkIo& sk) {
  if (col0 >= pc.N) return;                       // wave-uniform: no columns here
  const QkvOut& q = pc.qkv;
  const int frow = lane & 31, fhalf = lane >> 5;
  const int c4 = (lane & 15) * 4, lrow = lane >> 4;
  const int D = q.heads * 128;
  const int region = col0 / D;                    // 0 q, 1 k, 2 v (wave-uniform)
  const int h = (col0 - region * D) >> 7;
  float4 bA = make_float4(0.f, 0.f, 0.f, 0.f), bB = bA;
  if (pc.bias) {
    const uint2 ba = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(pc.bias) + col0 + c4);
    const uint2 bb = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(pc.bias) + col0 + 64 + c4);
    bA = make_float4(__uint_as_float(ba.x << 16), __uint_as_float(ba.x & 0xffff0000u), __uint_as_float(ba.y << 16),
                     __uint_as_float(ba.y & 0xffff0000u));
    bB = make_float4(__uint_as_float(bb.x << 16), __uint_as_float(bb.x & 0xffff0000u), __uint_as_float(bb.y << 16),
                     __uint_as_float(bb.y & 0xffff0000u));
  }
  float4 gA = make_float4(1.f, 1.f, 1.f, 1.f), gB = gA;
  const float* gm = region == 0 ? q.gq : q.gk;
  if (region < 2 && gm) {
    gA = *reinterpret_cast<const float4*>(gm + c4);
    gB = *reinterpret_cast<const float4*>(gm + 64 + c4);
  }
  bf16_t* dst = reinterpret_cast<bf16_t*>(region == 0 ? q.qh : q.kh);
  bf16_t* vt = reinterpret_cast<bf16_t*>(q.vt);
  const int seg = pc.omap0.seg;
  if (region == 2) {
    // v: each staged 32 x 64 quarter is read by columns (lane = head dim, a
    // conflict-free LDS row per step) and written transposed, 8 tokens per
    // 16-byte store, when the strip's 32 rows are 32 consecutive tokens of one
    // sample starting at a multiple of 8; otherwise element by element
    float bl0 = 0.f, bl1 = 0.f;   // bias of the lane's column in each half
    if (pc.bias) {
      const bf16_t* bp = reinterpret_cast<const bf16_t*>(pc.bias);
      bl0 = bf16_to_f32(bp[col0 + lane]);
      bl1 = bf16_to_f32(bp[col0 + 64 + lane]);
    }
#pragma unroll 1
    for (int Q = 0; Q < 8; ++Q) {
      switch (Q) {
        case 0: stage_quarter<0>(acc, cs, frow, fhalf); break;
        case 1: stage_quarter<1>(acc, cs, frow, fhalf); break;
        case 2: stage_quarter<2>(acc, cs, frow, fhalf); break;
        case 3: stage_quarter<3>(acc, cs, frow, fhalf); break;
        case 4: stage_quarter<4>(acc, cs, frow, fhalf); break;
        case 5: stage_quarter<5>(acc, cs, frow, fhalf); break;
        case 6: stage_quarter<6>(acc, cs, frow, fhalf); break;
        default: stage_quarter<7>(acc, cs, frow, fhalf); break;
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_sched_barrier(0);
      if (sk_quarter(cs, sk, Q, lane)) continue;
      const int half = Q & 1, r0 = row0 + (Q >> 1) * 32;
      const float bv = half ? bl1 : bl0;
      const int b0 = r0 < pc.M ? r0 / seg : 0;
      const int l0 = q.tok0 + (r0 < pc.M ? r0 % seg : 0);
      const bool fast = r0 + 31 < pc.M && (r0 % seg) + 31 < seg && (l0 & 7) == 0;   // wave-uniform
      bf16_t* col = vt + (((int64_t)b0 * q.heads + h) * 128 + half * 64 + lane) * q.seq_pad;
      if (fast) {
#pragma unroll
        for (int g8 = 0; g8 < 4; ++g8) {
          uint32_t pk[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pk[e] = pack_bf16x2(cs[(8 * g8 + 2 * e) * 64 + lane] * dq + bv, cs[(8 * g8 + 2 * e + 1) * 64 + lane] * dq + bv);
          *reinterpret_cast<uint4*>(col + l0 + 8 * g8) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
      } else {
        for (int r = 0; r < 32; ++r) {
          const int row = r0 + r;
          if (row >= pc.M) break;
          const int b = row / seg, l = q.tok0 + row % seg;
          vt[(((int64_t)b * q.heads + h) * 128 + half * 64 + lane) * q.seq_pad + l] =
              f32_to_bf16(cs[r * 64 + lane] * dq + bv);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
#pragma unroll 1
  for (int qq = 0; qq < 4; ++qq) {
    float4 wA[8], wB[8], tA[8], tB[8];
    int sb[8], sl[8];   // sample and position of the strip's rows (rows past M: sample 0, position 0)
    seg_rows(row0 + qq * 32 + lrow, seg, sb, sl);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (row0 + qq * 32 + lrow + 4 * u >= pc.M) {
        sb[u] = 0;
        sl[u] = 0;
      }
    }
    // the RoPE pairs of the strip's rows, loaded before the staging so their
    // latency overlaps it (rows past M read row 0's entry and store nothing)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* tab = q.rope + ((int64_t)sb[u] * q.seq + q.tok0 + sl[u]) * 128;   // 64 (cos, sin)
      if (q.rope) {
        tA[u] = *reinterpret_cast<const float4*>(tab + c4);
        tB[u] = *reinterpret_cast<const float4*>(tab + 64 + c4);
      }
    }
    switch (qq) {
      case 0: stage_quarter<0>(acc, cs, frow, fhalf); break;
      case 1: stage_quarter<2>(acc, cs, frow, fhalf); break;
      case 2: stage_quarter<4>(acc, cs, frow, fhalf); break;
      default: stage_quarter<6>(acc, cs, frow, fhalf); break;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
    const bool skip = sk_quarter(cs, sk, 2 * qq, lane);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float4 t = *reinterpret_cast<const float4*>(&cs[(lrow + 4 * u) * 64 + c4]);
      wA[u] = make_float4(t.x * dq + bA.x, t.y * dq + bA.y, t.z * dq + bA.z, t.w * dq + bA.w);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
    switch (qq) {
      case 0: stage_quarter<1>(acc, cs, frow, fhalf); break;
      case 1: stage_quarter<3>(acc, cs, frow, fhalf); break;
      case 2: stage_quarter<5>(acc, cs, frow, fhalf); break;
      default: stage_quarter<7>(acc, cs, frow, fhalf); break;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
    sk_quarter(cs, sk, 2 * qq + 1, lane);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float4 t = *reinterpret_cast<const float4*>(&cs[(lrow + 4 * u) * 64 + c4]);
      wB[u] = make_float4(t.x * dq + bB.x, t.y * dq + bB.y, t.z * dq + bB.z, t.w * dq + bB.w);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
    if (skip) continue;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = row0 + qq * 32 + lrow + 4 * u;
      const bool ok = row < pc.M;
      const int l = q.tok0 + sl[u];
      const int64_t hrow = (int64_t)sb[u] * q.heads + h;
      float4 a = wA[u], c = wB[u];
      {
        float ss = a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + c.x * c.x + c.y * c.y + c.z * c.z + c.w * c.w;
        ss = wave_sum<16>(ss);
        const float rs = 1.0f / sqrtf(ss / 128.0f + q.eps);
        a = make_float4(a.x * rs * gA.x, a.y * rs * gA.y, a.z * rs * gA.z, a.w * rs * gA.w);
        c = make_float4(c.x * rs * gB.x, c.y * rs * gB.y, c.z * rs * gB.z, c.w * rs * gB.w);
        if (q.rope) {
          const float4 ta = tA[u], tb = tB[u];
          a = make_float4(a.x * ta.x - a.y * ta.y, a.x * ta.y + a.y * ta.x, a.z * ta.z - a.w * ta.w,
                          a.z * ta.w + a.w * ta.z);
          c = make_float4(c.x * tb.x - c.y * tb.y, c.x * tb.y + c.y * tb.x, c.z * tb.z - c.w * tb.w,
                          c.z * tb.w + c.w * tb.z);
        }
        if (ok) {
          bf16_t* o = dst + (hrow * q.seq_pad + l) * 128;
          *reinterpret_cast<uint2*>(o + c4) = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
          *reinterpret_cast<uint2*>(o + 64 + c4) = make_uint2(pack_bf16x2(c.x, c.y), pack_bf16x2(c.z, c.w));
        }
      }
    }
  }
}

template <int EPI>
__device__ __forceinline__ void tile_epilogue(const GemmProblem& pc, const f32x16_t (&acc)[4][4], float* cs,
                                              int row0, int col0, int lane, float dq, float qs, uint32_t& mx,
                                              const SkIo& sk = SkIo{}) {
  if constexpr (EPI == kEpiQkv) {
    qkv_epilogue(pc, acc, cs, row0, col0, lane, dq, sk);
    return;
  } else if constexpr (EPI == kEpiQkvSplitGelu) {
    if (col0 < pc.n_split) {
      qkv_epilogue(pc, acc, cs, row0, col0, lane, dq, sk);
      return;
    }
  }
  constexpr int E = EPI == kEpiQkvSplitGelu ? (int)kEpiSplitGelu : EPI;   // columns past n_split: GELU to out1
  const int frow = lane & 31, fhalf = lane >> 5;
  const int c4 = (lane & 15) * 4, lrow = lane >> 4;
  // bias and gate of the lane's four columns in each column half, read once
  // per tile; the gate is that of the sample of the wave's rows (`uniform`
  // is false when they span two samples, and the gate is then read per row)
  const int rlast = min(row0 + 127, pc.M - 1);
  const int64_t b0 = (row0 < pc.M ? row0 : rlast) / pc.omap0.seg;
  const bool uniform = b0 == rlast / pc.omap0.seg;
  float4 bias0 = make_float4(0.f, 0.f, 0.f, 0.f), bias1 = bias0, gate0 = bias0, gate1 = bias0;
  {
    const int cA = min(col0 + c4, pc.N - 4), cB = min(col0 + 64 + c4, pc.N - 4);
    if (pc.bias) {
      const uint2 ba = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(pc.bias) + cA);
      const uint2 bb = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(pc.bias) + cB);
      bias0 = make_float4(__uint_as_float(ba.x << 16), __uint_as_float(ba.x & 0xffff0000u),
                          __uint_as_float(ba.y << 16), __uint_as_float(ba.y & 0xffff0000u));
      bias1 = make_float4(__uint_as_float(bb.x << 16), __uint_as_float(bb.x & 0xffff0000u),
                          __uint_as_float(bb.y << 16), __uint_as_float(bb.y & 0xffff0000u));
    }
    if constexpr (E == kEpiResid) {
      gate0 = *reinterpret_cast<const float4*>(pc.gate + b0 * pc.gate_bstride + cA);
      gate1 = *reinterpret_cast<const float4*>(pc.gate + b0 * pc.gate_bstride + cB);
    }
  }
  // quarters 2qq (columns 0..63 of the wave) and 2qq + 1 (columns 64..127);
  // residual rows are loaded one quarter ahead (xa for the first column half,
  // xb for the second)
  float4 xa[8], xb[8];
  if constexpr (E == kEpiResid) load_resid(pc, row0 + lrow, col0 + c4, xa);
#pragma unroll 1
  for (int qq = 0; qq < 4; ++qq) {
    if constexpr (E == kEpiResid) load_resid(pc, row0 + qq * 32 + lrow, col0 + 64 + c4, xb);
    switch (qq) {
      case 0: stage_quarter<0>(acc, cs, frow, fhalf); break;
      case 1: stage_quarter<2>(acc, cs, frow, fhalf); break;
      case 2: stage_quarter<4>(acc, cs, frow, fhalf); break;
      default: stage_quarter<6>(acc, cs, frow, fhalf); break;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's LDS writes have landed
    __builtin_amdgcn_sched_barrier(0);
    if (!sk_quarter(cs, sk, 2 * qq, lane))
      apply_quarter<E>(pc, cs, lrow, c4, row0 + qq * 32 + lrow, col0 + c4, bias0, gate0, uniform, dq, qs, mx, xa);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // reads done before the next quarter overwrites the staging
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (E == kEpiResid) {
      if (qq < 3) load_resid(pc, row0 + (qq + 1) * 32 + lrow, col0 + c4, xa);
    }
    switch (qq) {
      case 0: stage_quarter<1>(acc, cs, frow, fhalf); break;
      case 1: stage_quarter<3>(acc, cs, frow, fhalf); break;
      case 2: stage_quarter<5>(acc, cs, frow, fhalf); break;
      default: stage_quarter<7>(acc, cs, frow, fhalf); break;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
    if (!sk_quarter(cs, sk, 2 * qq + 1, lane))
      apply_quarter<E>(pc, cs, lrow, c4, row0 + qq * 32 + lrow, col0 + 64 + c4, bias1, gate1, uniform, dq, qs, mx,
                       xb);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// Persistent 16-bit kernel: one 256-thread block per CU walks the tiles
// t = blockIdx.x, blockIdx.x + gridDim.x, ...; 256 x 256 tiles, each wave
// owning 128 x 128 as 4 x 4 MFMA 32x32x16 tiles.  Operands move global -> LDS
// by direct loads in super-stages of k = 64, so each 8 lanes of a load read
// one whole 128-byte line of a row (64-byte row pieces left the kernel bound
// by L1 -> L2 requests; staging through VGPRs with ds_write cost more waits
// and LDS instructions than the direct path, measured on MI355X).
//  * LDS: a ring of five 32 KB slots, each holding one operand half of a
//    super-stage (A rows 0..255 or W rows 0..255, 128 bytes each, chunk c of
//    row r at physical chunk c ^ ((r >> 1) & 7)); slot 4 doubles as the
//    epilogue staging, which runs while no load targets it.  gfx950 serves
//    a 16-byte-per-lane LDS read in four cycles of 16 lanes, the lanes of a
//    cycle having equal lane bit 5 and equal (bit 4 xor bit 2) (measured
//    with the bank-conflict counter); under that grouping the fragment reads
//    of this layout hit each 4-bank group once per cycle.
//  * A super-stage is 4 slices of 16 MFMAs per wave (k = 16 each); the
//    fragments of slice n + 1 are read during slice n.  One barrier per
//    super-stage, between slices 2 and 3, before slice 3 reads the first
//    fragments of the next super-stage.  With five halves in the ring the A
//    half of super-stage j + 2 loads during slices 0-1 of j and its W half
//    during slice 3 of j, so each load has three to seven slices (0.8 to
//    1.8 us) to land before the barrier that waits for it; with two whole
//    64 KB slots, the W half had one to two slices and the waits for it cost
//    about 15 % of the kernel (measured on MI355X).  The barrier waits only
//    for the loads it needs (s_waitcnt vmcnt(8): the A half of j + 2 stays
//    in flight); __syncthreads() would wait for all of them.
//  * The next tile's first two super-stages are loaded while the epilogue
//    of the current tile runs (in slots 0-3).
//  * Operand rows are addressed as 32-bit byte offsets from the tile's A and
//    W base pointers (the launcher keeps both spans under 4 GiB).
// ---------------------------------------------------------------------------
constexpr int kHalf = 32768;   // one operand (A or W) of a super-stage: 256 rows x 128 bytes
constexpr int kHalfSlots = 5;  // LDS ring of operand halves; slot 4 doubles as the epilogue staging

// 128-byte rows (k = 64), chunk c of row r at physical chunk c ^ ((r >> 1) & 7)
__device__ __forceinline__ int ss_swz(int r) { return (r >> 1) & 7; }

template <int OP, int EPI>
__global__ void __launch_bounds__(256, 1) gemm_dl_kernel(GemmBatch bt) {
  constexpr int BM = kDlRows, BN = kDlRows, WM = 128, WN = 128, TM = 4, TN = 4;
  __shared__ __attribute__((aligned(1024))) char smem[kHalfSlots * kHalf];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 31, fhalf = lane >> 5;
  const int fs = ss_swz(frow);   // swizzle of every fragment row of this lane
  // fragment offsets in an operand half (slice sl: k16 step, chunks 2 sl + fhalf)
  int aoff[4], boff[4];
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    aoff[sl] = (wm * WM + frow) * 128 + (((2 * sl + fhalf) ^ fs) << 4);
    boff[sl] = (wn * WN + frow) * 128 + (((2 * sl + fhalf) ^ fs) << 4);
  }
  // direct load u (0..7) of an operand half by this wave: LDS rows (wave +
  // 4u) * 8 .. + 7, lane l at row + l / 8, physical chunk l % 8 = logical
  // chunk (l % 8) ^ swz
  const int lrow8 = lane >> 3;
  const int lchunk = (lane & 7) ^ ss_swz(wave * 8 + lrow8);   // swz(row) does not depend on u

  int prob = 0, m0 = 0, n0 = 0, NS = 0;   // NS: k128 units of the tile (two super-stages each)
  // A and W as raw buffers (the launcher keeps both spans under 4 GiB): a
  // load's address is the row offset soff (a VGPR, fixed per tile) plus the
  // super-stage's k offset (an SGPR), so issuing it takes no vector
  // arithmetic
  __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0x00020000), rsrc_w = rsrc_a;
  uint32_t soff[16];   // 0..7 A rows, 8..15 W rows
  auto setup = [&](int id) {   // tile id (see tile_coord)
    const TileCoord tc = tile_coord(bt, id, BM, BN);
    GemmProblem p = bt.p[0];
    if (tc.prob) p = bt.p[1];
    prob = tc.prob;
    m0 = tc.tm * BM;
    n0 = tc.tn * BN;
    NS = p.K / 128;
    rsrc_a = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.A), 0, -1, 0x00020000);
    rsrc_w = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.W), 0, -1, 0x00020000);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = ((wave + 4 * u) & 31) * 8 + lrow8;
      if (u < 8) {
        int gr = m0 + r;
        gr = gr < p.M ? gr : p.M - 1;
        soff[u] = (uint32_t)(((int64_t)(gr / p.amap.seg) * p.amap.bstride + (int64_t)(gr % p.amap.seg) * p.amap.ld +
                              lchunk * 8) * 2);
      } else {
        int gr = n0 + r;
        gr = gr < p.N ? gr : p.N - 1;
        soff[u] = (uint32_t)(((int64_t)gr * p.ldw + lchunk * 8) * 2);
      }
    }
  };
  // Operand halves in the ring: half h = 2 ss (A of super-stage ss) or 2 ss +
  // 1 (W of ss), counted from the first super-stage of the current range,
  // lives in slot h % 5.
  auto slot_of = [&](int h) { return smem + (h % kHalfSlots) * kHalf; };
  // load u (0..7) of half h (super-stage ss of the tile, W when w)
  auto dma_one = [&](int h, int ss, bool w, int u) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(w ? rsrc_w : rsrc_a,
                                             (lds_void_t*)(slot_of(h) + ((wave + 4 * u) & 31) * 1024), 16,
                                             (int)soff[(w ? 8 : 0) + u], ss * 128, 0, 0);
  };

  f32x16_t acc[TM][TN];
  u32x4_t af[2][TM], bfr[2][TN], bcv[TN];
  // fragment n (0..3 A, 4..7 W) of slice sl of local super-stage j into set s
  auto frag_one = [&](int j, int sl, int s, int n) {
    if (n < TM)
      af[s][n] = *reinterpret_cast<const u32x4_t*>(slot_of(2 * j) + aoff[sl] + n * 32 * 128);
    else
      bfr[s][n - TM] = *reinterpret_cast<const u32x4_t*>(slot_of(2 * j + 1) + boff[sl] + (n - TM) * 32 * 128);
  };
  auto mfma_one = [&](int s, int idx) {
    const int j = idx >> 2, i = idx & 3;
    if constexpr (OP == kF16) {
      if (i == 0) bcv[j] = bf16x8_to_f16x8(bfr[s][j]);
    } else {
      if (i == 0) bcv[j] = bfr[s][j];
    }
    if constexpr (OP == kF16 || OP == kF16W)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, af[s][i]),
                                                        __builtin_bit_cast(f16x8_t, bcv[j]), acc[i][j], 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[s][i]),
                                                         __builtin_bit_cast(bf16x8_t, bcv[j]), acc[i][j], 0, 0, 0);
  };
  // Super-stage j of the range (tile super-stage ss0 + j): slices 0..3 of 16
  // MFMAs, the fragments of slice n + 1 read during slice n.  ISSUE: the A
  // half of j + 2 loads during slices 0-1, at every other MFMA (into the slot
  // of W of j - 1, free since the previous barrier), and its W half during
  // slice 3, also at every other MFMA (into the slot of A of j, free after
  // this super-stage's barrier); denser load issue stalls the wave's MFMAs
  // (the W half one per MFMA over the last 8 of slice 3: 0.4-1.2 % slower).  NEXT: the barrier
  // between slices 2 and 3 waits until j + 1 has landed for every wave (VM:
  // loads left in flight, those of A of j + 2), and slice 3 reads the first
  // fragments of j + 1.  Flags are compile-time, so the k loop has no branches.
  auto super_stage = [&](int j, int ss0, auto issue, auto vm, auto next) __attribute__((always_inline)) {
    constexpr bool ISSUE = decltype(issue)::value, NEXT = decltype(next)::value;
    constexpr int VM = decltype(vm)::value;
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      mfma_one(0, idx);
      if (idx < 8) frag_one(j, 1, 1, idx);
      else if (ISSUE && (idx & 1) == 0) dma_one(2 * j + 4, ss0 + j + 2, false, (idx - 8) >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      mfma_one(1, idx);
      if (idx < 8) frag_one(j, 2, 0, idx);
      else if (ISSUE && (idx & 1) == 0) dma_one(2 * j + 4, ss0 + j + 2, false, 4 + ((idx - 8) >> 1));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      mfma_one(0, idx);
      if (idx < 8) frag_one(j, 3, 1, idx);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NEXT) {
      if constexpr (VM == 8) DL_WAIT_VM(8);
      else DL_WAIT_VM(0);
      lds_barrier();
    }
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      mfma_one(1, idx);
      if (NEXT && idx < 8) frag_one(j + 1, 0, 0, idx);
      if (ISSUE && (idx & 1) == 1) dma_one(2 * j + 5, ss0 + j + 2, true, idx >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using V8 = std::integral_constant<int, 8>;
  using V0 = std::integral_constant<int, 0>;

  // The first two super-stages (A, W, A, W halves 0..3) of the range of k128
  // units starting at u0 of the current tile.
  auto prologue = [&](int u0) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int u = 0; u < 8; ++u) dma_one(h, 2 * u0 + (h >> 1), (h & 1) != 0, u);
  };
  // k128 units [u0, u1) of the current tile into acc, the prologue of u0
  // already issued (settled: no other global memory operation was issued
  // after it, so the wait for super-stage 0 may leave super-stage 1 in
  // flight); on return every load has landed and every wave has read its
  // last fragments (the ring and the staging slot are free).  A range has at
  // least two super-stages, so it always ends in the same straight-line
  // drain (a branch between drains of different length makes the register
  // allocator spill the accumulators).
  auto run_stages = [&](int u0, int u1, bool settled) __attribute__((always_inline)) {
    const int ss0 = 2 * u0, n = 2 * (u1 - u0);
    if (settled) DL_WAIT_VM(16);
    else DL_WAIT_VM(0);
    lds_barrier();
#pragma unroll
    for (int m = 0; m < TM + TN; ++m) frag_one(0, 0, 0, m);
    int j = 0;
    for (; j + 2 < n; ++j) super_stage(j, ss0, T_{}, V8{}, T_{});
    super_stage(j, ss0, F_{}, V0{}, T_{});
    super_stage(j + 1, ss0, F_{}, V0{}, F_{});
    __syncthreads();
  };

  // Work items of this block (block i = blockIdx.x / 8 of XCD x = blockIdx.x %
  // 8, which owns the tile ids [xcd_first(x), + xcd_tiles(x))): the XCD's
  // tiles i, i + 32, ... of its data-parallel part, then (stream-K tail,
  // XCD-local) the block's share [u0, u1) of the units (tile x k128 unit) of
  // the XCD's remaining tiles, split evenly over its 32 blocks: first the
  // share of a tile it does not finish (contributor: its partial sums go to
  // its slot), then the end of a tile others began (owner: adds theirs before
  // the epilogue), then whole tiles.  Every block publishes before it waits,
  // so an owner only waits for shares that were computed first.  Slots and
  // flags are indexed x * 32 + i, so an owner's contributors are consecutive.
  enum { kFull = 0, kContrib = 1, kOwner = 2 };
  // GX: blocks of this XCD (blocks b with b % 8 == x; all XCDs have 32 in stream-K launches)
  const int G = gridDim.x, xcd = blockIdx.x % 8, bi = blockIdx.x / 8, GX = (G - xcd + 7) / 8;
  const int slot = xcd * GX + bi;
  const bool sk = bt.sk_part != nullptr && bt.sk_units > 0;
  const int first = xcd_first(bt.total_tiles, xcd), ntx = xcd_tiles(bt.total_tiles, xcd);
  const int ndx = sk ? min(ntx, (bt.sk_tail / G) * GX) : ntx;   // data-parallel tiles of the XCD
  const int n_dp = ndx > bi ? (ndx - bi + GX - 1) / GX : 0;
  int tns = 1;                                    // k128 units per tail tile (one K per split launch)
  int64_t UX = 0;                                 // tail units of the XCD
  int jc = -1, sac = 0, sbc = 0, jo = -1, sao = 0, jf0 = 0, jf1 = -1;
  if (sk) {
    tns = bt.p[0].K / 128;
    UX = (int64_t)(ntx - ndx) * tns;
    const int64_t u0 = (int64_t)bi * UX / GX, u1 = (int64_t)(bi + 1) * UX / GX;
    if (u1 > u0) {
      const int j0 = (int)(u0 / tns), j1 = (int)((u1 - 1) / tns);
      if (u1 < (int64_t)(j1 + 1) * tns) {   // the share ends inside tile j1
        jc = j1;
        sac = (int)((u0 > (int64_t)j1 * tns ? u0 : (int64_t)j1 * tns) - (int64_t)j1 * tns);
        sbc = (int)(u1 - (int64_t)j1 * tns);
      }
      if (u0 > (int64_t)j0 * tns && jc != j0) {   // the share begins inside tile j0 and finishes it
        jo = j0;
        sao = (int)(u0 - (int64_t)j0 * tns);
      }
      jf0 = u0 > (int64_t)j0 * tns ? j0 + 1 : j0;
      jf1 = jc == j1 ? j1 - 1 : j1;
    }
  }
  const int tail0 = first + ndx;                  // tile id of tail tile 0 of the XCD
  const int n_c = jc >= 0 ? 1 : 0, n_o = jo >= 0 ? 1 : 0, n_f = jf1 >= jf0 ? jf1 - jf0 + 1 : 0;
  const int n_items = n_dp + n_c + n_o + n_f;
  struct Item { int tile, s0, s1, kind; };
  auto item = [&](int i) __attribute__((always_inline)) {
    Item it;
    if (i < n_dp) {
      it.tile = first + bi + i * GX; it.s0 = 0; it.s1 = -1; it.kind = kFull;   // s1 = -1: all k units
      return it;
    }
    i -= n_dp;
    if (i < n_c) { it.tile = tail0 + jc; it.s0 = sac; it.s1 = sbc; it.kind = kContrib; return it; }
    i -= n_c;
    if (i < n_o) { it.tile = tail0 + jo; it.s0 = sao; it.s1 = -1; it.kind = kOwner; return it; }
    i -= n_o;
    it.tile = tail0 + jf0 + i; it.s0 = 0; it.s1 = -1; it.kind = kFull;
    return it;
  };
  // The owner of tail tile jo takes the shares of blocks b' < b that cover its
  // k units [0, sao): consecutive blocks bf..bl (every block holds at
  // least one unit).  It waits for their flags; a share that has not arrived
  // after sk_spin polls is computed here into acc instead, so the wait always
  // ends.  The arrived shares are added in block order at the staged-quarter
  // level of the epilogue (SkIo).
  // (the block-wide word lives in the epilogue staging area, free while an
  // owner waits: every wave has finished the previous epilogue)
  int* arrived = reinterpret_cast<int*>(smem + 4 * kHalf);
  auto owner_wait = [&](SkIo& io) __attribute__((always_inline)) {
    const int64_t U = UX;
    const int64_t t0 = (int64_t)jo * tns;
    // XCD-local block holding unit u: the largest i' with floor(i' U / GX) <= u
    auto block_of = [&](int64_t u) { return (int)(((u + 1) * GX + U - 1) / U - 1); };
    const int bf = block_of(t0), bl = block_of(t0 + sao - 1);
    const int spin = bt.sk_spin > 0 ? bt.sk_spin : (1 << 20);
    uint32_t mask = 0;
    for (int c = bf; c <= bl; ++c) {
      const int64_t cu0 = (int64_t)c * U / GX, cu1 = (int64_t)(c + 1) * U / GX;
      const int c0 = (int)((cu0 > t0 ? cu0 : t0) - t0), c1 = (int)((cu1 < t0 + sao ? cu1 : t0 + sao) - t0);
      if (c1 <= c0) continue;   // block c holds none of these units
      if (tid == 0) {
        int n = 0;
        while (__hip_atomic_load(bt.sk_flag + xcd * GX + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0 &&
               n < spin) {
          __builtin_amdgcn_s_sleep(2);
          ++n;
        }
        *arrived = __hip_atomic_load(bt.sk_flag + xcd * GX + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      const bool got = *arrived != 0;
      __syncthreads();
      if (got) {
        mask |= 1u << (c - bf);
      } else {
        prologue(c0);
        run_stages(c0, c1, false);
      }
    }
    io.in = bt.sk_part + (int64_t)(xcd * GX + bf) * kGemmSkSlotFloats + (int64_t)wave * 16384;
    io.nin = bl - bf + 1;
    io.mask = mask;
  };

  if (n_items == 0) return;
  Item cur = item(0);
  setup(cur.tile);
  prologue(cur.s0);
  for (int i = 0; i < n_items; ++i) {
#pragma unroll
    for (int ii = 0; ii < TM; ++ii)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[ii][j][e] = 0.f;
    run_stages(cur.s0, cur.s1 < 0 ? NS : cur.s1, i == 0);
    SkIo io{};
    if (cur.kind == kOwner) owner_wait(io);
    if (cur.kind == kContrib) io.out = bt.sk_part + (int64_t)slot * kGemmSkSlotFloats + (int64_t)wave * 16384;
    // all loads of this item have landed and every wave has read its last
    // fragments; the next item's first loads then overlap the epilogue
    const int cprob = prob, cm0 = m0, cn0 = n0;
    const int ckind = cur.kind;
    if (i + 1 < n_items) {
      cur = item(i + 1);
      setup(cur.tile);
      prologue(cur.s0);
    }
    GemmProblem pc = bt.p[0];
    if (cprob) pc = bt.p[1];
    uint32_t mx = 0;
    tile_epilogue<EPI>(pc, acc, reinterpret_cast<float*>(smem + 4 * kHalf) + wave * 32 * 64,
                       cm0 + wm * WM, cn0 + wn * WN, lane, 1.0f, 1.0f, mx, io);
    if (ckind == kContrib) {
      // every wave's device-coherent stores have completed before the flag is raised
      DL_WAIT_VM(0);
      __syncthreads();
      if (tid == 0) __hip_atomic_store(bt.sk_flag + slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Zero the stream-K flags of one launch (a kernel, so the launch can be captured).
__global__ void sk_clear_kernel(int32_t* flag, int n) {
  if ((int)threadIdx.x < n) flag[threadIdx.x] = 0;
}

// ---------------------------------------------------------------------------
// E4M3 operands ("FP8 training for Flux models", Configuration): persistent
// 256 x 256 kernel on v_mfma_f32_32x32x64_f8f6f4 (no block scales).  Same LDS
// ring layout and swizzle of 32 KB k32 stages, and the epilogue of the 16-bit
// persistent kernel, with a 5-stage ring filled by direct global->LDS loads; a 64-byte stage row
// now holds 64 k values, i.e. one MFMA k-step.  Lane half h of a fragment
// takes row chunks h and 2 + h (32 bytes); A and B use the same split, so each
// MFMA sums over all 64 k of the stage.  The 16 fragment reads of stage kt+1
// run under the 16 MFMAs of stage kt, into the other of two register sets.
// ---------------------------------------------------------------------------
typedef int i32x8_t __attribute__((ext_vector_type(8)));
template <int S> using SetTag = std::integral_constant<int, S>;

// Operand formats of gemm_fp8_kernel.  MXFP4 ("FP8 training for Flux models",
// Configuration, the microscaling recipes; OCP MX v1.0): a 64-byte stage row
// holds 128 E2M1 values, four 32-value MX blocks, one per 16-byte chunk.  The
// lane-half split is the one of E4M3: chunk h feeds the first fp4 MFMA of the
// stage and chunk 2 + h the second, each taking its low 16 bytes as the
// operand (the fp4 form of the instruction reads four registers).  A and W
// are packed alike, so whatever order the hardware gives the values inside a
// lane half, both operands agree on it.  The E8M0 scale a lane half passes
// covers exactly the 32 values it supplies; a lane's scales of both MFMAs are
// adjacent dwords (launch_mxfp4_quantize), loaded as one 8-byte word.
constexpr int kFmtE4M3 = 0, kFmtMx8 = 1, kFmtMx4 = 2;

template <int EPI, int FMT>
__global__ void __launch_bounds__(256, 1) gemm_fp8_kernel(GemmBatch bt) {
  constexpr bool MX = FMT != kFmtE4M3, FP4 = FMT == kFmtMx4;
  constexpr int BM = kDlRows, BN = kDlRows, WM = 128, WN = 128, TM = 4, TN = 4;
  constexpr int BK8 = 64;   // bytes per stage row: 64 E4M3 or 128 E2M1 values
  constexpr int SCS = FP4 ? 512 : 256;   // scale bytes of one stage for a wave's 128 rows
  __shared__ __attribute__((aligned(1024))) char smem[kDlStages * kDlStageBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 31, fhalf = lane >> 5;

  int aoff[TM][2], boff[TN][2];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = wm * WM + i * 32 + frow;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) aoff[i][kk] = r * 64 + (((2 * kk + fhalf) ^ dl_swz(r)) << 4);
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int r = wn * WN + j * 32 + frow;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) boff[j][kk] = (kDlRows + r) * 64 + (((2 * kk + fhalf) ^ dl_swz(r)) << 4);
  }

  int prob = 0, m0 = 0, n0 = 0, KT = 0;
  // operand rows as 32-bit byte offsets from the (wave-uniform) A and W bases
  const char* abase = nullptr;
  const char* wbase = nullptr;
  uint32_t src[8];
  // MX: the lane's scale word of step kt at sca + kt * SCS (A rows of the
  // wave) and scb + kt * SCS (W rows), loaded two steps ahead of use: cur
  // holds step kt's, nxt step kt + 1's (MXFP8 uses .x only)
  const uint8_t* sca = nullptr;   // wave-uniform: lane offset sc_lane added at the load
  const uint8_t* scb = nullptr;
  const int sc_lane = FP4 ? fhalf * 256 + frow * 8 : fhalf * 128 + frow * 4;
  uint2 cur_a = {0u, 0u}, cur_b = {0u, 0u}, nxt_a = {0u, 0u}, nxt_b = {0u, 0u};
  auto setup = [&](int t) {
    const TileCoord tc = decode_tile_id(bt, t, BM, BN);
    GemmProblem p = bt.p[0];
    if (tc.prob) p = bt.p[1];
    prob = tc.prob;
    m0 = tc.tm * BM;
    n0 = tc.tn * BN;
    KT = FP4 ? p.K / (2 * BK8) : p.K / BK8;
    if constexpr (MX) {
      sca = p.sa + (size_t)(m0 / 128 + wm) * KT * SCS;
      scb = p.sb + (size_t)(n0 / 128 + wn) * KT * SCS;
    }
    abase = reinterpret_cast<const char*>(p.A);
    wbase = reinterpret_cast<const char*>(p.W);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ins = wave + 4 * u;
      const int r = (ins & 15) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ dl_swz(r);
      if (ins < 16) {
        int gr = m0 + r;
        gr = gr < p.M ? gr : p.M - 1;
        src[u] = (uint32_t)((int64_t)(gr / p.amap.seg) * p.amap.bstride + (int64_t)(gr % p.amap.seg) * p.amap.ld +
                            c * 16);
      } else {
        int gr = n0 + r;
        gr = gr < p.N ? gr : p.N - 1;
        src[u] = (uint32_t)((int64_t)gr * p.ldw + c * 16);
      }
    }
  };
  auto issue = [&](int kt) {
    char* st = smem + (kt % kDlStages) * kDlStageBytes;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ins = wave + 4 * u;
      const char* g = (ins < 16 ? abase : wbase) + (int64_t)kt * BK8 + src[u];
      __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)(st + ins * 1024), 16, 0, 0);
    }
  };
  auto ld_scale = [&](int kk, uint2& a, uint2& b) {
    const int kc = kk < KT ? kk : KT - 1;
    if constexpr (FP4) {
      a = *reinterpret_cast<const uint2*>(sca + (size_t)kc * SCS + sc_lane);
      b = *reinterpret_cast<const uint2*>(scb + (size_t)kc * SCS + sc_lane);
    } else {
      a.x = *reinterpret_cast<const uint32_t*>(sca + (size_t)kc * SCS + sc_lane);
      b.x = *reinterpret_cast<const uint32_t*>(scb + (size_t)kc * SCS + sc_lane);
    }
  };
  auto prologue_issue = [&]() {
    const int pre = KT < 4 ? KT : 4;
    for (int t = 0; t < pre; ++t) issue(t);
    if constexpr (MX) {
      ld_scale(0, cur_a, cur_b);
      ld_scale(1, nxt_a, nxt_b);
    }
  };

  f32x16_t acc[TM][TN];
  u32x4_t fa[2][TM][2], fb[2][TN][2];   // [set][tile][chunk h or 2 + h]
  auto lfrag = [&](int kt, auto set) {
    constexpr int S = decltype(set)::value;
    const char* st = smem + (kt % kDlStages) * kDlStageBytes;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) fa[S][i][kk] = *reinterpret_cast<const u32x4_t*>(st + aoff[i][kk]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) fb[S][j][kk] = *reinterpret_cast<const u32x4_t*>(st + boff[j][kk]);
  };
  // MFMA (i, j) of a step; MX: the scale of A fragment i is byte i of the
  // lane's A dword, that of W fragment j byte j of its W dword (E8M0, one per
  // lane's row and 32-value half of the step)
  auto mma_ij = [&](auto set, auto ic, auto jc, uint32_t sa_w, uint32_t sb_w) {
    constexpr int S = decltype(set)::value, i = decltype(ic)::value, j = decltype(jc)::value;
    const i32x8_t b = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(fb[S][j][0], fb[S][j][1], 0, 1, 2, 3, 4, 5, 6, 7));
    const i32x8_t a = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(fa[S][i][0], fa[S][i][1], 0, 1, 2, 3, 4, 5, 6, 7));
    if constexpr (MX)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 0, 0, i, (int)sa_w, j, (int)sb_w);
    else
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 0, 0, 0, 0, 0, 0);
  };
  // MXFP4: fp4 MFMA (i, j) on chunk C (0: chunk h, 1: chunk 2 + h) of the
  // stage; the upper half of the 8-register operand is left undefined
  auto mma4_ij = [&](auto set, auto ic, auto jc, auto cc, uint32_t sa_w, uint32_t sb_w) {
    constexpr int S = decltype(set)::value, i = decltype(ic)::value, j = decltype(jc)::value;
    constexpr int C = decltype(cc)::value;
    const i32x8_t b = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(fb[S][j][C], fb[S][j][C], 0, 1, 2, 3, -1, -1, -1, -1));
    const i32x8_t a = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(fa[S][i][C], fa[S][i][C], 0, 1, 2, 3, -1, -1, -1, -1));
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 4, 4, i, (int)sa_w, j, (int)sb_w);
  };
  auto mma = [&](auto set) {
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    if constexpr (FP4) {
      auto half = [&](auto cc, uint32_t sa_w, uint32_t sb_w) {
        mma4_ij(set, I0{}, I0{}, cc, sa_w, sb_w); mma4_ij(set, I1{}, I0{}, cc, sa_w, sb_w);
        mma4_ij(set, I2{}, I0{}, cc, sa_w, sb_w); mma4_ij(set, I3{}, I0{}, cc, sa_w, sb_w);
        mma4_ij(set, I0{}, I1{}, cc, sa_w, sb_w); mma4_ij(set, I1{}, I1{}, cc, sa_w, sb_w);
        mma4_ij(set, I2{}, I1{}, cc, sa_w, sb_w); mma4_ij(set, I3{}, I1{}, cc, sa_w, sb_w);
        mma4_ij(set, I0{}, I2{}, cc, sa_w, sb_w); mma4_ij(set, I1{}, I2{}, cc, sa_w, sb_w);
        mma4_ij(set, I2{}, I2{}, cc, sa_w, sb_w); mma4_ij(set, I3{}, I2{}, cc, sa_w, sb_w);
        mma4_ij(set, I0{}, I3{}, cc, sa_w, sb_w); mma4_ij(set, I1{}, I3{}, cc, sa_w, sb_w);
        mma4_ij(set, I2{}, I3{}, cc, sa_w, sb_w); mma4_ij(set, I3{}, I3{}, cc, sa_w, sb_w);
      };
      half(I0{}, cur_a.x, cur_b.x);
      half(I1{}, cur_a.y, cur_b.y);
    } else {
      const uint32_t sa_w = cur_a.x, sb_w = cur_b.x;
      mma_ij(set, I0{}, I0{}, sa_w, sb_w); mma_ij(set, I1{}, I0{}, sa_w, sb_w);
      mma_ij(set, I2{}, I0{}, sa_w, sb_w); mma_ij(set, I3{}, I0{}, sa_w, sb_w);
      mma_ij(set, I0{}, I1{}, sa_w, sb_w); mma_ij(set, I1{}, I1{}, sa_w, sb_w);
      mma_ij(set, I2{}, I1{}, sa_w, sb_w); mma_ij(set, I3{}, I1{}, sa_w, sb_w);
      mma_ij(set, I0{}, I2{}, sa_w, sb_w); mma_ij(set, I1{}, I2{}, sa_w, sb_w);
      mma_ij(set, I2{}, I2{}, sa_w, sb_w); mma_ij(set, I3{}, I2{}, sa_w, sb_w);
      mma_ij(set, I0{}, I3{}, sa_w, sb_w); mma_ij(set, I1{}, I3{}, sa_w, sb_w);
      mma_ij(set, I2{}, I3{}, sa_w, sb_w); mma_ij(set, I3{}, I3{}, sa_w, sb_w);
    }
  };
  // Stage kt's fragments are in set S.  Wait until stage kt+1 has landed for
  // every wave (VM: loads allowed to stay outstanding, i.e. those of the
  // stages issued beyond kt+1), refill the stage freed two steps ago with
  // kt+4, read stage kt+1 into the other set while the MFMAs of stage kt run.
  // All flags are compile-time so the k loop carries no branches.
  // MX steps also load the scales of step kt + 2 right after the barrier, so
  // two scale dwords join each step's loads: the VM allowances grow from 16 /
  // 8 to 20 / 12 (loads issued after the stage being waited for).
  auto body = [&](int kt, auto set, auto vm, auto next, auto refill) {
    constexpr int S = decltype(set)::value;
    uint2 nn_a = {0u, 0u}, nn_b = {0u, 0u};
    if constexpr (decltype(next)::value) {
      constexpr int VM = decltype(vm)::value;
      if constexpr (MX) {
        if constexpr (VM == 16) DL_WAIT_VM(20); else if constexpr (VM == 8) DL_WAIT_VM(12); else DL_WAIT_VM(0);
      } else {
        if constexpr (VM == 16) DL_WAIT_VM(16); else if constexpr (VM == 8) DL_WAIT_VM(8); else DL_WAIT_VM(0);
      }
      lds_barrier();
      if constexpr (MX) ld_scale(kt + 2, nn_a, nn_b);
      if constexpr (decltype(refill)::value) issue(kt + 4);
      lfrag(kt + 1, SetTag<1 - S>{});
      mma(SetTag<S>{});
      constexpr int MF = FP4 ? 2 : 1;   // MFMAs per interleave slot
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8 * MF, 0);
    } else {
      mma(SetTag<S>{});
    }
    if constexpr (MX) {
      cur_a = nxt_a;
      cur_b = nxt_b;
      nxt_a = nn_a;
      nxt_b = nn_b;
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using V16 = std::integral_constant<int, 16>;
  using V8 = std::integral_constant<int, 8>;
  using V0 = std::integral_constant<int, 0>;

  int t = blockIdx.x;
  if (t >= bt.total_tiles) return;   // block-uniform
  setup(t);
  prologue_issue();
  // amax of each problem's E4M3 output over all tiles of this block, raised
  // once per block at the end: atomics on one address serialize (about 11 ns
  // each), so one per wave and tile would queue behind each other
  uint32_t mxp[2] = {0u, 0u};
  for (; t < bt.total_tiles; t += gridDim.x) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    {
      const int pre = KT < 4 ? KT : 4;   // stages of this tile already issued
      // (MX: the two scale loads of the prologue came after its stages)
      if (MX && pre == 4) DL_WAIT_VM(28);
      else if (pre == 4) DL_WAIT_VM(24); else if (pre == 3) DL_WAIT_VM(16); else if (pre == 2) DL_WAIT_VM(8); else DL_WAIT_VM(0);
    }
    __syncthreads();
    lfrag(0, SetTag<0>{});
    // KT is even and at least 4 (the launcher sends other K elsewhere).
    // Steady state: both steps of a pair refill; exactly 4 steps remain after
    // it, run straight-line so the accumulators never take two paths.
    int kt = 0;
    for (; kt + 5 < KT; kt += 2) {
      body(kt, SetTag<0>{}, V16{}, T_{}, T_{});
      body(kt + 1, SetTag<1>{}, V16{}, T_{}, T_{});
    }
    body(kt, SetTag<0>{}, V16{}, T_{}, F_{});
    body(kt + 1, SetTag<1>{}, V8{}, T_{}, F_{});
    body(kt + 2, SetTag<0>{}, V0{}, T_{}, F_{});
    body(kt + 3, SetTag<1>{}, V0{}, F_{}, F_{});

    // tile done: every wave has read its last fragments once it passes this
    // barrier, so the stages may be refilled for the next tile
    const int cprob = prob, cm0 = m0, cn0 = n0;
    __syncthreads();
    if (t + (int)gridDim.x < bt.total_tiles) {
      setup(t + gridDim.x);
      prologue_issue();
    }

    // epilogue through stage 4, which the next tile's prologue leaves alone
    GemmProblem pc = bt.p[0];
    if (cprob) pc = bt.p[1];
    uint32_t mx = 0;
    tile_epilogue<EPI>(pc, acc, reinterpret_cast<float*>(smem + 4 * kDlStageBytes) + wave * 32 * 64,
                       cm0 + wm * WM, cn0 + wn * WN, lane, epi_dequant(pc), epi_out_scale(pc), mx);
    if (cprob) mxp[1] = max(mxp[1], mx);
    else mxp[0] = max(mxp[0], mx);
  }
  if (bt.p[0].qo || (bt.count > 1 && bt.p[1].qo)) {   // block-uniform
    // stage 0 is idle: the last tile's barrier has passed and no prologue followed it
    uint32_t* red = reinterpret_cast<uint32_t*>(smem);   // [2][4]
    const uint32_t m0w = wave_max_u32(mxp[0]), m1w = wave_max_u32(mxp[1]);
    if (lane == 0) {
      red[wave] = m0w;
      red[4 + wave] = m1w;
    }
    __syncthreads();
    if (tid < 2 && (tid == 0 || bt.count > 1)) {
      const uint32_t m = max(max(red[4 * tid], red[4 * tid + 1]), max(red[4 * tid + 2], red[4 * tid + 3]));
      if (bt.p[tid].qo && m) fp8_amax_raise(bt.p[tid].qo, __uint_as_float(m));
    }
  }
}

// ---------------------------------------------------------------------------
// E4M3 operands on the ring of the 16-bit persistent kernel: a super-stage is
// k = 128 E4M3 values, i.e. the same 128-byte rows, 32 KB operand halves,
// swizzle, buffer loads and barrier schedule as gemm_dl_kernel, and two steps
// of the 32x32x64 fp8 MFMA.  In step t (0, 1) lane half h takes logical chunks
// 4t + h and 4t + 2 + h of a row (32 bytes); A and W use the same split, so
// each MFMA sums over 64 distinct k of the super-stage.  128-byte rows keep
// the loads at whole lines: 64-byte row pieces (one k64 step per stage) cap
// the global -> LDS rate below what the fp8 MFMAs consume (measured on
// MI355X).  Tiles t = blockIdx.x, + gridDim.x, ...; epilogue and the per-block
// output amax as gemm_fp8_kernel.
// ---------------------------------------------------------------------------
template <int EPI, int FMT>
__global__ void __launch_bounds__(256, 1) gemm_fp8r_kernel(GemmBatch bt) {
  constexpr bool MX = FMT != kFmtE4M3, FP4 = FMT == kFmtMx4;
  constexpr int BM = kDlRows, BN = kDlRows, WM = 128, WN = 128, TM = 4, TN = 4;
  constexpr int SCS = FP4 ? 512 : 256;   // MX: scale bytes of one 64-byte step for a wave's 128 rows
  __shared__ __attribute__((aligned(1024))) char smem[kHalfSlots * kHalf];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 31, fhalf = lane >> 5;
  const int fs = ss_swz(frow);
  // fragment offsets in an operand half: step t, chunk kk (0: 4t + h, 1: 4t + 2 + h)
  int aoff[2][2], boff[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      aoff[t][kk] = (wm * WM + frow) * 128 + (((4 * t + 2 * kk + fhalf) ^ fs) << 4);
      boff[t][kk] = (wn * WN + frow) * 128 + (((4 * t + 2 * kk + fhalf) ^ fs) << 4);
    }
  const int lrow8 = lane >> 3;
  const int lchunk = (lane & 7) ^ ss_swz(wave * 8 + lrow8);

  int prob = 0, m0 = 0, n0 = 0, NSS = 0;   // NSS: super-stages of the tile (K bytes / 128)
  // MX: the lane's scale word of 64-byte step kc at sca + kc * SCS (A rows of
  // the wave) and scb + kc * SCS (W rows), as gemm_fp8_kernel reads them;
  // step t of super-stage j is kc = 2 j + t.  Two register sets, super-stage
  // j in set j % 2, loaded two super-stages ahead (MXFP8 uses .x only).
  const uint8_t* sca = nullptr;
  const uint8_t* scb = nullptr;
  const int sc_lane = FP4 ? fhalf * 256 + frow * 8 : fhalf * 128 + frow * 4;
  uint2 scl_a[2][2], scl_b[2][2];   // [set][step]
  __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0x00020000), rsrc_w = rsrc_a;
  uint32_t soff[16];   // 0..7 A rows, 8..15 W rows (byte offsets; one byte per element)
  auto setup = [&](int t) {
    const TileCoord tc = decode_tile_id(bt, t, BM, BN);
    GemmProblem p = bt.p[0];
    if (tc.prob) p = bt.p[1];
    prob = tc.prob;
    m0 = tc.tm * BM;
    n0 = tc.tn * BN;
    NSS = (FP4 ? p.K / 2 : p.K) / 128;
    if constexpr (MX) {
      sca = p.sa + (size_t)(m0 / 128 + wm) * (2 * NSS) * SCS;
      scb = p.sb + (size_t)(n0 / 128 + wn) * (2 * NSS) * SCS;
    }
    rsrc_a = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.A), 0, -1, 0x00020000);
    rsrc_w = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.W), 0, -1, 0x00020000);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = ((wave + 4 * u) & 31) * 8 + lrow8;
      if (u < 8) {
        int gr = m0 + r;
        gr = gr < p.M ? gr : p.M - 1;
        soff[u] = (uint32_t)((int64_t)(gr / p.amap.seg) * p.amap.bstride + (int64_t)(gr % p.amap.seg) * p.amap.ld +
                             lchunk * 16);
      } else {
        int gr = n0 + r;
        gr = gr < p.N ? gr : p.N - 1;
        soff[u] = (uint32_t)((int64_t)gr * p.ldw + lchunk * 16);
      }
    }
  };
  auto slot_of = [&](int h) { return smem + (h % kHalfSlots) * kHalf; };
  auto dma_one = [&](int h, int ss, bool w, int u) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(w ? rsrc_w : rsrc_a,
                                             (lds_void_t*)(slot_of(h) + ((wave + 4 * u) & 31) * 1024), 16,
                                             (int)soff[(w ? 8 : 0) + u], ss * 128, 0, 0);
  };

  f32x16_t acc[TM][TN];
  u32x4_t fa[2][TM][2], fb[2][TN][2];   // [set][tile][chunk]
  // read q (0..15) of step t of super-stage j into set s: fragment q >> 1 (0..3 A,
  // 4..7 W), chunk q & 1
  auto frag_one = [&](int j, int t, int s, int q) {
    const int n = q >> 1, kk = q & 1;
    if (n < TM)
      fa[s][n][kk] = *reinterpret_cast<const u32x4_t*>(slot_of(2 * j) + aoff[t][kk] + n * 32 * 128);
    else
      fb[s][n - TM][kk] = *reinterpret_cast<const u32x4_t*>(slot_of(2 * j + 1) + boff[t][kk] + (n - TM) * 32 * 128);
  };
  // MX: the scale words of super-stage j into set Q
  auto ld_scales = [&](int j, auto set) __attribute__((always_inline)) {
    constexpr int Q = decltype(set)::value;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const size_t kc = (size_t)(2 * j + t) * SCS + sc_lane;
      if constexpr (FP4) {
        scl_a[Q][t] = *reinterpret_cast<const uint2*>(sca + kc);
        scl_b[Q][t] = *reinterpret_cast<const uint2*>(scb + kc);
      } else {
        scl_a[Q][t].x = *reinterpret_cast<const uint32_t*>(sca + kc);
        scl_b[Q][t].x = *reinterpret_cast<const uint32_t*>(scb + kc);
      }
    }
  };
  // MFMA of tile (I, J) in step T with fragments in set s and MX scales of
  // set Q: one E4M3 / MXFP8 MFMA over both chunks, or (MXFP4) one fp4 MFMA
  // per chunk; the scale of A fragment I is byte I of the lane's A word, that
  // of W fragment J byte J of its W word (the byte selectors are immediates,
  // hence the tile as a type)
  auto mfma_ij = [&](int s, auto ic, auto jc, auto step, auto set) __attribute__((always_inline)) {
    constexpr int I = decltype(ic)::value, J = decltype(jc)::value;
    constexpr int T = decltype(step)::value, Q = decltype(set)::value;
    if constexpr (FP4) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const i32x8_t b = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(fb[s][J][c], fb[s][J][c], 0, 1, 2, 3, -1, -1, -1, -1));
        const i32x8_t a = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(fa[s][I][c], fa[s][I][c], 0, 1, 2, 3, -1, -1, -1, -1));
        const uint32_t sa_w = c ? scl_a[Q][T].y : scl_a[Q][T].x, sb_w = c ? scl_b[Q][T].y : scl_b[Q][T].x;
        acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[I][J], 4, 4, I, (int)sa_w, J, (int)sb_w);
      }
    } else {
      const i32x8_t b = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(fb[s][J][0], fb[s][J][1], 0, 1, 2, 3, 4, 5, 6, 7));
      const i32x8_t a = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(fa[s][I][0], fa[s][I][1], 0, 1, 2, 3, 4, 5, 6, 7));
      if constexpr (MX)
        acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[I][J], 0, 0, I, (int)scl_a[Q][T].x, J,
                                                                   (int)scl_b[Q][T].x);
      else
        acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[I][J], 0, 0, 0, 0, 0, 0);
    }
  };
  // MFMA slot idx: tile (idx & 3, idx >> 2)
  auto mfma_one = [&](int s, int idx, auto step, auto set) __attribute__((always_inline)) {
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    switch (idx) {
      case 0: mfma_ij(s, C0{}, C0{}, step, set); break;
      case 1: mfma_ij(s, C1{}, C0{}, step, set); break;
      case 2: mfma_ij(s, C2{}, C0{}, step, set); break;
      case 3: mfma_ij(s, C3{}, C0{}, step, set); break;
      case 4: mfma_ij(s, C0{}, C1{}, step, set); break;
      case 5: mfma_ij(s, C1{}, C1{}, step, set); break;
      case 6: mfma_ij(s, C2{}, C1{}, step, set); break;
      case 7: mfma_ij(s, C3{}, C1{}, step, set); break;
      case 8: mfma_ij(s, C0{}, C2{}, step, set); break;
      case 9: mfma_ij(s, C1{}, C2{}, step, set); break;
      case 10: mfma_ij(s, C2{}, C2{}, step, set); break;
      case 11: mfma_ij(s, C3{}, C2{}, step, set); break;
      case 12: mfma_ij(s, C0{}, C3{}, step, set); break;
      case 13: mfma_ij(s, C1{}, C3{}, step, set); break;
      case 14: mfma_ij(s, C2{}, C3{}, step, set); break;
      default: mfma_ij(s, C3{}, C3{}, step, set); break;
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // Super-stage j: step 0 (set 0) under the reads of step 1 into set 1 and
  // (ISSUE) the loads of A of j + 2, at every other MFMA; then (NEXT) the
  // barrier once j + 1 has landed (VM loads left in flight: A of j + 2);
  // step 1 (set 1) under the reads of step 0 of j + 1 into set 0 and
  // (ISSUE) the loads of W of j + 2 into the slot of A of j.
  auto super_stage = [&](int j, auto issue, auto vm, auto next, auto set, auto lscale) __attribute__((always_inline)) {
    constexpr bool ISSUE = decltype(issue)::value, NEXT = decltype(next)::value;
    constexpr bool LSCALE = decltype(lscale)::value;
    constexpr int VM = decltype(vm)::value;
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      mfma_one(0, idx, S0{}, set);
      frag_one(j, 1, 1, idx);
      if (ISSUE && (idx & 1) == 1) dma_one(2 * j + 4, j + 2, false, idx >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NEXT) {
      if constexpr (VM == 8) DL_WAIT_VM(8);
      else DL_WAIT_VM(0);
      lds_barrier();
    }
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      mfma_one(1, idx, S1{}, set);
      if (NEXT) frag_one(j + 1, 0, 0, idx);
      if (ISSUE && (idx & 1) == 1) dma_one(2 * j + 5, j + 2, true, idx >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // MX: the scales of super-stage j + 2 into this set, free once its MFMAs
    // are issued; they precede the A loads of j + 3, so the barrier of j + 1
    // (which leaves only those in flight) finds them landed
    if constexpr (MX && LSCALE) ld_scales(j + 2, set);
    __builtin_amdgcn_sched_barrier(0);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using V8 = std::integral_constant<int, 8>;
  using V0 = std::integral_constant<int, 0>;
  // halves 0..3 (A, W of super-stages 0 and 1) of the current tile, after
  // (MX) the scales of super-stages 0 and 1
  auto prologue = [&]() __attribute__((always_inline)) {
    if constexpr (MX) {
      ld_scales(0, S0{});
      ld_scales(1, S1{});
    }
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int u = 0; u < 8; ++u) dma_one(h, h >> 1, (h & 1) != 0, u);
  };
  // all NSS (>= 2) super-stages of the current tile into acc, its prologue
  // issued (settled: no global memory operation after it); on return every
  // load has landed and every wave has read its last fragments
  auto run_stages = [&](bool settled) __attribute__((always_inline)) {
    if (settled) DL_WAIT_VM(16);
    else DL_WAIT_VM(0);
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 16; ++q) frag_one(0, 0, 0, q);
    int j = 0;
    if constexpr (MX) {
      // pairs, so super-stage j's scale set j % 2 is fixed at compile time
      // (NSS is even for MX launches)
      for (; j + 2 < NSS; j += 2) {
        super_stage(j, T_{}, V8{}, T_{}, S0{}, T_{});
        super_stage(j + 1, T_{}, V8{}, T_{}, S1{}, T_{});
      }
    } else {
      for (; j + 2 < NSS; ++j) super_stage(j, T_{}, V8{}, T_{}, S0{}, F_{});
    }
    super_stage(j, F_{}, V0{}, T_{}, S0{}, F_{});
    super_stage(j + 1, F_{}, V0{}, F_{}, S1{}, F_{});
    __syncthreads();
  };

  int t = blockIdx.x;
  if (t >= bt.total_tiles) return;   // block-uniform
  setup(t);
  prologue();
  // amax of each problem's E4M3 output over the block's tiles, raised once
  // per block (as gemm_fp8_kernel)
  uint32_t mxp[2] = {0u, 0u};
  for (bool first = true; t < bt.total_tiles; t += gridDim.x, first = false) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    run_stages(first);
    const int cprob = prob, cm0 = m0, cn0 = n0;
    if (t + (int)gridDim.x < bt.total_tiles) {
      setup(t + gridDim.x);
      prologue();
    }
    // epilogue through slot 4, which the next tile's prologue leaves alone
    GemmProblem pc = bt.p[0];
    if (cprob) pc = bt.p[1];
    uint32_t mx = 0;
    tile_epilogue<EPI>(pc, acc, reinterpret_cast<float*>(smem + 4 * kHalf) + wave * 32 * 64, cm0 + wm * WM,
                       cn0 + wn * WN, lane, epi_dequant(pc), epi_out_scale(pc), mx);
    if (cprob) mxp[1] = max(mxp[1], mx);
    else mxp[0] = max(mxp[0], mx);
  }
  if (bt.p[0].qo || (bt.count > 1 && bt.p[1].qo)) {   // block-uniform
    // slot 0 is idle: the last tile's barrier has passed and no prologue followed it
    __syncthreads();
    uint32_t* red = reinterpret_cast<uint32_t*>(smem);   // [2][4]
    const uint32_t m0w = wave_max_u32(mxp[0]), m1w = wave_max_u32(mxp[1]);
    if (lane == 0) {
      red[wave] = m0w;
      red[4 + wave] = m1w;
    }
    __syncthreads();
    if (tid < 2 && (tid == 0 || bt.count > 1)) {
      const uint32_t m = max(max(red[4 * tid], red[4 * tid + 1]), max(red[4 * tid + 2], red[4 * tid + 3]));
      if (bt.p[tid].qo && m) fp8_amax_raise(bt.p[tid].qo, __uint_as_float(m));
    }
  }
}

// Split-K reduction: out = epilogue(sum over splits s = 0..ksplit-1 in order
// of partials[s]), four consecutive columns per thread; the accumulator
// scale of E4M3 operands was applied when the partials were written.
__global__ void __launch_bounds__(256) gemm_splitk_reduce_kernel(GemmProblem p, const float* __restrict__ partials,
                                                                 int ksplit) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // over M * N / 4
  const int n4 = p.N / 4;
  if (i >= (int64_t)p.M * n4) return;
  const int row = (int)(i / n4), col = (int)(i % n4) * 4;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < ksplit; ++s) {
    const float4 t = *reinterpret_cast<const float4*>(partials + ((int64_t)s * p.M + row) * p.N + col);
    v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w;
  }
  uint32_t mx = 0;
  epi_apply4_any(p, row, col, v, 1.0f, 1.0f, mx);
}

// ---------------------------------------------------------------------------
// fp32 kernel: 64 x 64 tile, 16 x 16 threads with 4 x 4 outputs each
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmBatch bt) {
  constexpr int BM = 64, BN = 64, BKF = 16;
  __shared__ float As[BKF][BM + 4];
  __shared__ float Bs[BKF][BN + 4];
  const TileCoord tc = decode_tile(bt, BM, BN);
  // select by value: a dynamically indexed kernel-argument array would be
  // copied to scratch memory
  GemmProblem p = bt.p[0];
  if (tc.prob) p = bt.p[1];
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const float* A = reinterpret_cast<const float*>(p.A);
  const float* W = reinterpret_cast<const float*>(p.W);
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += BKF) {
    for (int i = threadIdx.x; i < BM * BKF; i += 256) {
      const int r = i / BKF, kk = i % BKF;
      int gr = m0 + r;
      gr = gr < p.M ? gr : p.M - 1;
      const int k = k0 + kk;
      As[kk][r] = k < p.K ? A[(int64_t)(gr / p.amap.seg) * p.amap.bstride + (int64_t)(gr % p.amap.seg) * p.amap.ld + k]
                          : 0.f;
      int gn = n0 + r;
      gn = gn < p.N ? gn : p.N - 1;
      Bs[kk][r] = k < p.K ? W[(int64_t)gn * p.ldw + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKF; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
  const float* bias = reinterpret_cast<const float*>(p.bias);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty + 16 * i;
    const EpiRow er = epi_row(p, row, 4);
    if (!er.valid) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx + 16 * j;
      if (col < p.N) epi_apply<float>(p, er, col, acc[i][j] + (bias ? bias[col] : 0.f));
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
static int assign_tiles(GemmBatch& bt, int BM, int BN) {
  int t = 0;
  for (int i = 0; i < bt.count; ++i) {
    bt.p[i].tile_begin = t;
    bt.p[i].tiles_n = (int)ceil_div(bt.p[i].N, BN);
    t += (int)ceil_div(bt.p[i].M, BM) * bt.p[i].tiles_n;
  }
  bt.total_tiles = t;
  return t;
}

static double gemm_flops(const GemmBatch& bt) {
  double f = 0.0;
  for (int i = 0; i < bt.count; ++i) f += 2.0 * bt.p[i].M * (double)bt.p[i].N * bt.p[i].K;
  return f;
}

// Operand rows of gemm_fp8_kernel are 32-bit byte offsets from A and W.
static bool fp8_span_ok(const GemmProblem& q) {
  const int64_t last = q.M - 1;
  const int64_t a_span = (last / q.amap.seg) * q.amap.bstride + (last % q.amap.seg) * q.amap.ld + q.K;
  const int64_t w_span = (int64_t)(q.N - 1) * q.ldw + q.K;
  return a_span < (int64_t(1) << 32) && w_span < (int64_t(1) << 32);
}

template <int OP, int EPI>
static void launch_persistent(const GemmBatch& big, int grid, hipStream_t stream) {
  // MX on the ring needs an even number of 128-byte super-stages (its scale
  // registers alternate between two sets); other K keep gemm_fp8_kernel
  bool even = true;
  for (int i = 0; i < big.count; ++i)
    even = even && ((OP == kMXFP4 ? big.p[i].K / 2 : big.p[i].K) / 128) % 2 == 0;
  if constexpr (OP == kFP8)
    hipLaunchKernelGGL((gemm_fp8r_kernel<EPI, kFmtE4M3>), dim3(grid), dim3(256), 0, stream, big);
  else if constexpr (OP == kMXFP8) {
    if (even) hipLaunchKernelGGL((gemm_fp8r_kernel<EPI, kFmtMx8>), dim3(grid), dim3(256), 0, stream, big);
    else hipLaunchKernelGGL((gemm_fp8_kernel<EPI, kFmtMx8>), dim3(grid), dim3(256), 0, stream, big);
  } else if constexpr (OP == kMXFP4) {
    if (even) hipLaunchKernelGGL((gemm_fp8r_kernel<EPI, kFmtMx4>), dim3(grid), dim3(256), 0, stream, big);
    else hipLaunchKernelGGL((gemm_fp8_kernel<EPI, kFmtMx4>), dim3(grid), dim3(256), 0, stream, big);
  }
  else
    hipLaunchKernelGGL((gemm_dl_kernel<OP, EPI>), dim3(grid), dim3(256), 0, stream, big);
}

// Conditions of the persistent 256 x 256 kernels for 16-bit or E4M3 operands.
static bool persistent_ok(GemmBatch big, int op) {
  const int tiles_big = assign_tiles(big, 256, 256);
  bool ok = true;   // the persistent kernel's epilogue needs >= 32 rows per sample (seg_rows)
  for (int i = 0; i < big.count; ++i)
    ok = ok && big.p[i].omap0.seg >= 32 && (big.p[i].out1 == nullptr || big.p[i].omap1.seg >= 32);
  if (op == kFP8) {   // gemm_fp8_kernel walks k in pairs of 64-wide steps, at least 4 of them
    for (int i = 0; i < big.count; ++i) ok = ok && big.p[i].K % 128 == 0 && big.p[i].K >= 256;
    for (int i = 0; i < big.count; ++i) ok = ok && fp8_span_ok(big.p[i]);
  } else {   // gemm_dl_kernel: k in units of 128; operand rows as 32-bit byte offsets
    for (int i = 0; i < big.count; ++i) {
      const GemmProblem& q = big.p[i];
      const int64_t last = q.M - 1;
      const int64_t a_span = ((last / q.amap.seg) * q.amap.bstride + (last % q.amap.seg) * q.amap.ld + q.K) * 2;
      const int64_t w_span = ((int64_t)(q.N - 1) * q.ldw + q.K) * 2;
      ok = ok && q.K % 128 == 0 && a_span < (int64_t(1) << 32) && w_span < (int64_t(1) << 32);
    }
  }
  // the persistent kernel needs at least half the CUs busy with 256 x 256
  // tiles; with K < 512 a tile is mostly epilogue, which smaller tiles spread
  // over more CUs
  for (int i = 0; i < big.count; ++i) ok = ok && big.p[i].K >= 512;
  return tiles_big >= 128 && ok;
}

bool gemm_is_persistent(const GemmBatch& bt, int op) {
  if (op == kMXFP8 || op == kMXFP4 || op == kF32) return false;   // no attention-layout epilogue there
  return persistent_ok(bt, op);
}

// Stream-K setting of the persistent 16-bit GEMM (flux_gemm_stream_k): off by
// default, since at the 12B block shapes the owners' waits for the partial
// sums cost more than the balanced tail gains; the spin limit of an owner's
// wait (0: the kernel's default).
static std::atomic<int> g_sk_mode{0};
static std::atomic<int> g_sk_spin{0};

int gemm_stream_k(int mode, int spin) {
  const int prev = g_sk_mode.load();
  if (mode >= 0) g_sk_mode.store(mode ? 1 : 0);
  g_sk_spin.store(spin > 0 ? spin : 0);
  return prev;
}

template <int OP>
static hipError_t launch_mfma(GemmBatch bt, hipStream_t stream, double flops) {
  bt.ksplit = 1;
  GemmBatch big = bt;
  const int tiles_big = assign_tiles(big, 256, 256);
  const int epi = big.p[0].epi;   // the problems of one launch share the epilogue kind
  if (persistent_ok(big, OP)) {
    int grid = tiles_big < 256 ? tiles_big : 256;
    // stream-K tail (16-bit operands, problems of one K, a workspace given):
    // the tiles past the last full round of 256 are shared out along K over
    // all 256 blocks when there are at least 64 of them (so a tile has at most
    // five shares and every block at least one k unit)
    big.sk_tail = tiles_big;
    big.sk_units = 0;
    if constexpr (OP == kBF16 || OP == kF16 || OP == kF16W) {
      bool same_k = true;
      for (int i = 1; i < big.count; ++i) same_k = same_k && big.p[i].K == big.p[0].K;
      const int full = (tiles_big / kGemmSkMaxGrid) * kGemmSkMaxGrid, rest = tiles_big - full;
      const int64_t units = (int64_t)rest * (big.p[0].K / 128);
      if (g_sk_mode.load() && big.sk_part && big.sk_flag && same_k && rest >= 64 && units >= kGemmSkMaxGrid &&
          units < (int64_t(1) << 30)) {
        grid = kGemmSkMaxGrid;
        big.sk_tail = full;
        big.sk_units = (int32_t)units;
        big.sk_spin = g_sk_spin.load();
        hipLaunchKernelGGL(sk_clear_kernel, dim3(1), dim3(kGemmSkMaxGrid), 0, stream, big.sk_flag, kGemmSkMaxGrid);
      }
    }
    TimingScope ts(OP == kFP8 ? kKcGemmPkFp8 : OP == kBF16 ? kKcGemmPkBf16 : kKcGemmPkF16, stream, flops);
    switch (epi) {
      case kEpiStore: launch_persistent<OP, kEpiStore>(big, grid, stream); break;
      case kEpiGelu: launch_persistent<OP, kEpiGelu>(big, grid, stream); break;
      case kEpiResid: launch_persistent<OP, kEpiResid>(big, grid, stream); break;
      case kEpiStoreF32: launch_persistent<OP, kEpiStoreF32>(big, grid, stream); break;
      case kEpiQkv: launch_persistent<OP, kEpiQkv>(big, grid, stream); break;
      case kEpiQkvSplitGelu: launch_persistent<OP, kEpiQkvSplitGelu>(big, grid, stream); break;
      default: launch_persistent<OP, kEpiSplitGelu>(big, grid, stream); break;
    }
    return hipSuccess;
  }
  // the attention-layout epilogues exist in the persistent kernels only; the
  // caller checks gemm_is_persistent first
  if (epi == kEpiQkv || epi == kEpiQkvSplitGelu) return hipErrorInvalidValue;
  {
    const int tiles = assign_tiles(bt, 128, 128);
    // split K when the tiles fill less than half the GPU, the caller gave
    // scratch and the epilogue writes no E4M3 output (whose amax the
    // reduction would have to raise)
    int ks = 1;
    const GemmProblem& q = bt.p[0];
    if (bt.partials && bt.count == 1 && !q.qo && q.N % 4 == 0) {
      while (ks < kGemmMaxSplit && tiles * ks * 2 <= 256 && q.K % (ks * 2 * kBK) == 0) ks *= 2;
    }
    bt.ksplit = ks;
    TimingScope ts(kKcGemm128, stream, flops);
    hipLaunchKernelGGL((gemm_mfma_kernel<128, 128, OP>), dim3(tiles, ks), dim3(256), 0, stream, bt);
    if (ks > 1) {
      const int64_t n = (int64_t)q.M * (q.N / 4);
      hipLaunchKernelGGL(gemm_splitk_reduce_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, q,
                         bt.partials, ks);
    }
  }
  return hipSuccess;
}

// MX operands: always the persistent kernel (its K loop needs an even number
// of at least 4 stages: MXFP8 K % 128 == 0 and K >= 256, MXFP4 K % 256 == 0
// and K >= 512, checked by the API), one or two problems sharing the epilogue
// kind.
template <int OP>
static void launch_mx(GemmBatch bt, hipStream_t stream, double flops) {
  bt.ksplit = 1;
  const int tiles = assign_tiles(bt, 256, 256);
  const int grid = tiles < 256 ? tiles : 256;
  TimingScope ts(OP == kMXFP4 ? kKcGemmPkMx4 : kKcGemmPkMx, stream, flops);
  switch (bt.p[0].epi) {
    case kEpiStore: launch_persistent<OP, kEpiStore>(bt, grid, stream); break;
    case kEpiGelu: launch_persistent<OP, kEpiGelu>(bt, grid, stream); break;
    case kEpiResid: launch_persistent<OP, kEpiResid>(bt, grid, stream); break;
    case kEpiStoreF32: launch_persistent<OP, kEpiStoreF32>(bt, grid, stream); break;
    default: launch_persistent<OP, kEpiSplitGelu>(bt, grid, stream); break;
  }
}

// Zero the rows [seq, seq_pad) of every (batch, head) of qh and kh and the
// columns [seq, seq_pad) of every row of vt.
__global__ void attn_pad_zero_kernel(bf16_t* qh, bf16_t* kh, bf16_t* vt, int batch, int heads, int seq,
                                     int seq_pad) {
  const int pad = seq_pad - seq;
  const int64_t bh = blockIdx.y;              // (batch, head)
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < pad * 128; i += gridDim.x * blockDim.x) {
    const int r = seq + i / 128, d = i % 128;
    qh[(bh * seq_pad + r) * 128 + d] = 0;
    kh[(bh * seq_pad + r) * 128 + d] = 0;
    vt[(bh * 128 + d) * seq_pad + r] = 0;
  }
}

hipError_t launch_attn_pad_zero(void* qh, void* kh, void* vt, int batch, int heads, int seq, int seq_pad,
                                hipStream_t stream) {
  if (seq_pad <= seq) return hipSuccess;
  TimingScope ts(kKcMisc, stream);
  const int n = (seq_pad - seq) * 128;
  hipLaunchKernelGGL(attn_pad_zero_kernel, dim3((unsigned)ceil_div(n, 256), (unsigned)(batch * heads)), dim3(256), 0,
                     stream, static_cast<bf16_t*>(qh), static_cast<bf16_t*>(kh), static_cast<bf16_t*>(vt), batch,
                     heads, seq, seq_pad);
  return hipGetLastError();
}

hipError_t launch_gemm(GemmBatch bt, int op, hipStream_t stream) {
  const double flops = gemm_flops(bt);
  if (op == kMXFP8 || op == kMXFP4) {
    if (op == kMXFP8) launch_mx<kMXFP8>(bt, stream, flops);
    else launch_mx<kMXFP4>(bt, stream, flops);
    return hipGetLastError();
  }
  if (op == kF32) {
    bt.ksplit = 1;
    const int tiles = assign_tiles(bt, 64, 64);
    TimingScope ts(kKcGemmF32, stream, flops);
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(tiles), dim3(256), 0, stream, bt);
    return hipGetLastError();
  }
  hipError_t e;
  if (op == kFP8)
    e = launch_mfma<kFP8>(bt, stream, flops);
  else if (op == kF16W)
    e = launch_mfma<kF16W>(bt, stream, flops);
  else if (op == kF16)
    e = launch_mfma<kF16>(bt, stream, flops);
  else
    e = launch_mfma<kBF16>(bt, stream, flops);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace flux
