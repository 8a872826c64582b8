// Joint softmax attention O = softmax(Q K^T / sqrt(Dh)) V, no mask, over the
// concatenated image|text sequence ("Flux architecture deep dive",
// Implementation details / Attention implementation and the joint attention
// trick; Mathematical formulation).  Exact attention evaluated flash-style:
// K / V tiles streamed through LDS, running max and sum in registers, no
// L x L buffer.
//
// bf16 kernel (CDNA4, wave64, v_mfma_f32_32x32x16_bf16): a block owns 256
// queries of one (batch, head); each of its 8 waves (2 per SIMD, so one
// wave's softmax overlaps the other's MFMAs) owns 32 queries.  256 queries
// share each K / V^T tile, which halves the operand traffic per FLOP against
// 128-query blocks; at 128 the tile stream needed about 32 bytes per clock
// per CU from L2, beyond what MI355X sustains.  Blocks are placed so that the
// query blocks of one (batch, head) run on one XCD and share its L2.
// Per 64-key tile a wave computes S^T = K Q^T (keys on MFMA rows, its queries
// on MFMA columns), so lane l holds 32 scores of query l % 32 and the row max
// / sum need a single exchange with lane l ^ 32.  The probabilities then feed
// O^T = V^T P^T directly from registers: K rows are stored in LDS in a
// permuted order (bits 2 and 3 of the row index swapped within each 32-row
// half) so that the accumulator registers of each lane hold 8 consecutive
// keys per 16-key MFMA step, matching 8 consecutive keys of a V^T row.
// The running max is raised lazily: O and the running sum are rescaled only
// when a row's tile max exceeds its running max by more than 2^8 (log2
// units), so probabilities stay below 256 (exact in bf16's range, same
// relative rounding) and the 64 multiplies of O are skipped on almost every
// tile.  The result is the same softmax; only the reference point of the
// exponentials differs.
// K and V^T tiles reach LDS by direct global -> LDS loads (16 bytes per lane,
// no register round trip) into a ring of four slots each: iteration t reads
// K(t + 1) and V(t) while V(t + 3) and K(t + 4) load, so every load has two
// iterations to land, and the one barrier per tile waits only for the loads
// the next iteration reads (counted vmcnt; __syncthreads() would wait for
// all).  Against K / V staged through registers with two LDS buffers each:
// 328 -> 300 us at B=1, L=4608, 24 heads on MI355X, bit-identical results.
// All slots are one LDS array: with one array per tile kind the compiler
// adds a wait for every load in flight before each fragment read.
// Inputs, as the q|k|v GEMM epilogue or launch_prep write them: Q, K
// head-major [B, H, Lp, Dh] and V transposed [B, H, Dh, Lp], Lp = seq
// rounded up to 256, zero padded.  The
// output is written as bf16, fp16 or E4M3 (the operand type of the next
// linear; E4M3 with the delayed scale of the row's stream).
#include <math.h>

#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace flux {

__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <int DH, int OUT>
__global__ void __launch_bounds__(512, 1) attn_bf16_kernel(AttnArgs a) {
  constexpr int KT = 64;          // keys per tile
  constexpr int QW = 32;          // queries per wave
  constexpr int NW = 8;           // waves per block
  constexpr int QB = NW * QW;     // queries per block
  constexpr int KS = DH / 16;     // MFMA k-steps of S^T
  constexpr int DT = DH / 32;     // 32-row tiles of O^T
  constexpr float kLazy = 8.0f;   // rescale when a tile max exceeds the running max by this (log2)
  constexpr int KSL = 4;                      // ring slots of K and of V^T tiles
  constexpr int KRB = DH * 2;                 // K row bytes (256 or 128); V^T rows are 128
  constexpr int TB = KT * DH * 2;             // bytes of one K or V^T tile
  constexpr int NKD = TB / 1024 / NW;         // 1 KB loads per wave and tile, K
  constexpr int NVD = TB / 1024 / NW;         // and V^T
  constexpr int VMW = 2 * (NKD + NVD);        // loads left in flight at the end of an iteration
  // Rows unpadded; 16-byte chunk c of row r at physical chunk c ^ swz(r), with
  // swz(r) = r & 15 for 256-byte rows and (r >> 1) & 7 for 128-byte rows.
  // gfx950 serves a 16-byte-per-lane read in four cycles of 16 lanes, those of
  // a cycle having equal lane bit 5 and equal (bit 4 xor bit 2) (measured with
  // the bank-conflict counter); a fragment read of 32 consecutive rows at one
  // logical chunk then hits each 4-bank group once per cycle.
  __shared__ __attribute__((aligned(1024))) char ring[2 * KSL * TB];
  auto kslot = [&](int j) { return ring + (j % KSL) * TB; };
  auto vslot = [&](int j) { return ring + (KSL + j % KSL) * TB; };

  // work item of this block: XCD x (blocks are dispatched round-robin over the
  // 8 XCDs) takes the contiguous item range [x * per, (x + 1) * per), so the
  // query blocks of a (batch, head) stay on one XCD
  const int nq = a.seq_pad / QB;
  const int total = a.batch * a.heads * nq;
  const int per = (total + 7) / 8;
  const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (item >= total) return;
  const int qb = item % nq;
  const int64_t bh = item / nq;
  const int b = (int)(bh / a.heads), h = (int)(bh % a.heads);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int kswz = KRB == 256 ? (l32 & 15) : ((l32 >> 1) & 7);   // swz of the lane's fragment rows
  const int vswz = (l32 >> 1) & 7;
  const bf16_t* Qh = reinterpret_cast<const bf16_t*>(a.qh) + bh * a.seq_pad * DH;
  const bf16_t* Kh = reinterpret_cast<const bf16_t*>(a.kh) + bh * a.seq_pad * DH;
  const bf16_t* Vt = reinterpret_cast<const bf16_t*>(a.vt) + bh * DH * a.seq_pad;

  const int q = qb * QB + wave * QW + l32;
  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(Qh + (int64_t)q * DH + ks * 16 + half * 8);

  f32x16_t o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = a.scale_log2;

  // S^T of tile t (64 keys x 32 queries, two 32 x 32 tiles)
  auto s_tile = [&](int t, f32x16_t (&sv)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sv[u][e] = 0.f;
      const int rho = u * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t kf =
            *reinterpret_cast<const bf16x8_t*>(kslot(t) + rho * KRB + (((ks * 2 + half) ^ kswz) << 4));
        sv[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sv[u], 0, 0, 0);
      }
    }
  };
  // softmax of tile t's scores (sv[u][e] is the score of key
  // t*64 + (2u + e/8)*16 + half*8 + e%8 for query l32), in two parts: the
  // row max and the (rare) rescale, which branch, then the exponentials and
  // sums, straight-line code that the scheduler can interleave with MFMAs
  bf16x8_t pf[4];
  auto softmax_max = [&](int t, f32x16_t (&sv)[2]) {
    if ((t + 1) * KT > a.seq) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = t * KT + (2 * u + (e >> 3)) * 16 + half * 8 + (e & 7);
          if (key >= a.seq) sv[u][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sv[u][e]);
    {
      // with lane l ^ 32, through the VALU: the swap leaves lane l holding its
      // own max and its partner's in the two results (no LDS round trip)
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // lazy max: move the reference point only when the tile max exceeds it
    // by more than kLazy (always on the first tile, where m_run = -inf)
    const float m_tile = mx * sc;
    if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
      m_run = m_new;
    }
  };
  // Direct global -> LDS loads, 1 KB per instruction (lane l writes bytes
  // 16 l .. 16 l + 15 of it).  Lane l of a K load fills LDS row r at physical
  // chunk p, so it loads logical chunk p ^ swz(r) of the key stored in row r
  // (rows hold keys in the permuted order, swap23 being its own inverse); a
  // V^T load fills 8 rows of 128 bytes the same way.  A tile index past the
  // last tile loads the last tile again (into a slot no one reads), so every
  // iteration issues the same number of loads.  Offsets: per lane (fixed),
  // plus the tile's (a scalar).
  const int ntl = (a.seq + KT - 1) / KT;
  __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(Kh), 0, -1, 0x00020000);
  __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(Vt), 0, -1, 0x00020000);
  int koff[NKD], voff[NVD];
#pragma unroll
  for (int u = 0; u < NKD; ++u) {
    const int r = (wave * NKD + u) * (1024 / KRB) + lane / (KRB / 16);
    const int c = (lane % (KRB / 16)) ^ (KRB == 256 ? (r & 15) : ((r >> 1) & 7));
    koff[u] = ((r & 32) | swap23(r & 31)) * KRB + c * 16;
  }
#pragma unroll
  for (int u = 0; u < NVD; ++u) {
    const int d = (wave * NVD + u) * 8 + (lane >> 3);
    voff[u] = d * a.seq_pad * 2 + (((lane & 7) ^ ((d >> 1) & 7)) << 4);
  }
  auto dma_k = [&](int j, int u) {
    const int jj = j < ntl ? j : ntl - 1;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_k, (lds_void_t*)(kslot(j) + (wave * NKD + u) * 1024), 16,
                                             (int)koff[u], (int)(jj * KT * KRB), 0, 0);
  };
  auto dma_v = [&](int j, int u) {
    const int jj = j < ntl ? j : ntl - 1;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_v, (lds_void_t*)(vslot(j) + (wave * NVD + u) * 1024), 16,
                                             (int)voff[u], (int)(jj * KT * 2), 0, 0);
  };

  // Fragment reads run AH MFMAs ahead of their use.  V^T fragment m of tile
  // t: output tile i = m % DT, key step m / DT (the chains alternate); K
  // fragment m: score tile m % 2, k step m / 2.
  constexpr int NP = DT * 4, NM = 2 * KS, AH = 3;
  bf16x8_t vq[NP], kq[NM];
  auto vfrag = [&](int t, int m) {
    return *reinterpret_cast<const bf16x8_t*>(vslot(t) + ((m % DT) * 32 + l32) * 128 +
                                              ((((m / DT) * 2 + half) ^ vswz) << 4));
  };
  auto kfrag = [&](int t, int m) {
    return *reinterpret_cast<const bf16x8_t*>(kslot(t) + ((m & 1) * 32 + l32) * KRB +
                                              ((((m >> 1) * 2 + half) ^ kswz) << 4));
  };
  // O^T += V^T P^T over the 4 16-key steps of tile t (its first AH fragments
  // already read); the loads of V(t + 3) and K(t + 4) are spread over the
  // MFMAs
  auto pv_tile = [&](int t) {
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      if (m + AH < NP) vq[m + AH] = vfrag(t, m + AH);
      o[m % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[m], pf[m / DT], o[m % DT], 0, 0, 0);
      if ((m & 3) == 1) {
        const int d = m >> 2;
        if (d < NVD) dma_v(t + 3, d);
        else if (d < NVD + NKD) dma_k(t + 4, d - NVD);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Software pipeline, one barrier per tile: iteration t computes S(t + 1)
  // while the softmax of S(t) runs (the MFMAs do not depend on it, so the
  // SIMD executes both at once), then O += V(t) P(t).  Loads in issue order:
  // K(0) V(0) K(1) V(1) K(2) V(2) K(3) before the loop, V(t + 3) K(t + 4) in
  // iteration t, into the slots of V(t - 1) and K(t), last read in iteration
  // t - 1.  At the end of iteration t, K(t + 2) and V(t + 1) must have landed:
  // the four tiles issued after them may still be in flight (VMW loads).
  const int ntiles = ntl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int u = 0; u < NKD; ++u) dma_k(j, u);
    if (j < 3) {
#pragma unroll
      for (int u = 0; u < NVD; ++u) dma_v(j, u);
    }
  }
  DL_WAIT_VM(VMW);   // K(0), V(0), K(1)
  lds_barrier();
  f32x16_t sc_cur[2], sc_nxt[2];
  s_tile(0, sc_cur);
  // iteration 0 loads K(4) into K(0)'s slot: every wave must have read K(0)
  lds_barrier();
  for (int t = 0; t < ntiles; ++t) {
    // the first K fragments of S(t + 1) (K(t + 1) landed before the last
    // barrier): their latency hides under the row max
#pragma unroll
    for (int m = 0; m < AH; ++m) kq[m] = kfrag(t + 1, m);
    softmax_max(t, sc_cur);
    // S(t + 1) with the exponentials of tile t in its MFMA shadow: step m
    // (of 2 KS) issues one MFMA, the K fragment read of step m + 3 (in the
    // last steps, the first V^T fragments of P V(t)) and 16 / (2 KS)
    // probability pairs of tile t, fenced so the compiler keeps the
    // interleave.  On the last tile the product is of a resident buffer and
    // is discarded (no branch in the interleaved code).  The two
    // accumulation chains alternate, so consecutive MFMAs are independent.
    {
      constexpr int PP = 16 / NM;   // probability pairs per step
      float psum = 0.f;
      uint32_t w[4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc_nxt[u][e] = 0.f;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int u = m & 1, ks = m >> 1;
        if (m + AH < NM) kq[m + AH] = kfrag(t + 1, m + AH);
        else vq[m + AH - NM] = vfrag(t, m + AH - NM);
        sc_nxt[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[m], qf[ks], sc_nxt[u], 0, 0, 0);
#pragma unroll
        for (int pp = 0; pp < PP; ++pp) {
          // pair idx: scores (hh * 8 + 2 e2, + 1) of 32 x 32 tile uu
          const int idx = m * PP + pp;
          const int uu = idx >> 3, hh = (idx >> 2) & 1, e2 = idx & 3;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc_cur[uu][hh * 8 + 2 * e2], sc, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc_cur[uu][hh * 8 + 2 * e2 + 1], sc, -m_run));
          psum += p0 + p1;
          w[e2] = pack_bf16x2(p0, p1);
          if (e2 == 3) {
            u32x4_t wv = {w[0], w[1], w[2], w[3]};
            pf[2 * uu + hh] = __builtin_bit_cast(bf16x8_t, wv);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      l_run += psum;
    }
    pv_tile(t);
#pragma unroll
    for (int u = 0; u < 2; ++u) sc_cur[u] = sc_nxt[u];
    DL_WAIT_VM(VMW);   // K(t + 2), V(t + 1)
    lds_barrier();
  }
  DL_WAIT_VM(0);       // no load into LDS outlives the loop
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  // training: P = exp2(s * sc - m_run) / l_tot = exp2(s * sc - lse)
  if (a.lse && half == 0) a.lse[bh * a.seq_pad + q] = q < a.seq ? m_run + __log2f(l_tot) : INFINITY;
  if constexpr (OUT == kFP8) {
    // E4M3 output with the delayed scale of the row's stream (image rows
    // oq[0], text rows oq[1]); each stream's amax is raised once per wave
    const bool img_row = q < a.l_img;
    flux_fp8_tensor* rec = img_row ? a.oq[0] : a.oq[1];
    uint32_t mx = 0;
    if (q < a.seq) {
      const float qs = fp8_scale(rec);
      uint8_t* out = reinterpret_cast<uint8_t*>(a.out) + (int64_t)b * a.out_bstride + (int64_t)q * a.out_ld + h * DH;
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = i * 32 + 8 * g + 4 * half;
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[e] = o[i][4 * g + e] * inv;
            mx = max(mx, abs_bits(y[e]));
          }
          *reinterpret_cast<uint32_t*>(out + d0) = f32x4_to_e4m3(y[0] * qs, y[1] * qs, y[2] * qs, y[3] * qs);
        }
    }
    const uint32_t m_img = wave_max_u32(img_row ? mx : 0u);
    const uint32_t m_txt = wave_max_u32(img_row ? 0u : mx);
    if (lane == 0) {
      if (m_img) fp8_amax_raise(a.oq[0], __uint_as_float(m_img));
      if (m_txt && a.oq[1]) fp8_amax_raise(a.oq[1], __uint_as_float(m_txt));
    }
  } else if (q < a.seq) {
    bf16_t* out = reinterpret_cast<bf16_t*>(a.out) + (int64_t)b * a.out_bstride + (int64_t)q * a.out_ld + h * DH;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = i * 32 + 8 * g + 4 * half;
        uint2 v;
        if constexpr (OUT == kF16) {
          v.x = pack_f16x2(o[i][4 * g] * inv, o[i][4 * g + 1] * inv);
          v.y = pack_f16x2(o[i][4 * g + 2] * inv, o[i][4 * g + 3] * inv);
        } else {
          v.x = pack_bf16x2(o[i][4 * g] * inv, o[i][4 * g + 1] * inv);
          v.y = pack_bf16x2(o[i][4 * g + 2] * inv, o[i][4 * g + 3] * inv);
        }
        *reinterpret_cast<uint2*>(out + d0) = v;
      }
  }
}

// fp32 kernel for the fp32 workloads: one thread per query, online softmax,
// keys and values read as broadcasts (every thread of the block walks the
// same key).
template <int DH>
__global__ void __launch_bounds__(64) attn_f32_kernel(AttnArgs a) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int q = blockIdx.x * 64 + threadIdx.x;
  const int64_t bh = (int64_t)b * a.heads + h;
  const float* Qh = reinterpret_cast<const float*>(a.qh) + bh * a.seq_pad * DH;
  const float* Kh = reinterpret_cast<const float*>(a.kh) + bh * a.seq_pad * DH;
  const float* Vt = reinterpret_cast<const float*>(a.vt) + bh * DH * a.seq_pad;
  float qv[DH], o[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    qv[d] = Qh[(int64_t)q * DH + d];
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < a.seq; ++j) {
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < DH; ++d) s += qv[d] * Kh[(int64_t)j * DH + d];
    s *= a.scale_log2;
    const float m_new = fmaxf(m, s);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(s - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int d = 0; d < DH; ++d) o[d] = o[d] * alpha + p * Vt[(int64_t)d * a.seq_pad + j];
    m = m_new;
  }
  if (q < a.seq) {
    float* out = reinterpret_cast<float*>(a.out) + (int64_t)b * a.out_bstride + (int64_t)q * a.out_ld + h * DH;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < DH; ++d) out[d] = o[d] * inv;
  }
}

// E4M3 kernel ("FP8 training for Flux models": fp8 attention, off by default):
// Q, K and V^T are E4M3 codes with one scale per tensor; S^T = K Q^T and
// O^T = V^T P^T run on v_mfma_f32_32x32x64_f8f6f4, the probabilities are
// packed to E4M3 (below 2^8 with the lazy max, inside E4M3's range).  Same
// block shape, placement, lazy max and software pipeline as the bf16 kernel.
// The MFMA sums its 64 products in an order of its own; A and B only have to
// give each lane half and register byte the same k.  For S^T lane half h holds
// head-dim bytes [64 s + 32 h, + 32) of k step s in both operands.  For O^T
// the B operand is the lane's 32 probabilities in accumulator order, i.e. keys
// 32 u + 8 (e / 4) + 4 h + e % 4 for byte 16 u + e; V^T tiles are stored with
// their columns permuted in groups of 4 keys so that these 32 keys are the
// 32 contiguous bytes [32 h, 32 h + 32) of the lane's V^T row.
typedef int i32x8a_t __attribute__((ext_vector_type(8)));

__global__ void __launch_bounds__(512, 1) attn_fp8_kernel(AttnArgs a) {
  constexpr int DH = 128, KT = 64, QW = 32, NW = 8, QB = NW * QW, DT = DH / 32;
  constexpr int KLD = DH + 16;    // K tile row stride (bytes): 16 lanes of a read hit distinct bank groups
  constexpr int VLD = KT + 16;    // V^T tile row stride (bytes)
  constexpr float kLazy = 8.0f;
  __shared__ __attribute__((aligned(16))) uint8_t Ks[2][KT * KLD];
  __shared__ __attribute__((aligned(16))) uint8_t Vs[2][DH * VLD];
  const int nq = a.seq_pad / QB;
  const int total = a.batch * a.heads * nq;
  const int per = (total + 7) / 8;
  const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (item >= total) return;
  const int qb = item % nq;
  const int64_t bh = item / nq;
  const int b = (int)(bh / a.heads), h = (int)(bh % a.heads);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const uint8_t* Qh = reinterpret_cast<const uint8_t*>(a.qh) + bh * a.seq_pad * DH;
  const uint8_t* Kh = reinterpret_cast<const uint8_t*>(a.kh) + bh * a.seq_pad * DH;
  const uint8_t* Vt = reinterpret_cast<const uint8_t*>(a.vt) + bh * DH * a.seq_pad;

  const int q = qb * QB + wave * QW + l32;
  i32x8a_t qf[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) qf[st] = *reinterpret_cast<const i32x8a_t*>(Qh + (int64_t)q * DH + 64 * st + 32 * half);
  f32x16_t o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = a.scale_log2 * fp8_scale_inv(a.sq) * fp8_scale_inv(a.sk);

  auto mma = [](i32x8a_t x, i32x8a_t y, f32x16_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
  };
  auto kfrag = [&](int t, int u, int st) {
    return *reinterpret_cast<const i32x8a_t*>(&Ks[t & 1][(u * 32 + l32) * KLD + 64 * st + 32 * half]);
  };
  // S^T of tile t: sv[u][e] is the score of key t*64 + 32u + 8(e/4) + 4 half + e%4
  auto s_tile = [&](int t, f32x16_t (&sv)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sv[u][e] = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st) sv[u] = mma(kfrag(t, u, st), qf[st], sv[u]);
    }
  };
  auto softmax_max = [&](int t, f32x16_t (&sv)[2]) {
    if ((t + 1) * KT > a.seq) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = t * KT + 32 * u + 8 * (e >> 2) + 4 * half + (e & 3);
          if (key >= a.seq) sv[u][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sv[u][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_tile = mx * sc;
    if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
      m_run = m_new;
    }
  };
  uint32_t pw[8];   // E4M3 probabilities of the current tile: dword 4u + g holds elements 4g..4g+3 of tile u
  auto pv_tile = [&](int t) {
    const i32x8a_t pb = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
#pragma unroll
    for (int i = 0; i < DT; ++i) {
      const i32x8a_t vf = *reinterpret_cast<const i32x8a_t*>(&Vs[t & 1][(i * 32 + l32) * VLD + 32 * half]);
      o[i] = mma(vf, pb, o[i]);
    }
  };
  u32x4_t rk, rv;
  const int kr = tid >> 3, kc = (tid & 7) * 16;    // K tile: 64 rows x 8 chunks
  const int vd = tid >> 2, va = tid & 3;           // V^T tile: 128 rows x 4 chunks of 16 keys
  auto gload_k = [&](int j) { rk = *reinterpret_cast<const u32x4_t*>(Kh + (int64_t)(j * KT + kr) * DH + kc); };
  auto gload_v = [&](int j) { rv = *reinterpret_cast<const u32x4_t*>(Vt + (int64_t)vd * a.seq_pad + j * KT + va * 16); };
  auto lstore_k = [&](int j) { *reinterpret_cast<u32x4_t*>(&Ks[j & 1][kr * KLD + kc]) = rk; };
  auto lstore_v = [&](int j) {
    // keys 16 va + 4 g2 .. + 4 go to column 32 (g2 & 1) + 16 (va >> 1) + 4 ((2 va + (g2 >> 1)) & 3)
#pragma unroll
    for (int g2 = 0; g2 < 4; ++g2) {
      const int col = 32 * (g2 & 1) + 16 * (va >> 1) + 4 * ((2 * va + (g2 >> 1)) & 3);
      *reinterpret_cast<uint32_t*>(&Vs[j & 1][vd * VLD + col]) = rv[g2];
    }
  };
  const int ntiles = (a.seq + KT - 1) / KT;
  gload_k(0);
  gload_v(0);
  lstore_k(0);
  lstore_v(0);
  if (ntiles > 1) {
    gload_k(1);
    lstore_k(1);
  }
  if (ntiles > 2) gload_k(2);
  if (ntiles > 1) gload_v(1);
  __syncthreads();
  f32x16_t sc_cur[2], sc_nxt[2];
  s_tile(0, sc_cur);
  // iteration 0 overwrites K(0)'s buffer with K(2): every wave must have read K(0) first
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    softmax_max(t, sc_cur);
    // S(t + 1) (from a resident buffer, discarded, on the last tile) with the
    // exponentials of tile t in its MFMA shadow: step m issues one MFMA and
    // the 8 probabilities of elements 8 (m & 1) .. + 8 of tile m >> 1
    {
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc_nxt[u][e] = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int u = m & 1, st = m >> 1;
        sc_nxt[u] = mma(kfrag(t + 1, u, st), qf[st], sc_nxt[u]);
        const int uu = m >> 1;
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const int g = 2 * (m & 1) + gg;
          float p[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            p[c] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc_cur[uu][4 * g + c], sc, -m_run));
            psum += p[c];
          }
          pw[4 * uu + g] = f32x4_to_e4m3(p[0], p[1], p[2], p[3]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      l_run += psum;
    }
    pv_tile(t);
    if (t + 2 < ntiles) lstore_k(t + 2);
    if (t + 1 < ntiles) lstore_v(t + 1);
    if (t + 3 < ntiles) gload_k(t + 3);
    if (t + 2 < ntiles) gload_v(t + 2);
#pragma unroll
    for (int u = 0; u < 2; ++u) sc_cur[u] = sc_nxt[u];
    // K(t + 3) and V(t + 2) are only stored to LDS in the next iteration:
    // the barrier waits for the LDS stores, not for these loads
    lds_barrier();
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = fp8_scale_inv(a.sv) / l_tot;
  if (q < a.seq) {
    bf16_t* out = reinterpret_cast<bf16_t*>(a.out) + (int64_t)b * a.out_bstride + (int64_t)q * a.out_ld + h * DH;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = i * 32 + 8 * g + 4 * half;
        uint2 v;
        v.x = pack_bf16x2(o[i][4 * g] * inv, o[i][4 * g + 1] * inv);
        v.y = pack_bf16x2(o[i][4 * g + 2] * inv, o[i][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(out + d0) = v;
      }
  }
}

hipError_t launch_attention(const AttnArgs& a, int dtype, int out_dtype, hipStream_t stream) {
  TimingScope ts(kKcAttn, stream, 4.0 * a.batch * a.heads * (double)a.seq * a.seq * a.head_dim);
  if (dtype == kFP8) {
    if (a.head_dim != 128 || out_dtype != kBF16 || !a.sq || !a.sk || !a.sv) return hipErrorInvalidValue;
    const int items = a.batch * a.heads * (a.seq_pad / 256);
    const dim3 grid(((items + 7) / 8) * 8);
    hipLaunchKernelGGL(attn_fp8_kernel, grid, dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  if (dtype == kBF16) {
    // K and V^T of one (batch, head) are addressed by 32-bit byte offsets
    if ((int64_t)a.seq_pad * a.head_dim * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    // one block per 256 queries of a (batch, head), rounded up to whole XCD
    // groups (blocks past the work exit at once)
    const int items = a.batch * a.heads * (a.seq_pad / 256);
    const dim3 grid(((items + 7) / 8) * 8);
    if (a.head_dim == 128) {
      if (out_dtype == kF16)
        hipLaunchKernelGGL((attn_bf16_kernel<128, kF16>), grid, dim3(512), 0, stream, a);
      else if (out_dtype == kFP8)
        hipLaunchKernelGGL((attn_bf16_kernel<128, kFP8>), grid, dim3(512), 0, stream, a);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<128, kBF16>), grid, dim3(512), 0, stream, a);
    } else {
      if (out_dtype == kF16)
        hipLaunchKernelGGL((attn_bf16_kernel<64, kF16>), grid, dim3(512), 0, stream, a);
      else if (out_dtype == kFP8)
        hipLaunchKernelGGL((attn_bf16_kernel<64, kFP8>), grid, dim3(512), 0, stream, a);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<64, kBF16>), grid, dim3(512), 0, stream, a);
    }
  } else {
    const dim3 grid(a.seq_pad / 64, a.heads, a.batch);
    if (a.head_dim == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace flux
