// Internal launch interface of libflux: argument structs and host launchers.
// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/flux.h"

namespace flux {

// Element types.  GEMM "operand type": kF32 = fp32 FMA kernel; kBF16 = bf16 A
// times bf16 W on bf16 MFMA; kF16 = fp16 A times bf16 W converted to fp16 in
// the LDS staging, on fp16 MFMA.
enum Dtype : int { kF32 = 0, kBF16 = 1, kF16 = 2 };
// GEMM operand type with fp16 weights already in memory (fp16 x fp16 MFMA)
constexpr int kF16W = 3;
// OCP E4M3FN bytes: as a GEMM operand type, e4m3 activations times e4m3
// weights on the fp8 MFMA; as an output type, values quantized with the
// scale of an flux_fp8_tensor record whose amax they raise.
constexpr int kFP8 = 4;
// MXFP8 (OCP MX, E4M3 elements): as a GEMM operand type, E4M3 bytes of A and W
// with one E8M0 scale per 32 values along K, applied by the scaled MFMA.
constexpr int kMXFP8 = 5;
// MXFP4 (OCP MX, E2M1 elements): as a GEMM operand type, A and W rows of
// packed E2M1 codes (two per byte, the even element in the low nibble; K counts
// values, the row strides amap.ld and ldw count bytes) with one E8M0 scale per
// 32 values along K in the layout of launch_mxfp4_quantize.
constexpr int kMXFP4 = 6;

// ---------------------------------------------------------------------------
// Row addressing shared by the token-wise kernels.  A logical row r of a
// segment with `seg` rows per sample lives at
//     base + (r / seg) * bstride + (r % seg) * ld      (elements)
// which covers contiguous [B*L, ld] buffers, per-sample strided residual
// streams and the image / text halves of a joint [B, L, ld] buffer.
// ---------------------------------------------------------------------------
struct RowMap {
  int64_t bstride;
  int64_t ld;
  int32_t seg;
};

// ---------------------------- GEMM (C = A W^T) -----------------------------
enum EpiKind : int {
  kEpiStore = 0,      // out0 = T0(acc + bias)                  (T0 = out0_dt)
  kEpiGelu = 1,       // out0 = T0(GELU(acc + bias))
  kEpiResid = 2,      // out0 (float) += gate[b, col] * (acc + bias)
  kEpiStoreF32 = 3,   // out0 (float) = acc + bias            (column stride col_stride)
  kEpiSplitGelu = 4,  // col < n_split: out0 = T0(acc + bias); else out1[col - n_split] = T1(GELU(acc + bias))
  // The attention operands straight from the q|k|v projection (persistent
  // kernel, head_dim 128): columns [0, D) are q, [D, 2D) k, [2D, 3D) v of
  // `QkvOut`; q and k rows get RMSNorm (per head, scale gq / gk) and RoPE,
  // then go to the head-major layouts qh / kh; v goes to vt transposed.
  kEpiQkv = 5,
  // kEpiQkv on columns < n_split (= 3D), GELU to out1 on the rest (single block)
  kEpiQkvSplitGelu = 6,
};

// Destination of the kEpiQkv epilogues: the layouts launch_prep writes.
struct QkvOut {
  void* qh; void* kh;                   // [B, heads, seq_pad, 128] bf16
  void* vt;                             // [B, heads, 128, seq_pad] bf16
  const float* gq; const float* gk;     // RMSNorm scales [128]
  const float* rope;                    // [B, seq, 64, 2] (cos, sin) per pair
  int32_t heads, seq, seq_pad;          // joint sequence
  int32_t tok0;                         // joint position of this problem's row l = 0 of a sample
  float eps;
};

struct GemmProblem {
  const void* A;  RowMap amap;          // [M, K] rows
  const void* W;  int64_t ldw;          // [N, K]
  const void* bias;                     // [N] or null (operand type)
  int32_t M, N, K;
  int32_t epi;
  void* out0;     RowMap omap0;  int64_t col_stride0;
  void* out1;     RowMap omap1;  int32_t n_split;
  const float* gate; int64_t gate_bstride;   // gate[(r / omap0.seg) * gate_bstride + col]
  int32_t out0_dt, out1_dt;             // Dtype of out0 / out1 for the store epilogues
  const flux_fp8_tensor* qa;            // kFP8 operands: records A and W were quantized with;
  const flux_fp8_tensor* qw;            //   the accumulator is multiplied by both scale_inv
  flux_fp8_tensor* qo;                  // kFP8 output (out0 of kEpiGelu, out1 of kEpiSplitGelu)
  const uint8_t* sa;                    // kMXFP8 / kMXFP4 operands: E8M0 block scales of A and W in
  const uint8_t* sb;                    //   the GEMM layout of their quantizer (null otherwise)
  QkvOut qkv;                           // kEpiQkv / kEpiQkvSplitGelu (rows map to samples by omap0.seg)
  int32_t tile_begin;                   // filled by the launcher
  int32_t tiles_n;                      // filled by the launcher
};

constexpr int kMaxGemmProblems = 2;
struct GemmBatch {
  GemmProblem p[kMaxGemmProblems];
  int32_t count;
  int32_t total_tiles;
  // Optional split-K scratch for a single problem too small to fill the GPU
  // with tiles: [kGemmMaxSplit, M, N] fp32 partial sums (null: no split).
  float* partials;
  int32_t ksplit;   // filled by the launcher
  // Stream-K tail of the persistent 16-bit kernel (sk_part null: off).  The
  // tiles past the grid's last full round are cut along K into equal shares
  // of super-stages, one contiguous share per block; a block hands the part
  // of a tile it does not finish to the block that does, through sk_part
  // (kGemmSkSlotFloats fp32 per block) and sk_flag (one int per block, zeroed
  // by the launcher before each launch).  Needs kGemmSkMaxGrid slots.
  float* sk_part;
  int32_t* sk_flag;
  int32_t sk_tail;    // filled by the launcher: first tile of the tail
  int32_t sk_units;   // filled by the launcher: tail tiles x super-stages (0: no tail split)
  int32_t sk_spin;    // polls an owner waits for a share before computing it itself (0: default)
};
constexpr int kGemmMaxSplit = 8;
constexpr int kGemmSkMaxGrid = 256;
constexpr int64_t kGemmSkSlotFloats = 256 * 256;
constexpr int64_t kGemmSkBytes = kGemmSkMaxGrid * kGemmSkSlotFloats * 4 + 1024;   // partials + flags

hipError_t launch_gemm(GemmBatch batch, int op, hipStream_t stream);
// Stream-K tail of the persistent 16-bit GEMM: mode 1 on, 0 off, < 0 leave;
// spin > 0 sets the owner's poll limit (0: default).  Returns the previous mode.
int gemm_stream_k(int mode, int spin);
// True when launch_gemm runs this batch (16-bit or E4M3 operands) on the
// persistent 256 x 256 kernel, the only one with the kEpiQkv epilogues.
bool gemm_is_persistent(const GemmBatch& batch, int op);
// Zero the padded rows [seq, seq_pad) of qh / kh and the padded columns of vt
// (the attention kernels read them; kEpiQkv writes real rows only).
hipError_t launch_attn_pad_zero(void* qh, void* kh, void* vt, int batch, int heads, int seq, int seq_pad,
                                hipStream_t stream);

// ------------------------------ LN + modulate ------------------------------
struct LnSeg {
  const float* x;  RowMap xmap;         // fp32 residual rows
  void* out;       RowMap omap;         // T rows
  const float* shift; const float* scale; int64_t mod_bstride;   // [b * mod_bstride + col]
  flux_fp8_tensor* q;                   // kFP8 output: scale source and amax destination
  int32_t rows;                         // B * seg
};
struct LnArgs {
  LnSeg s[2];
  int32_t count;
  int32_t dim;
  float eps;
};
hipError_t launch_ln_mod(const LnArgs& a, int out_dtype, hipStream_t stream);

// ------------------------------- GEMV (M = B) -------------------------------
struct GemvProblem {
  const void* W; const void* bias;      // [N, K], [N] (operand type)
  int32_t N, K;
  const float* x; int64_t x_bstride;    // input [B, K] float
  float* y; int64_t y_bstride;          // output [B, N] float
  int32_t act_silu;                     // apply SiLU to x first
  int32_t accumulate;                   // y += instead of y =
};
struct GemvBatch {
  GemvProblem p[2];
  int32_t count;
  int32_t batch;
};
hipError_t launch_gemv(const GemvBatch& a, int dtype, hipStream_t stream);

// ------------------ q/k RMSNorm + RoPE + head-major layout ------------------
struct PrepArgs {
  const void* src_q; const void* src_k; const void* src_v; // token rows (operand type)
  int64_t src_bstride; int64_t src_ld;
  int32_t batch, seq, seq_pad, heads, head_dim, l_img;
  const float* gq_img; const float* gk_img;               // RMSNorm scales (null -> no norm)
  const float* gq_txt; const float* gk_txt;               // rows >= l_img use these
  const float* rope;                                      // [B, seq, head_dim/2, 2] or null
  float eps;
  void* qh; void* kh;                                     // [B, H, seq_pad, head_dim]
  void* vt;                                               // [B, H, head_dim, seq_pad]
};
hipError_t launch_prep(const PrepArgs& a, int dtype, hipStream_t stream);

// -------------------------------- attention --------------------------------
struct AttnArgs {
  const void* qh; const void* kh; const void* vt;         // as written by launch_prep
  void* out; int64_t out_bstride; int64_t out_ld;         // [B, seq, ...], head h at column h*head_dim
  int32_t batch, seq, seq_pad, heads, head_dim;
  float scale_log2;                                       // log2(e) / sqrt(head_dim)
  flux_fp8_tensor* oq[2];                                 // kFP8 output: rows < l_img use oq[0], others oq[1]
  int32_t l_img;
  float* lse;   // optional [B, H, seq_pad]: log2-domain log-sum-exp of the scaled scores per query
                //   (+inf for queries >= seq), so that P = exp2(s * scale_log2 - lse); bf16 kernel only
  // kFP8 inputs (head_dim 128, bf16 output): qh, kh, vt hold E4M3 codes quantized
  // with the scales of these records; scores and output are rescaled by scale_inv
  const flux_fp8_tensor* sq; const flux_fp8_tensor* sk; const flux_fp8_tensor* sv;
};
// in_dtype kBF16 (bf16 MFMA), kFP8 (E4M3 codes on the fp8 MFMA, bf16 output) or
// kF32; out_dtype kBF16 / kF16 / kFP8 with bf16 inputs, kF32 with fp32 inputs
hipError_t launch_attention(const AttnArgs& a, int in_dtype, int out_dtype, hipStream_t stream);

// ------------------------------- backward --------------------------------
// dst[z][c][r] = bf16(src[z][r][c]) for r < R, c < C; zero for R <= r < R_fill.
// src_dtype kF32, kBF16 or kF16.  C, R_fill, the source row stride and dst_ld
// multiples of 4.
struct TransposeArgs {
  const void* src; int64_t src_zstride; RowMap smap;     // row r of slice z at src + z * src_zstride + smap(r)
  void* dst; int64_t dst_zstride; int64_t dst_ld;
  int32_t R, C, R_fill, Z;
};
hipError_t launch_transpose(const TransposeArgs& a, int src_dtype, hipStream_t stream);

// out[z * out_zstride + c] (mode 0 =, 1 +=) sum over the R rows of sample z
// (global row z * R + r addressed through amap / bmap) of A (* Bm); fixed order.
// part: scratch of Z * nrb * C floats; C % 4 == 0.
struct ColsumArgs {
  const void* A; RowMap amap;
  const float* Bm; RowMap bmap;          // optional elementwise factor (fp32)
  int32_t R, C, Z;
  int32_t rpb, nrb;                      // rows per partial, partial count (rpb * nrb >= R)
  float* part;
};
hipError_t launch_colsum(ColsumArgs a, int a_dtype, float* out, int64_t out_zstride, int mode, hipStream_t stream);

struct ReduceArgs {
  const float* part; int32_t np; int32_t C; int32_t Z;
  int64_t pstride;                       // floats from one partial to the next (0: C)
  float* out; int64_t out_zstride;
  int32_t mode;                          // 0 store, 1 add, 2 add times SiLU'(aux), 3 store times SiLU'(aux)
  const float* aux; int64_t aux_zstride;
};
// the partials are scratch: the fixed-order tree sums them in place
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream);

enum EwOp : int { kEwGateBwd = 0, kEwGeluBwd = 1, kEwGelu = 2, kEwGateAdd = 3 };
struct EwArgs {
  int32_t op;
  const void* x; RowMap xmap;
  const void* y; RowMap ymap;
  void* out; RowMap omap;
  const float* gate; int64_t gate_bstride;   // gate[(r / xmap.seg) * gate_bstride + c]
  int64_t rows; int32_t C;                   // C % 4 == 0
  int32_t f16;                               // 16-bit operands that are fp16 (else bf16): 1 x, 2 y, 4 out
};
hipError_t launch_elementwise(const EwArgs& a, hipStream_t stream);

// LayerNorm-modulate backward over `batch` samples of `seg` rows each:
// dx (fp32, +=), dshift / dscale (fp32, written at [b * mod_bstride + c]).
// part_sh / part_sc: scratch of batch * ln_bwd_blocks(seg, batch) * 4 * dim floats each.
struct LnBwdArgs {
  const float* x; RowMap xmap;
  const float* dh; RowMap dhmap;
  float* dx; RowMap dxmap;
  const float* scale; int64_t mod_bstride;
  float* dshift; float* dscale;
  float* part_sh; float* part_sc;
  int32_t seg, batch, rpb;
  float eps;
};
int ln_bwd_blocks(int seg, int batch);
hipError_t launch_ln_mod_bwd(LnBwdArgs a, int dim, hipStream_t stream);

// q / k RMSNorm + RoPE backward (head_dim 128).  dq, dk, dv fp32 head-major
// [B, H, seq_pad, 128]; src: the forward's q|k|v token rows (bf16, q at column
// 0, k at D, v at 2D); dst: bf16 token rows of the same layout.  part:
// prep_bwd_parts(...) * 512 floats, [block][stream][q / k][d].
struct PrepBwdArgs {
  const float* dq; const float* dk; const float* dv;
  const void* src; int64_t src_bstride; int64_t src_ld;
  void* dst; int64_t dst_bstride; int64_t dst_ld;
  const float* gq_img; const float* gk_img; const float* gq_txt; const float* gk_txt;
  const float* rope;
  int32_t batch, seq, seq_pad, heads, l_img;
  float eps;
  float* part;
};
int prep_bwd_parts(int batch, int seq, int heads);
hipError_t launch_prep_bwd(const PrepBwdArgs& a, hipStream_t stream);

// Attention backward (bf16, head_dim 128).  Inputs head-major bf16: qh, kh, vh
// [B, H, seq_pad, 128], qt, kt [B, H, 128, seq_pad]; lse [B, H, seq_pad] from
// the forward; dout bf16 and o bf16 or fp16 (o_f16) token rows (head h at
// column h * 128).  Scratch:
// doh [B, H, seq_pad, 128], dot [B, H, 128, seq_pad] bf16, dd [B, H, seq_pad]
// fp32.  Outputs fp32 head-major dq, dk, dv [B, H, seq_pad, 128] (rows < seq).
struct AttnBwdArgs {
  const void* qh; const void* kh; const void* vh; const void* qt; const void* kt;
  const float* lse;
  const void* dout; int64_t dout_bstride; int64_t dout_ld;
  const void* o; int64_t o_bstride; int64_t o_ld;
  void* doh; void* dot; float* dd;
  float* dq; float* dk; float* dv;
  int32_t batch, seq, seq_pad, heads;
  float scale_log2, scale;
  int32_t o_f16;                         // o is fp16 (else bf16)
};
hipError_t launch_attention_bwd(const AttnBwdArgs& a, hipStream_t stream);

// adaLN modulation backward: m = W SiLU(vec) + b, W [N, K] (weight dtype),
// dm [B, N] (row stride dm_bstride).  dw [N, K], db [N] written; dvec [B, K]
// += SiLU'(vec) * W^T dm.  part: scratch of batch * nrc * K floats; K % 4 == 0.
struct ModBwdArgs {
  const void* w; const float* vec; const float* dm; int64_t dm_bstride;
  float* dw; float* db; float* dvec;     // dvec may be NULL (no input gradient)
  int32_t N, K, batch, nrc, rpc;
  int32_t silu_in;                       // 1: m = W SiLU(vec) + b; 0: m = W vec + b (dW only, dvec must be NULL)
  int32_t dvec_store;                    // 1: dvec = instead of +=
  float* part;
};
hipError_t launch_mod_bwd(ModBwdArgs a, int w_dtype, hipStream_t stream);

// dv = (2 / n) (v - (z1 - z0)) over n fp32 elements (velocity MSE gradient)
// dW = sum_b g_b dvec_b and db = sum_b dvec_b of the guidance embedding (fp32)
hipError_t launch_guidance_bwd(const float* dvec, const float* g, int batch, int D, float* dw, float* db,
                               hipStream_t stream);
hipError_t launch_rf_loss_grad(const float* v, const float* z0, const float* z1, float* dv, int64_t n,
                               hipStream_t stream);

// ------------------------------ small kernels ------------------------------
hipError_t launch_rope_table(const float* ids, int batch, int seq, const int32_t axes[3], float theta,
                             float* table, hipStream_t stream);
hipError_t launch_timestep_embed(const float* t, int batch, int dim, float time_factor, float max_period,
                                 float* out, hipStream_t stream);
hipError_t launch_patchify(const float* z, int batch, int channels, int hw, void* out, int dtype,
                           hipStream_t stream);
// src [batch, rows, width] (kBF16 or kF32, width % 4 == 0) -> fp32 rows at dst + b * dst_bstride
hipError_t launch_rows_to_f32(const void* src, int batch, int rows, int width, int dtype, float* dst,
                              int64_t dst_bstride, hipStream_t stream);
hipError_t launch_rf_noise(int batch, int64_t n, const float* z0, const float* z1, const float* t,
                           float* zt, float* vt, hipStream_t stream);
hipError_t launch_rf_loss(int batch, int64_t n, const float* z0, const float* z1, const float* vpred,
                          float* loss, float* loss_ps, double* partials, int parts_per_sample,
                          hipStream_t stream);
int rf_parts_per_sample(int64_t n);
// z <- z - dt * (cfg ? v_u + w (v_c - v_u) : v); z also copied into `copies`
// batch-halves of zm; tm[0..tm_n) = t_next
hipError_t launch_euler_step(int batch, int64_t n, const float* v, int cfg, float w, float dt, float* z, float* zm,
                             int copies, float t_next, float* tm, int tm_n, hipStream_t stream);
// vec[b, :] += g[b] * W[:, 0] + bias  (W, bias in `dtype`, kBF16 or kF32)
hipError_t launch_guidance_embed(int batch, int dim, const float* g, const void* w, const void* bias, int dtype,
                                 float* vec, hipStream_t stream);
hipError_t launch_convert_bf16_f16(const void* src, void* dst, int64_t n, hipStream_t stream);

// --------------------------------- MXFP8 -----------------------------------
// Block-scaled E4M3 of rows x k values (k % 64 == 0): codes [rows, k] row-major
// and one E8M0 byte per 32 values along k, stored for the persistent GEMM:
// the byte of (row, block kb) sits at
//   (((row / 128) * (k / 64) + kb / 2) * 2 + kb % 2) * 128 + (row % 32) * 4 + (row / 32) % 4,
// so one dword per lane holds the scales of its four 32-row fragments for one
// 64-wide k step.  Rows are padded to a multiple of 256 (pad rows: zeros).
inline size_t mx_scale_bytes(int64_t rows, int64_t k) { return (size_t)(((rows + 255) / 256) * 256 * (k / 32)); }
hipError_t launch_mx_quantize(const void* src, int src_dtype, int rows, int k, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream);
// MXFP4: codes [rows, k / 2] (two E2M1 codes a byte, the even element in the
// low nibble) and one E8M0 byte per 32 values, k a multiple of 128.  The scale
// layout serves the two fp4 MFMAs of one 128-value stage of the persistent
// GEMM with a single 8-byte load per lane: the byte of (row, block kb) sits at
//   ((row / 128) * (k / 128) + kb / 4) * 512 + (kb % 2) * 256 + (row % 32) * 8
//     + ((kb % 4) / 2) * 4 + (row / 32) % 4.
// The byte count is that of mx_scale_bytes (rows padded to 256).
// Blockwise E4M3 (tiles of tile_rows x 128 along k, tile_rows 1 or 128, one
// power-of-two scale each): codes [rows, k] and E8M0 bytes 127 - e in the
// mx_quantize layout, so the MXFP8 GEMM takes the operands as they are.
hipError_t launch_fp8_block_quantize(const void* src, int src_dtype, int rows, int k, int tile_rows, uint8_t* codes,
                                     uint8_t* scales, hipStream_t stream);
hipError_t launch_mxfp4_quantize(const void* src, int src_dtype, int rows, int k, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream);

// ---------------------------------- fp8 ------------------------------------
// dst = e4m3(src * scale(rec)); rec->amax_bits raised to max |src|.  src_dtype kF32 or kBF16.
hipError_t launch_fp8_quantize(const void* src, int src_dtype, int64_t n, flux_fp8_tensor* rec, uint8_t* dst,
                               hipStream_t stream);
// current scaling: rec->amax = max |src|, then scale = fp32(448 / amax), scale_inv = 1 / scale
hipError_t launch_fp8_current_scale(const void* src, int src_dtype, int64_t n, flux_fp8_tensor* rec,
                                    hipStream_t stream);
// delayed-scaling update of n records (algo 0 most_recent, 1 max)
hipError_t launch_fp8_update(flux_fp8_tensor* rec, int n, int algo, int margin, hipStream_t stream);

}  // namespace flux
