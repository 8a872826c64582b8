// libflux C ABI, training: the block forwards that keep what the backward
// needs, and the block backwards under the rectified-flow objective ("Flux
// architecture deep dive", Flow matching framework: predict the velocity,
// mean squared error, backpropagate; Model components: the double and single
// blocks differentiated step by step).
//
// Weights are bf16; head_dim 128.  The forward's block linears take fp16
// activation operands (LayerNorm-modulate, attention and GELU outputs) times
// the bf16 weights converted to fp16 per tile, on the fp16 MFMA with fp32
// accumulation, as the inference forward does; the q|k|v projection is kept
// in bf16 for the q / k norm, and the residual stream and every gradient are
// fp32 or bf16.  Data gradients of a linear y = x W^T are dy W (bf16 MFMA,
// the forward GEMM with the transposed weight), weight gradients dy^T x (the
// same GEMM on the transposed activations, rounded to bf16, the token axis
// zero-padded to a multiple of 64).
#include "api_common.h"

using namespace flux;
using namespace flux::api;

namespace {

constexpr int64_t kTokPad = 64;   // token axis of the weight-gradient GEMMs

int64_t tok_pad(int64_t t) { return round_up(t > 0 ? t : 1, kTokPad); }

flux_status check_train_dims(const flux_dims* d) {
  flux_status s = check_dims(d);
  if (s != FLUX_OK) return s;
  if (d->precision != FLUX_PREC_BF16 || d->weights_f16)
    return fail(FLUX_ERR_UNSUPPORTED, "training runs in FLUX_PREC_BF16 with bf16 weights");
  if (d->head_dim != 128) return fail(FLUX_ERR_UNSUPPORTED, "training needs head_dim 128 (got %d)", d->head_dim);
  return FLUX_OK;
}

// ------------------------------ saved activations ------------------------------
struct SingleSaved {
  float* mod;      // [B, 3D]
  float* x0;       // [B, L, D] block input
  void* h;         // [B, L, D]      fp16 LN-modulate output
  void* qkv;       // [B, L, 3D]     bf16 q|k|v columns of linear1
  void* a;         // [B, L, F]      fp16 MLP pre-activation columns of linear1
  void* cat;       // [B, L, D + F]  fp16 attention output | GELU(a)
  void* qh; void* kh; void* vt;   // attention operands
  float* lse;      // [B, H, Lp]
  float* y;        // [B, L, D] linear2 output before the gate
  size_t bytes;
};

SingleSaved single_saved(const flux_dims* d, void* base) {
  Carve c(base);
  SingleSaved s{};
  const int64_t B = d->batch, L = (int64_t)d->l_img + d->l_txt, D = d->hidden, F = d->mlp_hidden, Lp = seq_pad_of(L);
  s.mod = static_cast<float*>(c.take(B * 3 * D * 4));
  s.x0 = static_cast<float*>(c.take(B * L * D * 4));
  s.h = c.take(B * L * D * 2);
  s.qkv = c.take(B * L * 3 * D * 2);
  s.a = c.take(B * L * F * 2);
  s.cat = c.take(B * L * (D + F) * 2);
  s.qh = c.take(B * d->heads * Lp * 128 * 2);
  s.kh = c.take(B * d->heads * Lp * 128 * 2);
  s.vt = c.take(B * d->heads * Lp * 128 * 2);
  s.lse = static_cast<float*>(c.take(B * d->heads * Lp * 4));
  s.y = static_cast<float*>(c.take(B * L * D * 4));
  s.bytes = (size_t)round_up((int64_t)c.off, 256);
  return s;
}

struct BlockSaved {   // joint [B, L, .] rows, image rows first
  float* mod[2];      // [B, 6D] per stream
  float* x0; float* x1;   // residual before the block and after the attention half
  void* h1; void* qkv; void* o; void* h2; void* a1; void* u;   // fp16 but qkv (bf16)
  float* y1; float* y2;   // projection and fc2 outputs before their gates
  void* qh; void* kh; void* vt; float* lse;
  size_t bytes;
};

BlockSaved block_saved(const flux_dims* d, void* base) {
  Carve c(base);
  BlockSaved s{};
  const int64_t B = d->batch, L = (int64_t)d->l_img + d->l_txt, D = d->hidden, F = d->mlp_hidden, Lp = seq_pad_of(L);
  s.mod[0] = static_cast<float*>(c.take(B * 6 * D * 4));
  s.mod[1] = static_cast<float*>(c.take(B * 6 * D * 4));
  s.x0 = static_cast<float*>(c.take(B * L * D * 4));
  s.x1 = static_cast<float*>(c.take(B * L * D * 4));
  s.h1 = c.take(B * L * D * 2);
  s.qkv = c.take(B * L * 3 * D * 2);
  s.o = c.take(B * L * D * 2);
  s.h2 = c.take(B * L * D * 2);
  s.a1 = c.take(B * L * F * 2);
  s.u = c.take(B * L * F * 2);
  s.y1 = static_cast<float*>(c.take(B * L * D * 4));
  s.y2 = static_cast<float*>(c.take(B * L * D * 4));
  s.qh = c.take(B * d->heads * Lp * 128 * 2);
  s.kh = c.take(B * d->heads * Lp * 128 * 2);
  s.vt = c.take(B * d->heads * Lp * 128 * 2);
  s.lse = static_cast<float*>(c.take(B * d->heads * Lp * 4));
  s.bytes = (size_t)round_up((int64_t)c.off, 256);
  return s;
}

// --------------------------- backward workspaces ---------------------------
struct AttnWs {
  void* qt; void* kt; void* vh; void* doh; void* dot; float* dd;
  float* dq; float* dk; float* dv;
};

AttnWs attn_ws(Carve& c, int64_t B, int64_t H, int64_t Lp) {
  AttnWs w{};
  const int64_t n = B * H * Lp * 128;
  w.qt = c.take(n * 2); w.kt = c.take(n * 2); w.vh = c.take(n * 2);
  w.doh = c.take(n * 2); w.dot = c.take(n * 2);
  w.dd = static_cast<float*>(c.take(B * H * Lp * 4));
  w.dq = static_cast<float*>(c.take(n * 4)); w.dk = static_cast<float*>(c.take(n * 4));
  w.dv = static_cast<float*>(c.take(n * 4));
  return w;
}

constexpr int kColParts = 64;    // row partials of a column sum
constexpr int kModParts = 256;   // row chunks of the modulation GEMV transpose

struct Parts {
  float* col; float* ln_sh; float* ln_sc; float* prep; float* mod;
};

Parts parts_ws(Carve& c, const flux_dims* d, int64_t maxC, int64_t kD) {
  Parts p{};
  const int64_t B = d->batch, L = (int64_t)d->l_img + d->l_txt, D = d->hidden;
  p.col = static_cast<float*>(c.take(B * kColParts * maxC * 4));
  const int64_t ln_parts = (int64_t)B * ln_bwd_blocks((int)L, (int)B) * 4 * D;   // worst case: one stream of L rows
  p.ln_sh = static_cast<float*>(c.take(ln_parts * 4));
  p.ln_sc = static_cast<float*>(c.take(ln_parts * 4));
  p.prep = static_cast<float*>(c.take((int64_t)prep_bwd_parts((int)B, (int)L, d->heads) * 512 * 4));
  p.mod = static_cast<float*>(c.take(B * kModParts * D * 4));
  (void)kD;
  return p;
}

struct SingleBwdWs {
  float* dm; void* dy; void* dyT; void* catT; void* w2T; void* dcat; void* dlin1; void* dlin1T; void* hT; void* w1T;
  float* dh; AttnWs at; Parts pt;
  size_t bytes;
};

SingleBwdWs single_bwd_ws(const flux_dims* d, void* base) {
  Carve c(base);
  SingleBwdWs w{};
  const int64_t B = d->batch, L = (int64_t)d->l_img + d->l_txt, D = d->hidden, F = d->mlp_hidden, Lp = seq_pad_of(L);
  const int64_t T = B * L, Tp = tok_pad(T);
  w.dm = static_cast<float*>(c.take(B * 3 * D * 4));
  w.dy = c.take(T * D * 2);
  w.dyT = c.take(D * Tp * 2);
  w.catT = c.take((D + F) * Tp * 2);
  w.w2T = c.take((D + F) * D * 2);
  w.dcat = c.take(T * (D + F) * 2);
  w.dlin1 = c.take(T * (3 * D + F) * 2);
  w.dlin1T = c.take((3 * D + F) * Tp * 2);
  w.hT = c.take(D * Tp * 2);
  w.w1T = c.take(D * (3 * D + F) * 2);
  w.dh = static_cast<float*>(c.take(T * D * 4));
  w.at = attn_ws(c, B, d->heads, Lp);
  w.pt = parts_ws(c, d, 3 * D + F, 3 * D);
  w.bytes = (size_t)round_up((int64_t)c.off, 256);
  return w;
}

struct BlockBwdWs {
  float* dm[2];
  void* dy;      // [B, L, D] bf16 gated output gradient (fc2, then proj)
  void* du;      // [B, L, F] bf16 d(u), then d(pre-activation) in place
  void* dO;      // [B, L, D] bf16 attention output gradient
  void* dqkv;    // [B, L, 3D] bf16
  float* dh;     // [B, L, D] fp32 LN-modulate output gradient
  void* yT[2];   // [max(F, 3D), Tp_s] bf16 transposed output gradient per stream
  void* xT[2];   // [max(F, D), Tp_s] bf16 transposed linear input per stream
  void* wT[2];   // [max(F, 3D) * D] bf16 transposed weight per stream
  AttnWs at; Parts pt;
  size_t bytes;
};

BlockBwdWs block_bwd_ws(const flux_dims* d, void* base) {
  Carve c(base);
  BlockBwdWs w{};
  const int64_t B = d->batch, L = (int64_t)d->l_img + d->l_txt, D = d->hidden, F = d->mlp_hidden, Lp = seq_pad_of(L);
  const int64_t seg[2] = {d->l_img, d->l_txt};
  const int64_t ry = F > 3 * D ? F : 3 * D, rx = F > D ? F : D;
  w.dm[0] = static_cast<float*>(c.take(B * 6 * D * 4));
  w.dm[1] = static_cast<float*>(c.take(B * 6 * D * 4));
  w.dy = c.take(B * L * D * 2);
  w.du = c.take(B * L * F * 2);
  w.dO = c.take(B * L * D * 2);
  w.dqkv = c.take(B * L * 3 * D * 2);
  w.dh = static_cast<float*>(c.take(B * L * D * 4));
  for (int i = 0; i < 2; ++i) {
    const int64_t Tp = tok_pad(B * seg[i]);
    w.yT[i] = c.take(ry * Tp * 2);
    w.xT[i] = c.take(rx * Tp * 2);
    w.wT[i] = c.take(ry * D * 2);
  }
  w.at = attn_ws(c, B, d->heads, Lp);
  w.pt = parts_ws(c, d, F > 3 * D ? F : 3 * D, 6 * D);
  w.bytes = (size_t)round_up((int64_t)c.off, 256);
  return w;
}

// ------------------------------- launch helpers -------------------------------
// transpose R rows (addressed by m from src) of C columns into dst [C, R_fill]
hipError_t transpose_rows(const void* src, int src_dt, RowMap m, int64_t R, int64_t C, void* dst, int64_t R_fill,
                          hipStream_t st) {
  TransposeArgs a{};
  a.src = src; a.src_zstride = 0; a.smap = m;
  a.dst = dst; a.dst_zstride = 0; a.dst_ld = R_fill;
  a.R = (int32_t)R; a.C = (int32_t)C; a.R_fill = (int32_t)R_fill; a.Z = 1;
  return launch_transpose(a, src_dt, st);
}

// head-major [Z, R, C] -> [Z, C, R] (bf16)
hipError_t transpose_heads(const void* src, void* dst, int64_t Z, int64_t R, int64_t C, hipStream_t st) {
  TransposeArgs a{};
  a.src = src; a.src_zstride = R * C; a.smap = rmap(R * C, C, R);
  a.dst = dst; a.dst_zstride = R * C; a.dst_ld = R;
  a.R = (int32_t)R; a.C = (int32_t)C; a.R_fill = (int32_t)R; a.Z = (int32_t)Z;
  return launch_transpose(a, kBF16, st);
}

// column sums of A (* Bm) over the rows of each sample (Z = samples, R rows each)
// or over all rows (Z = 1, R = all rows)
hipError_t colsum(const void* A, int a_dt, RowMap am, const float* Bm, RowMap bm, int64_t R, int64_t C, int64_t Z,
                  float* out, int64_t out_zstride, float* part, hipStream_t st) {
  ColsumArgs a{};
  a.A = A; a.amap = am; a.Bm = Bm; a.bmap = bm;
  a.R = (int32_t)R; a.C = (int32_t)C; a.Z = (int32_t)Z;
  a.nrb = (int32_t)(R < kColParts ? (R > 0 ? R : 1) : kColParts);
  a.rpb = (int32_t)ceil_div(R > 0 ? R : 1, a.nrb);
  a.part = part;
  return launch_colsum(a, a_dt, out, out_zstride, 0, st);
}

hipError_t elementwise(int op, const void* x, RowMap xm, const void* y, RowMap ym, void* out, RowMap om,
                       const float* gate, int64_t gate_bs, int64_t rows, int64_t C, hipStream_t st, int f16 = 0) {
  EwArgs a{};
  a.op = op; a.x = x; a.xmap = xm; a.y = y; a.ymap = ym; a.out = out; a.omap = om;
  a.gate = gate; a.gate_bstride = gate_bs; a.rows = rows; a.C = (int32_t)C; a.f16 = f16;
  return launch_elementwise(a, st);
}

hipError_t ln_bwd(const float* x, RowMap xm, const float* dh, RowMap dhm, float* dx, RowMap dxm, const float* scale,
                  int64_t mod_bs, float* dshift, float* dscale, int64_t seg, int64_t B, int64_t D, float eps,
                  const Parts& p, hipStream_t st) {
  LnBwdArgs a{};
  a.x = x; a.xmap = xm; a.dh = dh; a.dhmap = dhm; a.dx = dx; a.dxmap = dxm;
  a.scale = scale; a.mod_bstride = mod_bs; a.dshift = dshift; a.dscale = dscale;
  a.part_sh = p.ln_sh; a.part_sc = p.ln_sc;
  a.seg = (int32_t)seg; a.batch = (int32_t)B; a.eps = eps;
  return launch_ln_mod_bwd(a, (int)D, st);
}

hipError_t mod_bwd(const void* w, const float* vec, const float* dm, int64_t N, int64_t D, int64_t B, float* dw,
                   float* db, float* dvec, const Parts& p, hipStream_t st) {
  ModBwdArgs a{};
  a.w = w; a.vec = vec; a.dm = dm; a.dm_bstride = N;
  a.dw = dw; a.db = db; a.dvec = dvec;
  a.N = (int32_t)N; a.K = (int32_t)D; a.batch = (int32_t)B; a.nrc = kModParts;
  a.silu_in = 1;
  a.part = p.mod;
  return launch_mod_bwd(a, kBF16, st);
}

// attention backward from saved head-major operands; dO bf16 and O (bf16, or
// fp16 when o_f16) token rows
hipError_t attention_bwd(int64_t B, int64_t L, int64_t H, const void* qh, const void* kh, const void* vt,
                         const float* lse, const void* dO, int64_t do_bs, int64_t do_ld, const void* o, int64_t o_bs,
                         int64_t o_ld, bool o_f16, const AttnWs& w, hipStream_t st) {
  const int64_t Lp = seq_pad_of(L);
  hipError_t e = transpose_heads(qh, w.qt, B * H, Lp, 128, st);
  if (e == hipSuccess) e = transpose_heads(kh, w.kt, B * H, Lp, 128, st);
  if (e == hipSuccess) e = transpose_heads(vt, w.vh, B * H, 128, Lp, st);
  if (e != hipSuccess) return e;
  AttnBwdArgs a{};
  a.qh = qh; a.kh = kh; a.vh = w.vh; a.qt = w.qt; a.kt = w.kt; a.lse = lse;
  a.dout = dO; a.dout_bstride = do_bs; a.dout_ld = do_ld;
  a.o = o; a.o_bstride = o_bs; a.o_ld = o_ld; a.o_f16 = o_f16 ? 1 : 0;
  a.doh = w.doh; a.dot = w.dot; a.dd = w.dd;
  a.dq = w.dq; a.dk = w.dk; a.dv = w.dv;
  a.batch = (int32_t)B; a.seq = (int32_t)L; a.seq_pad = (int32_t)Lp; a.heads = (int32_t)H;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  a.scale = (float)(1.0 / sqrt(128.0));
  return launch_attention_bwd(a, st);
}

// dgamma of q / k per stream from prep_bwd's partials: slice (s, which) of 512
hipError_t gamma_grads(const float* part, int nblk, float* out[2][2], hipStream_t st) {
  for (int s = 0; s < 2; ++s)
    for (int w = 0; w < 2; ++w) {
      if (!out[s][w]) continue;
      ReduceArgs r{};
      r.part = part + s * 256 + w * 128; r.np = nblk; r.C = 128; r.Z = 1; r.pstride = 512;
      r.out = out[s][w]; r.out_zstride = 0; r.mode = 0;
      hipError_t e = launch_reduce(r, st);
      if (e != hipSuccess) return e;
    }
  return hipSuccess;
}

// y = A W^T (+ bias) stored as out_dt (kF32, kBF16 or kF16); A is bf16 for
// launch_gemm(.., kBF16) and fp16 for launch_gemm(.., kF16), W bf16 for both
GemmProblem lin_problem(const void* A, RowMap am, const void* W, const void* bias, int64_t M, int64_t N, int64_t K,
                        void* out, RowMap om, int out_dt) {
  GemmProblem p = gemm_problem(A, am, W, bias, (int)M, (int)N, (int)K, out_dt == kF32 ? kEpiStoreF32 : kEpiStore, out,
                               om);
  p.out0_dt = out_dt;
  return p;
}

GemmProblem bf16_problem(const void* A, RowMap am, const void* W, const void* bias, int64_t M, int64_t N, int64_t K,
                         void* out, RowMap om, bool out_f32) {
  return lin_problem(A, am, W, bias, M, N, K, out, om, out_f32 ? kF32 : kBF16);
}

// GELU elementwise masks: fp16 pre-activation in, fp16 activation out (forward);
// fp16 pre-activation beside the bf16 gradients (backward)
constexpr int kGeluF16 = 1 | 4, kGeluBwdF16 = 2;

flux_status check_single_weights(const flux_single_weights* sw) {
  REQUIRE(sw, "weights are NULL");
  REQUIRE(sw->mod_w && sw->mod_b && sw->lin1_w && sw->lin1_b && sw->q_norm && sw->k_norm && sw->lin2_w && sw->lin2_b,
          "single block weights: a pointer is NULL");
  const void* ps[] = {sw->mod_w, sw->mod_b, sw->lin1_w, sw->lin1_b, sw->q_norm, sw->k_norm, sw->lin2_w, sw->lin2_b};
  for (const void* p : ps) REQUIRE(aligned16(p), "single block weights: pointers must be 16-byte aligned");
  return FLUX_OK;
}

flux_status check_grad_ptrs(float* const* ps, int n, const char* what) {
  for (int i = 0; i < n; ++i) REQUIRE(ps[i] && aligned16(ps[i]), "%s: every gradient pointer must be non-NULL and 16-byte aligned", what);
  return FLUX_OK;
}

}  // namespace

extern "C" {

// the sequential single block is a one-stream double block over all L tokens
static flux_dims one_stream(const flux_dims* d) {
  flux_dims one = *d;
  one.l_img = d->l_img + d->l_txt;
  one.l_txt = 0;
  return one;
}

size_t flux_train_saved_bytes(const flux_dims* d, int32_t op) {
  if (check_train_dims(d) != FLUX_OK) return 0;
  if (op == 0) return block_saved(d, nullptr).bytes;
  if (op == 2) {
    const flux_dims one = one_stream(d);
    return block_saved(&one, nullptr).bytes;
  }
  if (op == 1) return single_saved(d, nullptr).bytes;
  return 0;
}

size_t flux_bwd_workspace_bytes(const flux_dims* d, int32_t op) {
  if (check_train_dims(d) != FLUX_OK) return 0;
  if (op == 0) return block_bwd_ws(d, nullptr).bytes;
  if (op == 2) {
    const flux_dims one = one_stream(d);
    return block_bwd_ws(&one, nullptr).bytes;
  }
  if (op == 1) return single_bwd_ws(d, nullptr).bytes;
  return 0;
}

// ------------------------------ single block ------------------------------
flux_status flux_single_fwd_train(const flux_dims* d, const flux_single_weights* sw, float* x, int64_t x_bstride,
                                  const float* vec, const float* rope, void* saved, size_t saved_bytes, void* stream) {
  g_err[0] = 0;
  flux_status s = check_train_dims(d);
  if (s != FLUX_OK) return s;
  if ((s = check_single_weights(sw)) != FLUX_OK) return s;
  const int64_t B = d->batch, L = (int64_t)d->l_img + d->l_txt, D = d->hidden, F = d->mlp_hidden, Lp = seq_pad_of(L);
  REQUIRE(x && aligned16(x) && x_bstride >= L * D && x_bstride % 4 == 0, "x must be 16-byte aligned, x_bstride >= L*hidden, a multiple of 4");
  REQUIRE(vec && aligned16(vec) && rope && aligned16(rope), "vec and rope must be non-NULL and 16-byte aligned");
  if ((s = check_workspace(saved, saved_bytes, single_saved(d, nullptr).bytes)) != FLUX_OK) return s;
  const SingleSaved sv = single_saved(d, saved);
  hipStream_t st = static_cast<hipStream_t>(stream);

  GemvBatch gv{};
  gv.count = 1;
  gv.p[0] = gemv_problem(sw->mod_w, sw->mod_b, (int)(3 * D), (int)D, vec, D, sv.mod, 3 * D, 1, 0);
  FLUX_HIP(run_gemv(gv, (int)B, kBF16, st), "modulation GEMV");
  FLUX_HIP(hipMemcpy2DAsync(sv.x0, L * D * 4, x, x_bstride * 4, L * D * 4, B, hipMemcpyDeviceToDevice, st),
           "residual snapshot");
  LnArgs la{};
  la.count = 1; la.dim = (int)D; la.eps = d->eps;
  la.s[0].x = x; la.s[0].xmap = rmap(x_bstride, D, L);
  la.s[0].out = sv.h; la.s[0].omap = rmap(L * D, D, L);
  la.s[0].shift = sv.mod; la.s[0].scale = sv.mod + D; la.s[0].mod_bstride = 3 * D;
  la.s[0].rows = (int32_t)(B * L);
  FLUX_HIP(launch_ln_mod(la, kF16, st), "LayerNorm-modulate");
  // linear1 as two problems of one launch: the q|k|v rows of W1 into bf16, the MLP rows into fp16
  GemmBatch g{};
  g.count = 2;
  g.p[0] = lin_problem(sv.h, rmap(L * D, D, L), sw->lin1_w, sw->lin1_b, B * L, 3 * D, D, sv.qkv, rmap(L * 3 * D, 3 * D, L),
                       kBF16);
  g.p[1] = lin_problem(sv.h, rmap(L * D, D, L), elem_ptr(sw->lin1_w, 3 * D * D, 2), elem_ptr(sw->lin1_b, 3 * D, 2), B * L,
                       F, D, sv.a, rmap(L * F, F, L), kF16);
  FLUX_HIP(launch_gemm(g, kF16, st), "linear1 GEMM");
  FLUX_HIP(elementwise(kEwGelu, sv.a, rmap(L * F, F, L), nullptr, rmap(0, 1, 1), elem_ptr(sv.cat, D, 2),
                       rmap(L * (D + F), D + F, L), nullptr, 0, B * L, F, st, kGeluF16),
           "GELU");
  PrepArgs pa{};
  pa.src_q = sv.qkv; pa.src_k = elem_ptr(sv.qkv, D, 2); pa.src_v = elem_ptr(sv.qkv, 2 * D, 2);
  pa.src_bstride = L * 3 * D; pa.src_ld = 3 * D;
  pa.batch = (int)B; pa.seq = (int)L; pa.seq_pad = (int)Lp; pa.heads = d->heads; pa.head_dim = 128;
  pa.l_img = (int)L;
  pa.gq_img = pa.gq_txt = sw->q_norm;
  pa.gk_img = pa.gk_txt = sw->k_norm;
  pa.rope = rope; pa.eps = d->eps;
  pa.qh = sv.qh; pa.kh = sv.kh; pa.vt = sv.vt;
  FLUX_HIP(launch_prep(pa, kBF16, st), "q/k norm + RoPE");
  AttnArgs aa{};
  aa.qh = sv.qh; aa.kh = sv.kh; aa.vt = sv.vt;
  aa.out = sv.cat; aa.out_bstride = L * (D + F); aa.out_ld = D + F;
  aa.batch = (int)B; aa.seq = (int)L; aa.seq_pad = (int)Lp; aa.heads = d->heads; aa.head_dim = 128;
  aa.scale_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  aa.l_img = (int)L;
  aa.lse = sv.lse;
  FLUX_HIP(launch_attention(aa, kBF16, kF16, st), "attention");
  g.count = 1;
  g.p[0] = lin_problem(sv.cat, rmap(L * (D + F), D + F, L), sw->lin2_w, sw->lin2_b, B * L, D, D + F, sv.y,
                       rmap(L * D, D, L), kF32);
  FLUX_HIP(launch_gemm(g, kF16, st), "linear2 GEMM");
  FLUX_HIP(elementwise(kEwGateAdd, sv.y, rmap(L * D, D, L), nullptr, rmap(0, 1, 1), x, rmap(x_bstride, D, L),
                       sv.mod + 2 * D, 3 * D, B * L, D, st),
           "gated residual");
  if (debug_checks_on())
    FLUX_HIP(debug_check(x, kF32, B, L * D, x_bstride, -kDbgBig, kDbgBig, FLUX_DBG_NONFINITE_RESIDUAL, st),
             "debug check of the residual");
  return FLUX_OK;
}

flux_status flux_single_bwd(const flux_dims* d, const flux_single_weights* sw, float* dx, int64_t dx_bstride,
                            const float* vec, const float* rope, const void* saved, size_t saved_bytes,
                            const flux_single_grads* gr, float* dvec, void* workspace, size_t workspace_bytes,
                            void* stream) {
  g_err[0] = 0;
  flux_status s = check_train_dims(d);
  if (s != FLUX_OK) return s;
  if ((s = check_single_weights(sw)) != FLUX_OK) return s;
  const int64_t B = d->batch, L = (int64_t)d->l_img + d->l_txt, D = d->hidden, F = d->mlp_hidden, Lp = seq_pad_of(L);
  const int64_t T = B * L, Tp = tok_pad(T);
  REQUIRE(dx && aligned16(dx) && dx_bstride >= L * D && dx_bstride % 4 == 0,
          "dx must be 16-byte aligned, dx_bstride >= L*hidden, a multiple of 4");
  REQUIRE(vec && aligned16(vec) && rope && aligned16(rope) && dvec && aligned16(dvec),
          "vec, rope and dvec must be non-NULL and 16-byte aligned");
  REQUIRE(gr, "grads are NULL");
  float* const gp[] = {gr->mod_w, gr->mod_b, gr->lin1_w, gr->lin1_b, gr->q_norm, gr->k_norm, gr->lin2_w, gr->lin2_b};
  if ((s = check_grad_ptrs(gp, 8, "single block grads")) != FLUX_OK) return s;
  if ((s = check_workspace(const_cast<void*>(saved), saved_bytes, single_saved(d, nullptr).bytes)) != FLUX_OK) return s;
  if ((s = check_workspace(workspace, workspace_bytes, single_bwd_ws(d, nullptr).bytes)) != FLUX_OK) return s;
  const SingleSaved sv = single_saved(d, const_cast<void*>(saved));
  const SingleBwdWs w = single_bwd_ws(d, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const RowMap dxm = rmap(dx_bstride, D, L), rowsD = rmap(L * D, D, L);
  const RowMap rowsCat = rmap(L * (D + F), D + F, L), rowsLin1 = rmap(L * (3 * D + F), 3 * D + F, L);
  const RowMap none = rmap(0, 1, 1);

  // x_out = x + gate * y: dgate = sum_t y dx_out, dy = gate * dx_out
  FLUX_HIP(colsum(dx, kF32, dxm, sv.y, rowsD, L, D, B, w.dm + 2 * D, 3 * D, w.pt.col, st), "gate gradient");
  FLUX_HIP(elementwise(kEwGateBwd, dx, dxm, nullptr, none, w.dy, rowsD, sv.mod + 2 * D, 3 * D, T, D, st), "dy");
  FLUX_HIP(colsum(w.dy, kBF16, rowsD, nullptr, none, T, D, 1, gr->lin2_b, 0, w.pt.col, st), "linear2 bias gradient");
  // linear2: d[O | u] = dy W2, dW2 = dy^T [O | u]
  FLUX_HIP(transpose_rows(sw->lin2_w, kBF16, rmap(D * (D + F), D + F, D), D, D + F, w.w2T, D, st), "W2^T");
  FLUX_HIP(transpose_rows(w.dy, kBF16, rowsD, T, D, w.dyT, Tp, st), "dy^T");
  FLUX_HIP(transpose_rows(sv.cat, kF16, rowsCat, T, D + F, w.catT, Tp, st), "[O|u]^T");
  GemmBatch g{};
  g.count = 1;
  g.p[0] = bf16_problem(w.dy, rowsD, w.w2T, nullptr, T, D + F, D, w.dcat, rmap(T * (D + F), D + F, T), false);
  FLUX_HIP(launch_gemm(g, kBF16, st), "linear2 data gradient");
  g.p[0] = bf16_problem(w.dyT, rmap(D * Tp, Tp, D), w.catT, nullptr, D, D + F, Tp, gr->lin2_w,
                        rmap(D * (D + F), D + F, D), true);
  FLUX_HIP(launch_gemm(g, kBF16, st), "linear2 weight gradient");
  // u = GELU(a): da = du GELU'(a) -> columns 3D.. of d(linear1 output)
  FLUX_HIP(elementwise(kEwGeluBwd, elem_ptr(w.dcat, D, 2), rmap(T * (D + F), D + F, T), sv.a, rmap(L * F, F, L),
                       elem_ptr(w.dlin1, 3 * D, 2), rmap(T * (3 * D + F), 3 * D + F, T), nullptr, 0, T, F, st,
                       kGeluBwdF16),
           "GELU backward");
  // attention, then q / k RMSNorm + RoPE backward -> columns 0..3D
  FLUX_HIP(attention_bwd(B, L, d->heads, sv.qh, sv.kh, sv.vt, sv.lse, w.dcat, L * (D + F), D + F, sv.cat, L * (D + F),
                         D + F, true, w.at, st),
           "attention backward");
  PrepBwdArgs pb{};
  pb.dq = w.at.dq; pb.dk = w.at.dk; pb.dv = w.at.dv;
  pb.src = sv.qkv; pb.src_bstride = L * 3 * D; pb.src_ld = 3 * D;
  pb.dst = w.dlin1; pb.dst_bstride = L * (3 * D + F); pb.dst_ld = 3 * D + F;
  pb.gq_img = pb.gq_txt = sw->q_norm;
  pb.gk_img = pb.gk_txt = sw->k_norm;
  pb.rope = rope;
  pb.batch = (int)B; pb.seq = (int)L; pb.seq_pad = (int)Lp; pb.heads = d->heads; pb.l_img = (int)L;
  pb.eps = d->eps; pb.part = w.pt.prep;
  FLUX_HIP(launch_prep_bwd(pb, st), "q/k norm + RoPE backward");
  float* gg[2][2] = {{gr->q_norm, gr->k_norm}, {nullptr, nullptr}};
  FLUX_HIP(gamma_grads(w.pt.prep, prep_bwd_parts((int)B, (int)L, d->heads), gg, st), "norm scale gradients");
  // linear1: dh = d(lin1) W1, dW1 = d(lin1)^T h
  FLUX_HIP(colsum(w.dlin1, kBF16, rowsLin1, nullptr, none, T, 3 * D + F, 1, gr->lin1_b, 0, w.pt.col, st),
           "linear1 bias gradient");
  FLUX_HIP(transpose_rows(sw->lin1_w, kBF16, rmap((3 * D + F) * D, D, 3 * D + F), 3 * D + F, D, w.w1T, 3 * D + F, st),
           "W1^T");
  FLUX_HIP(transpose_rows(w.dlin1, kBF16, rowsLin1, T, 3 * D + F, w.dlin1T, Tp, st), "d(lin1)^T");
  FLUX_HIP(transpose_rows(sv.h, kF16, rowsD, T, D, w.hT, Tp, st), "h^T");
  g.p[0] = bf16_problem(w.dlin1, rowsLin1, w.w1T, nullptr, T, D, 3 * D + F, w.dh, rmap(T * D, D, T), true);
  FLUX_HIP(launch_gemm(g, kBF16, st), "linear1 data gradient");
  g.p[0] = bf16_problem(w.dlin1T, rmap((3 * D + F) * Tp, Tp, 3 * D + F), w.hT, nullptr, 3 * D + F, D, Tp, gr->lin1_w,
                        rmap((3 * D + F) * D, D, 3 * D + F), true);
  FLUX_HIP(launch_gemm(g, kBF16, st), "linear1 weight gradient");
  // LayerNorm-modulate: dx += ..., dshift, dscale
  FLUX_HIP(ln_bwd(sv.x0, rowsD, w.dh, rowsD, dx, dxm, sv.mod + D, 3 * D, w.dm, w.dm + D, L, B, D, d->eps, w.pt, st),
           "LayerNorm-modulate backward");
  // modulation: dW, db, dvec += SiLU'(vec) W^T dm
  FLUX_HIP(mod_bwd(sw->mod_w, vec, w.dm, 3 * D, D, B, gr->mod_w, gr->mod_b, dvec, w.pt, st), "modulation backward");
  if (debug_checks_on())
    FLUX_HIP(debug_check(dx, kF32, B, L * D, dx_bstride, -kDbgBig, kDbgBig, FLUX_DBG_NONFINITE_GRAD, st),
             "debug check of the input gradient");
  return FLUX_OK;
}

// ------------------------------ double block ------------------------------
flux_status flux_block_fwd_train(const flux_dims* d, const flux_stream_weights* iw, const flux_stream_weights* tw,
                                 float* img, int64_t img_bstride, float* txt, int64_t txt_bstride, const float* vec,
                                 const float* rope, void* saved, size_t saved_bytes, void* stream) {
  g_err[0] = 0;
  flux_status s = check_train_dims(d);
  if (s != FLUX_OK) return s;
  const int64_t B = d->batch, Li = d->l_img, Lt = d->l_txt, L = Li + Lt, D = d->hidden, F = d->mlp_hidden;
  const int64_t Lp = seq_pad_of(L);
  if ((s = check_stream_weights(iw, "image")) != FLUX_OK) return s;
  if (Lt > 0 && (s = check_stream_weights(tw, "text")) != FLUX_OK) return s;
  REQUIRE(img && aligned16(img) && img_bstride >= Li * D && img_bstride % 4 == 0, "img: 16-byte aligned, img_bstride >= l_img*hidden, a multiple of 4");
  if (Lt > 0) REQUIRE(txt && aligned16(txt) && txt_bstride >= Lt * D && txt_bstride % 4 == 0, "txt: 16-byte aligned, txt_bstride >= l_txt*hidden, a multiple of 4");
  REQUIRE(vec && aligned16(vec) && rope && aligned16(rope), "vec and rope must be non-NULL and 16-byte aligned");
  if ((s = check_workspace(saved, saved_bytes, block_saved(d, nullptr).bytes)) != FLUX_OK) return s;
  const BlockSaved sv = block_saved(d, saved);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int ns = Lt > 0 ? 2 : 1;
  const flux_stream_weights* sw[2] = {iw, tw};
  float* xs[2] = {img, txt};
  const int64_t xbs[2] = {img_bstride, txt_bstride}, seg[2] = {Li, Lt}, off[2] = {0, Li};
  auto jrow = [&](int i, int64_t C) { return rmap(L * C, C, seg[i]); };   // stream rows of a joint [B, L, C]

  GemvBatch gv{};
  gv.count = ns;
  for (int i = 0; i < ns; ++i)
    gv.p[i] = gemv_problem(sw[i]->mod_w, sw[i]->mod_b, (int)(6 * D), (int)D, vec, D, sv.mod[i], 6 * D, 1, 0);
  FLUX_HIP(run_gemv(gv, (int)B, kBF16, st), "modulation GEMV");
  auto snapshot = [&](float* dst) -> hipError_t {
    for (int i = 0; i < ns; ++i) {
      hipError_t e = hipMemcpy2DAsync(dst + off[i] * D, L * D * 4, xs[i], xbs[i] * 4, seg[i] * D * 4, B,
                                      hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  };
  auto ln_mod = [&](int chunk, void* out) -> hipError_t {
    LnArgs a{};
    a.count = ns; a.dim = (int)D; a.eps = d->eps;
    for (int i = 0; i < ns; ++i) {
      a.s[i].x = xs[i]; a.s[i].xmap = rmap(xbs[i], D, seg[i]);
      a.s[i].out = elem_ptr(out, off[i] * D, 2); a.s[i].omap = jrow(i, D);
      a.s[i].shift = sv.mod[i] + chunk * D; a.s[i].scale = sv.mod[i] + (chunk + 1) * D; a.s[i].mod_bstride = 6 * D;
      a.s[i].rows = (int32_t)(B * seg[i]);
    }
    return launch_ln_mod(a, kF16, st);
  };
  FLUX_HIP(snapshot(sv.x0), "residual snapshot");
  FLUX_HIP(ln_mod(0, sv.h1), "LayerNorm-modulate (attention)");
  GemmBatch g{};
  g.count = ns;
  for (int i = 0; i < ns; ++i)
    g.p[i] = lin_problem(elem_ptr(sv.h1, off[i] * D, 2), jrow(i, D), sw[i]->qkv_w, sw[i]->qkv_b, B * seg[i], 3 * D, D,
                         elem_ptr(sv.qkv, off[i] * 3 * D, 2), jrow(i, 3 * D), kBF16);
  FLUX_HIP(launch_gemm(g, kF16, st), "qkv GEMM");
  PrepArgs pa{};
  pa.src_q = sv.qkv; pa.src_k = elem_ptr(sv.qkv, D, 2); pa.src_v = elem_ptr(sv.qkv, 2 * D, 2);
  pa.src_bstride = L * 3 * D; pa.src_ld = 3 * D;
  pa.batch = (int)B; pa.seq = (int)L; pa.seq_pad = (int)Lp; pa.heads = d->heads; pa.head_dim = 128;
  pa.l_img = (int)Li;
  pa.gq_img = iw->q_norm; pa.gk_img = iw->k_norm;
  pa.gq_txt = Lt > 0 ? tw->q_norm : iw->q_norm;
  pa.gk_txt = Lt > 0 ? tw->k_norm : iw->k_norm;
  pa.rope = rope; pa.eps = d->eps;
  pa.qh = sv.qh; pa.kh = sv.kh; pa.vt = sv.vt;
  FLUX_HIP(launch_prep(pa, kBF16, st), "q/k norm + RoPE");
  AttnArgs aa{};
  aa.qh = sv.qh; aa.kh = sv.kh; aa.vt = sv.vt;
  aa.out = sv.o; aa.out_bstride = L * D; aa.out_ld = D;
  aa.batch = (int)B; aa.seq = (int)L; aa.seq_pad = (int)Lp; aa.heads = d->heads; aa.head_dim = 128;
  aa.scale_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  aa.l_img = (int)Li;
  aa.lse = sv.lse;
  FLUX_HIP(launch_attention(aa, kBF16, kF16, st), "joint attention");
  for (int i = 0; i < ns; ++i)
    g.p[i] = lin_problem(elem_ptr(sv.o, off[i] * D, 2), jrow(i, D), sw[i]->proj_w, sw[i]->proj_b, B * seg[i], D, D,
                         sv.y1 + off[i] * D, jrow(i, D), kF32);
  FLUX_HIP(launch_gemm(g, kF16, st), "output projection GEMM");
  for (int i = 0; i < ns; ++i)
    FLUX_HIP(elementwise(kEwGateAdd, sv.y1 + off[i] * D, jrow(i, D), nullptr, rmap(0, 1, 1), xs[i],
                         rmap(xbs[i], D, seg[i]), sv.mod[i] + 2 * D, 6 * D, B * seg[i], D, st),
             "gated residual (attention)");
  FLUX_HIP(snapshot(sv.x1), "residual snapshot");
  FLUX_HIP(ln_mod(3, sv.h2), "LayerNorm-modulate (MLP)");
  for (int i = 0; i < ns; ++i)
    g.p[i] = lin_problem(elem_ptr(sv.h2, off[i] * D, 2), jrow(i, D), sw[i]->fc1_w, sw[i]->fc1_b, B * seg[i], F, D,
                         elem_ptr(sv.a1, off[i] * F, 2), jrow(i, F), kF16);
  FLUX_HIP(launch_gemm(g, kF16, st), "fc1 GEMM");
  FLUX_HIP(elementwise(kEwGelu, sv.a1, rmap(L * F, F, L), nullptr, rmap(0, 1, 1), sv.u, rmap(L * F, F, L), nullptr, 0,
                       B * L, F, st, kGeluF16),
           "GELU");
  for (int i = 0; i < ns; ++i)
    g.p[i] = lin_problem(elem_ptr(sv.u, off[i] * F, 2), jrow(i, F), sw[i]->fc2_w, sw[i]->fc2_b, B * seg[i], D, F,
                         sv.y2 + off[i] * D, jrow(i, D), kF32);
  FLUX_HIP(launch_gemm(g, kF16, st), "fc2 GEMM");
  for (int i = 0; i < ns; ++i)
    FLUX_HIP(elementwise(kEwGateAdd, sv.y2 + off[i] * D, jrow(i, D), nullptr, rmap(0, 1, 1), xs[i],
                         rmap(xbs[i], D, seg[i]), sv.mod[i] + 5 * D, 6 * D, B * seg[i], D, st),
             "gated residual (MLP)");
  if (debug_checks_on())
    for (int i = 0; i < ns; ++i)
      FLUX_HIP(debug_check(xs[i], kF32, B, seg[i] * D, xbs[i], -kDbgBig, kDbgBig, FLUX_DBG_NONFINITE_RESIDUAL, st),
               "debug check of the residual");
  return FLUX_OK;
}

flux_status flux_block_bwd(const flux_dims* d, const flux_stream_weights* iw, const flux_stream_weights* tw,
                           float* d_img, int64_t img_bstride, float* d_txt, int64_t txt_bstride, const float* vec,
                           const float* rope, const void* saved, size_t saved_bytes, const flux_stream_grads* gi,
                           const flux_stream_grads* gt, float* dvec, void* workspace, size_t workspace_bytes,
                           void* stream) {
  g_err[0] = 0;
  flux_status s = check_train_dims(d);
  if (s != FLUX_OK) return s;
  const int64_t B = d->batch, Li = d->l_img, Lt = d->l_txt, L = Li + Lt, D = d->hidden, F = d->mlp_hidden;
  if ((s = check_stream_weights(iw, "image")) != FLUX_OK) return s;
  if (Lt > 0 && (s = check_stream_weights(tw, "text")) != FLUX_OK) return s;
  REQUIRE(d_img && aligned16(d_img) && img_bstride >= Li * D && img_bstride % 4 == 0, "d_img: 16-byte aligned, img_bstride >= l_img*hidden, a multiple of 4");
  if (Lt > 0) REQUIRE(d_txt && aligned16(d_txt) && txt_bstride >= Lt * D && txt_bstride % 4 == 0, "d_txt: 16-byte aligned, txt_bstride >= l_txt*hidden, a multiple of 4");
  REQUIRE(vec && aligned16(vec) && rope && aligned16(rope) && dvec && aligned16(dvec),
          "vec, rope and dvec must be non-NULL and 16-byte aligned");
  const flux_stream_grads* gs[2] = {gi, Lt > 0 ? gt : nullptr};
  const int ns = Lt > 0 ? 2 : 1;
  for (int i = 0; i < ns; ++i) {
    REQUIRE(gs[i], "%s grads are NULL", i ? "text" : "image");
    float* const gp[] = {gs[i]->mod_w, gs[i]->mod_b, gs[i]->qkv_w, gs[i]->qkv_b, gs[i]->q_norm, gs[i]->k_norm,
                         gs[i]->proj_w, gs[i]->proj_b, gs[i]->fc1_w, gs[i]->fc1_b, gs[i]->fc2_w, gs[i]->fc2_b};
    if ((s = check_grad_ptrs(gp, 12, i ? "text grads" : "image grads")) != FLUX_OK) return s;
  }
  if ((s = check_workspace(const_cast<void*>(saved), saved_bytes, block_saved(d, nullptr).bytes)) != FLUX_OK) return s;
  if ((s = check_workspace(workspace, workspace_bytes, block_bwd_ws(d, nullptr).bytes)) != FLUX_OK) return s;
  const BlockSaved sv = block_saved(d, const_cast<void*>(saved));
  const BlockBwdWs w = block_bwd_ws(d, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const flux_stream_weights* sw[2] = {iw, tw};
  float* ds[2] = {d_img, d_txt};
  const int64_t dbs[2] = {img_bstride, txt_bstride}, seg[2] = {Li, Lt}, off[2] = {0, Li};
  int64_t Tp[2];
  for (int i = 0; i < 2; ++i) Tp[i] = tok_pad(B * seg[i]);
  const RowMap none = rmap(0, 1, 1);
  auto jrow = [&](int i, int64_t C) { return rmap(L * C, C, seg[i]); };
  auto drow = [&](int i) { return rmap(dbs[i], D, seg[i]); };
  GemmBatch g{};
  g.count = ns;
  // one linear of both streams: y = x W^T + b with output gradient dyv (bf16 joint rows, width N) and
  // input x (the forward's fp16 joint rows, width K); writes dx (joint rows, width K; fp32 or bf16), dW and db
  auto linear_bwd = [&](const void* dyv, int64_t N, const void* x, int64_t K, const void* const* W, int wsel,
                        void* dxv, bool dx_f32) -> flux_status {
    for (int i = 0; i < ns; ++i) {
      float* gb = wsel == 0 ? gs[i]->qkv_b : wsel == 1 ? gs[i]->proj_b : wsel == 2 ? gs[i]->fc1_b : gs[i]->fc2_b;
      const void* dyi = elem_ptr(dyv, off[i] * N, 2);
      FLUX_HIP(colsum(dyi, kBF16, jrow(i, N), nullptr, none, B * seg[i], N, 1, gb, 0, w.pt.col, st), "bias gradient");
      FLUX_HIP(transpose_rows(W[i], kBF16, rmap(N * K, K, N), N, K, w.wT[i], N, st), "W^T");
      FLUX_HIP(transpose_rows(dyi, kBF16, jrow(i, N), B * seg[i], N, w.yT[i], Tp[i], st), "dy^T");
      FLUX_HIP(transpose_rows(elem_ptr(x, off[i] * K, 2), kF16, jrow(i, K), B * seg[i], K, w.xT[i], Tp[i], st), "x^T");
      g.p[i] = bf16_problem(dyi, jrow(i, N), w.wT[i], nullptr, B * seg[i], K, N,
                            elem_ptr(dxv, off[i] * K, dx_f32 ? 4 : 2), jrow(i, K), dx_f32);
    }
    FLUX_HIP(launch_gemm(g, kBF16, st), "data gradient GEMM");
    for (int i = 0; i < ns; ++i)
      g.p[i] = bf16_problem(w.yT[i], rmap(N * Tp[i], Tp[i], N), w.xT[i], nullptr, N, K, Tp[i],
                            wsel == 0 ? gs[i]->qkv_w : wsel == 1 ? gs[i]->proj_w : wsel == 2 ? gs[i]->fc1_w : gs[i]->fc2_w,
                            rmap(N * K, K, N), true);
    FLUX_HIP(launch_gemm(g, kBF16, st), "weight gradient GEMM");
    return FLUX_OK;
  };
  const void* Wfc2[2] = {iw->fc2_w, Lt > 0 ? tw->fc2_w : nullptr};
  const void* Wfc1[2] = {iw->fc1_w, Lt > 0 ? tw->fc1_w : nullptr};
  const void* Wproj[2] = {iw->proj_w, Lt > 0 ? tw->proj_w : nullptr};
  const void* Wqkv[2] = {iw->qkv_w, Lt > 0 ? tw->qkv_w : nullptr};

  // MLP half: x_out = x1 + g5 * fc2(GELU(fc1(LN(x1)(1 + s4) + sh3)))
  for (int i = 0; i < ns; ++i) {
    FLUX_HIP(colsum(ds[i], kF32, drow(i), sv.y2 + off[i] * D, jrow(i, D), seg[i], D, B, w.dm[i] + 5 * D, 6 * D,
                    w.pt.col, st), "gate2 gradient");
    FLUX_HIP(elementwise(kEwGateBwd, ds[i], drow(i), nullptr, none, elem_ptr(w.dy, off[i] * D, 2), jrow(i, D),
                         sv.mod[i] + 5 * D, 6 * D, B * seg[i], D, st), "dy (MLP)");
  }
  if ((s = linear_bwd(w.dy, D, sv.u, F, Wfc2, 3, w.du, false)) != FLUX_OK) return s;
  FLUX_HIP(elementwise(kEwGeluBwd, w.du, rmap(L * F, F, L), sv.a1, rmap(L * F, F, L), w.du, rmap(L * F, F, L), nullptr,
                       0, B * L, F, st, kGeluBwdF16), "GELU backward");
  if ((s = linear_bwd(w.du, F, sv.h2, D, Wfc1, 2, w.dh, true)) != FLUX_OK) return s;
  for (int i = 0; i < ns; ++i)
    FLUX_HIP(ln_bwd(sv.x1 + off[i] * D, jrow(i, D), w.dh + off[i] * D, jrow(i, D), ds[i], drow(i), sv.mod[i] + 4 * D,
                    6 * D, w.dm[i] + 3 * D, w.dm[i] + 4 * D, seg[i], B, D, d->eps, w.pt, st),
             "LayerNorm-modulate backward (MLP)");
  // attention half: x1 = x0 + g2 * proj(O)
  for (int i = 0; i < ns; ++i) {
    FLUX_HIP(colsum(ds[i], kF32, drow(i), sv.y1 + off[i] * D, jrow(i, D), seg[i], D, B, w.dm[i] + 2 * D, 6 * D,
                    w.pt.col, st), "gate1 gradient");
    FLUX_HIP(elementwise(kEwGateBwd, ds[i], drow(i), nullptr, none, elem_ptr(w.dy, off[i] * D, 2), jrow(i, D),
                         sv.mod[i] + 2 * D, 6 * D, B * seg[i], D, st), "dy (attention)");
  }
  if ((s = linear_bwd(w.dy, D, sv.o, D, Wproj, 1, w.dO, false)) != FLUX_OK) return s;
  FLUX_HIP(attention_bwd(B, L, d->heads, sv.qh, sv.kh, sv.vt, sv.lse, w.dO, L * D, D, sv.o, L * D, D, true, w.at, st),
           "attention backward");
  PrepBwdArgs pb{};
  pb.dq = w.at.dq; pb.dk = w.at.dk; pb.dv = w.at.dv;
  pb.src = sv.qkv; pb.src_bstride = L * 3 * D; pb.src_ld = 3 * D;
  pb.dst = w.dqkv; pb.dst_bstride = L * 3 * D; pb.dst_ld = 3 * D;
  pb.gq_img = iw->q_norm; pb.gk_img = iw->k_norm;
  pb.gq_txt = Lt > 0 ? tw->q_norm : iw->q_norm;
  pb.gk_txt = Lt > 0 ? tw->k_norm : iw->k_norm;
  pb.rope = rope;
  pb.batch = (int)B; pb.seq = (int)L; pb.seq_pad = (int)seq_pad_of(L); pb.heads = d->heads; pb.l_img = (int)Li;
  pb.eps = d->eps; pb.part = w.pt.prep;
  FLUX_HIP(launch_prep_bwd(pb, st), "q/k norm + RoPE backward");
  float* gg[2][2] = {{gi->q_norm, gi->k_norm}, {Lt > 0 ? gt->q_norm : nullptr, Lt > 0 ? gt->k_norm : nullptr}};
  FLUX_HIP(gamma_grads(w.pt.prep, prep_bwd_parts((int)B, (int)L, d->heads), gg, st), "norm scale gradients");
  if ((s = linear_bwd(w.dqkv, 3 * D, sv.h1, D, Wqkv, 0, w.dh, true)) != FLUX_OK) return s;
  for (int i = 0; i < ns; ++i) {
    FLUX_HIP(ln_bwd(sv.x0 + off[i] * D, jrow(i, D), w.dh + off[i] * D, jrow(i, D), ds[i], drow(i), sv.mod[i] + D,
                    6 * D, w.dm[i], w.dm[i] + D, seg[i], B, D, d->eps, w.pt, st),
             "LayerNorm-modulate backward (attention)");
    FLUX_HIP(mod_bwd(sw[i]->mod_w, vec, w.dm[i], 6 * D, D, B, gs[i]->mod_w, gs[i]->mod_b, dvec, w.pt, st),
             "modulation backward");
  }
  if (debug_checks_on())
    for (int i = 0; i < ns; ++i)
      FLUX_HIP(debug_check(ds[i], kF32, B, seg[i] * D, dbs[i], -kDbgBig, kDbgBig, FLUX_DBG_NONFINITE_GRAD, st),
               "debug check of the input gradient");
  return FLUX_OK;
}

// ------------------------ sequential single block ------------------------
flux_status flux_single_seq_fwd_train(const flux_dims* d, const flux_stream_weights* w, float* x, int64_t x_bstride,
                                      const float* vec, const float* rope, void* saved, size_t saved_bytes,
                                      void* stream) {
  g_err[0] = 0;
  REQUIRE(d, "dims is NULL");
  const flux_dims one = one_stream(d);
  return flux_block_fwd_train(&one, w, nullptr, x, x_bstride, nullptr, 0, vec, rope, saved, saved_bytes, stream);
}

flux_status flux_single_seq_bwd(const flux_dims* d, const flux_stream_weights* w, float* dx, int64_t x_bstride,
                                const float* vec, const float* rope, const void* saved, size_t saved_bytes,
                                const flux_stream_grads* grads, float* dvec, void* workspace, size_t workspace_bytes,
                                void* stream) {
  g_err[0] = 0;
  REQUIRE(d, "dims is NULL");
  const flux_dims one = one_stream(d);
  return flux_block_bwd(&one, w, nullptr, dx, x_bstride, nullptr, 0, vec, rope, saved, saved_bytes, grads, nullptr,
                        dvec, workspace, workspace_bytes, stream);
}

// ------------------------- attention alone (bf16) -------------------------
size_t flux_attention_train_workspace_bytes(int32_t batch, int32_t seq, int32_t heads) {
  if (batch < 1 || seq < 1 || heads < 1) return 0;
  Carve c(nullptr);
  const int64_t Lp = seq_pad_of(seq), n = (int64_t)batch * heads * Lp * 128;
  c.take(n * 2); c.take(n * 2); c.take(n * 2);   // qh, kh, vt
  attn_ws(c, batch, heads, Lp);
  c.take((int64_t)prep_bwd_parts(batch, seq, heads) * 512 * 4);
  return (size_t)round_up((int64_t)c.off, 256);
}

flux_status flux_attention_fwd_train(int32_t batch, int32_t seq, int32_t heads, const void* q, const void* k,
                                     const void* v, int64_t ld, void* o, int64_t ldo, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  REQUIRE(batch >= 1 && seq >= 1 && heads >= 1, "batch, seq and heads must be >= 1");
  if (seq_pad_of(seq) * 128 * 2 >= (int64_t)1 << 31)
    return fail(FLUX_ERR_UNSUPPORTED, "seq %d too long (one head's keys must stay under 2 GiB)", seq);
  REQUIRE(q && k && v && o && lse && aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o) && aligned16(lse),
          "q, k, v, o and lse must be non-NULL and 16-byte aligned");
  REQUIRE(ld >= heads * 128 && ld % 8 == 0 && ldo >= heads * 128 && ldo % 8 == 0, "ld, ldo >= heads*128, multiples of 8");
  flux_status s = check_workspace(workspace, workspace_bytes, flux_attention_train_workspace_bytes(batch, seq, heads));
  if (s != FLUX_OK) return s;
  const int64_t Lp = seq_pad_of(seq), n = (int64_t)batch * heads * Lp * 128;
  Carve c(workspace);
  void* qh = c.take(n * 2); void* kh = c.take(n * 2); void* vt = c.take(n * 2);
  hipStream_t st = static_cast<hipStream_t>(stream);
  PrepArgs pa{};
  pa.src_q = q; pa.src_k = k; pa.src_v = v; pa.src_bstride = seq * ld; pa.src_ld = ld;
  pa.batch = batch; pa.seq = seq; pa.seq_pad = (int)Lp; pa.heads = heads; pa.head_dim = 128; pa.l_img = seq;
  pa.qh = qh; pa.kh = kh; pa.vt = vt;
  FLUX_HIP(launch_prep(pa, kBF16, st), "head-major layout");
  AttnArgs aa{};
  aa.qh = qh; aa.kh = kh; aa.vt = vt;
  aa.out = o; aa.out_bstride = seq * ldo; aa.out_ld = ldo;
  aa.batch = batch; aa.seq = seq; aa.seq_pad = (int)Lp; aa.heads = heads; aa.head_dim = 128;
  aa.scale_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  aa.l_img = seq;
  aa.lse = lse;
  FLUX_HIP(launch_attention(aa, kBF16, kBF16, st), "attention");
  return FLUX_OK;
}

flux_status flux_attention_bwd(int32_t batch, int32_t seq, int32_t heads, const void* q, const void* k, const void* v,
                               int64_t ld, const void* o, const void* dout, int64_t ldo, const float* lse, void* dqkv,
                               void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  REQUIRE(batch >= 1 && seq >= 1 && heads >= 1, "batch, seq and heads must be >= 1");
  REQUIRE(q && k && v && o && dout && lse && dqkv, "every pointer is required");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o) && aligned16(dout) && aligned16(lse) &&
              aligned16(dqkv), "pointers must be 16-byte aligned");
  REQUIRE(ld >= heads * 128 && ld % 8 == 0 && ldo >= heads * 128 && ldo % 8 == 0, "ld, ldo >= heads*128, multiples of 8");
  flux_status s = check_workspace(workspace, workspace_bytes, flux_attention_train_workspace_bytes(batch, seq, heads));
  if (s != FLUX_OK) return s;
  const int64_t Lp = seq_pad_of(seq), n = (int64_t)batch * heads * Lp * 128, D = (int64_t)heads * 128;
  Carve c(workspace);
  void* qh = c.take(n * 2); void* kh = c.take(n * 2); void* vt = c.take(n * 2);
  const AttnWs w = attn_ws(c, batch, heads, Lp);
  float* part = static_cast<float*>(c.take((int64_t)prep_bwd_parts(batch, seq, heads) * 512 * 4));
  hipStream_t st = static_cast<hipStream_t>(stream);
  PrepArgs pa{};
  pa.src_q = q; pa.src_k = k; pa.src_v = v; pa.src_bstride = seq * ld; pa.src_ld = ld;
  pa.batch = batch; pa.seq = seq; pa.seq_pad = (int)Lp; pa.heads = heads; pa.head_dim = 128; pa.l_img = seq;
  pa.qh = qh; pa.kh = kh; pa.vt = vt;
  FLUX_HIP(launch_prep(pa, kBF16, st), "head-major layout");
  FLUX_HIP(attention_bwd(batch, seq, heads, qh, kh, vt, lse, dout, seq * ldo, ldo, o, seq * ldo, ldo, false, w, st),
           "attention backward");
  PrepBwdArgs pb{};
  pb.dq = w.dq; pb.dk = w.dk; pb.dv = w.dv;
  pb.dst = dqkv; pb.dst_bstride = (int64_t)seq * 3 * D; pb.dst_ld = 3 * D;
  pb.batch = batch; pb.seq = seq; pb.seq_pad = (int)Lp; pb.heads = heads; pb.l_img = seq;
  pb.part = part;
  FLUX_HIP(launch_prep_bwd(pb, st), "token-major gradients");
  return FLUX_OK;
}


// ------------------- loss, output head and embeddings -------------------
flux_status flux_rf_loss_grad(int32_t batch, int64_t n_per_sample, const float* v_pred, const float* z0,
                              const float* z1, float* dv, void* stream) {
  g_err[0] = 0;
  REQUIRE(batch >= 1 && n_per_sample >= 1, "batch and n_per_sample must be >= 1");
  REQUIRE(v_pred && z0 && z1 && dv, "v_pred, z0, z1 and dv are required");
  FLUX_HIP(launch_rf_loss_grad(v_pred, z0, z1, dv, (int64_t)batch * n_per_sample, static_cast<hipStream_t>(stream)),
           "loss gradient");
  return FLUX_OK;
}

namespace {
struct FinalBwdWs {
  float* mod; void* h; void* dtok; void* dtokT; void* hT; void* woT; float* dh; float* dm; Parts pt;
  size_t bytes;
};
FinalBwdWs final_bwd_ws(int64_t B, int64_t C, int64_t HW, int64_t D, void* base) {
  Carve c(base);
  FinalBwdWs w{};
  const int64_t T = B * HW, Tp = tok_pad(T);
  w.mod = static_cast<float*>(c.take(B * 2 * D * 4));
  w.h = c.take(T * D * 2);
  w.dtok = c.take(T * C * 2);
  w.dtokT = c.take(C * Tp * 2);
  w.hT = c.take(D * Tp * 2);
  w.woT = c.take(D * C * 2);
  w.dh = static_cast<float*>(c.take(T * D * 4));
  w.dm = static_cast<float*>(c.take(B * 2 * D * 4));
  w.pt.col = static_cast<float*>(c.take(kColParts * (C > D ? C : D) * 4));
  const int64_t ln_parts = B * ln_bwd_blocks((int)HW, (int)B) * 4 * D;
  w.pt.ln_sh = static_cast<float*>(c.take(ln_parts * 4));
  w.pt.ln_sc = static_cast<float*>(c.take(ln_parts * 4));
  w.pt.mod = static_cast<float*>(c.take(B * kModParts * D * 4));
  w.bytes = (size_t)round_up((int64_t)c.off, 256);
  return w;
}

struct EmbedBwdWs {
  void* tok; void* tokT; void* dT; void* txtT; float* emb; float* a1; float* da1; Parts pt;
  size_t bytes;
};
EmbedBwdWs embed_bwd_ws(int64_t B, int64_t C, int64_t HW, int64_t Lt, int64_t ctx, int64_t D, void* base) {
  Carve c(base);
  EmbedBwdWs w{};
  const int64_t Ti = tok_pad(B * HW), Tt = tok_pad(B * (Lt > 0 ? Lt : 1));
  const int64_t Tm = Ti > Tt ? Ti : Tt;
  w.tok = c.take(B * HW * C * 2);
  w.tokT = c.take(C * Ti * 2);
  w.dT = c.take(D * Tm * 2);
  w.txtT = c.take((ctx > 0 ? ctx : 1) * Tt * 2);
  w.emb = static_cast<float*>(c.take(B * 256 * 4));
  w.a1 = static_cast<float*>(c.take(B * D * 4));
  w.da1 = static_cast<float*>(c.take(B * D * 4));
  w.pt.col = static_cast<float*>(c.take(kColParts * D * 4));
  w.pt.mod = static_cast<float*>(c.take(B * kModParts * D * 4));
  w.bytes = (size_t)round_up((int64_t)c.off, 256);
  return w;
}
}  // namespace

size_t flux_final_bwd_workspace_bytes(int32_t batch, int32_t channels, int32_t height, int32_t width, int32_t hidden) {
  if (batch < 1 || channels < 1 || height < 1 || width < 1 || hidden < 1) return 0;
  return final_bwd_ws(batch, channels, (int64_t)height * width, hidden, nullptr).bytes;
}

flux_status flux_final_bwd(int32_t batch, int32_t channels, int32_t height, int32_t width, int32_t hidden, float eps,
                           const void* mod_w, const void* mod_b, const void* out_w, const float* x_img,
                           int64_t bstride, const float* vec, const float* dv, float* dx_img, float* dvec,
                           float* g_mod_w, float* g_mod_b, float* g_out_w, float* g_out_b, void* workspace,
                           size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  REQUIRE(batch >= 1 && channels >= 1 && height >= 1 && width >= 1, "sizes must be >= 1");
  if (hidden % 256 != 0 || hidden > 4096)
    return fail(FLUX_ERR_UNSUPPORTED, "hidden %d unsupported (a multiple of 256, at most 4096)", hidden);
  if (channels % 64 != 0) return fail(FLUX_ERR_UNSUPPORTED, "channels must be a multiple of 64 (got %d)", channels);
  REQUIRE(eps > 0.f, "eps must be positive");
  const void* req[] = {mod_w, mod_b, out_w, x_img, vec, dv, dx_img, dvec, g_mod_w, g_mod_b, g_out_w, g_out_b};
  for (const void* p : req) REQUIRE(p && aligned16(p), "every pointer is required, 16-byte aligned");
  const int64_t B = batch, C = channels, HW = (int64_t)height * width, D = hidden, T = B * HW, Tp = tok_pad(T);
  REQUIRE(bstride >= HW * D && bstride % 4 == 0, "bstride too small or not a multiple of 4");
  flux_status s = check_workspace(workspace, workspace_bytes, final_bwd_ws(B, C, HW, D, nullptr).bytes);
  if (s != FLUX_OK) return s;
  const FinalBwdWs w = final_bwd_ws(B, C, HW, D, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const RowMap xm = rmap(bstride, D, HW), rowsD = rmap(T * D, D, T), rowsC = rmap(T * C, C, T), none = rmap(0, 1, 1);
  GemvBatch gv{};
  gv.count = 1;
  gv.p[0] = gemv_problem(mod_w, mod_b, (int)(2 * D), (int)D, vec, D, w.mod, 2 * D, 1, 0);
  FLUX_HIP(run_gemv(gv, (int)B, kBF16, st), "final modulation GEMV");
  LnArgs la{};
  la.count = 1; la.dim = (int)D; la.eps = eps;
  la.s[0].x = x_img; la.s[0].xmap = xm;
  la.s[0].out = w.h; la.s[0].omap = rmap(HW * D, D, HW);
  la.s[0].shift = w.mod; la.s[0].scale = w.mod + D; la.s[0].mod_bstride = 2 * D;
  la.s[0].rows = (int32_t)T;
  FLUX_HIP(launch_ln_mod(la, kBF16, st), "final LayerNorm-modulate");
  FLUX_HIP(launch_patchify(dv, (int)B, (int)C, (int)HW, w.dtok, kBF16, st), "velocity gradient tokens");
  FLUX_HIP(colsum(w.dtok, kBF16, rowsC, nullptr, none, T, C, 1, g_out_b, 0, w.pt.col, st), "output bias gradient");
  FLUX_HIP(transpose_rows(out_w, kBF16, rmap(C * D, D, C), C, D, w.woT, C, st), "W_out^T");
  FLUX_HIP(transpose_rows(w.dtok, kBF16, rowsC, T, C, w.dtokT, Tp, st), "dtok^T");
  FLUX_HIP(transpose_rows(w.h, kBF16, rowsD, T, D, w.hT, Tp, st), "h^T");
  GemmBatch g{};
  g.count = 1;
  g.p[0] = bf16_problem(w.dtok, rowsC, w.woT, nullptr, T, D, C, w.dh, rowsD, true);
  FLUX_HIP(launch_gemm(g, kBF16, st), "output data gradient");
  g.p[0] = bf16_problem(w.dtokT, rmap(C * Tp, Tp, C), w.hT, nullptr, C, D, Tp, g_out_w, rmap(C * D, D, C), true);
  FLUX_HIP(launch_gemm(g, kBF16, st), "output weight gradient");
  FLUX_HIP(ln_bwd(x_img, xm, w.dh, rowsD, dx_img, xm, w.mod + D, 2 * D, w.dm, w.dm + D, HW, B, D, eps, w.pt, st),
           "final LayerNorm-modulate backward");
  FLUX_HIP(mod_bwd(mod_w, vec, w.dm, 2 * D, D, B, g_mod_w, g_mod_b, dvec, w.pt, st), "final modulation backward");
  return FLUX_OK;
}

size_t flux_embed_bwd_workspace_bytes(int32_t batch, int32_t channels, int32_t height, int32_t width, int32_t l_txt,
                                      int32_t ctx_dim, int32_t hidden) {
  if (batch < 1 || channels < 1 || height < 1 || width < 1 || hidden < 1 || l_txt < 0 || ctx_dim < 0) return 0;
  return embed_bwd_ws(batch, channels, (int64_t)height * width, l_txt, ctx_dim, hidden, nullptr).bytes;
}

flux_status flux_embed_bwd(int32_t batch, int32_t channels, int32_t height, int32_t width, int32_t l_txt,
                           int32_t ctx_dim, int32_t hidden, int32_t time_dim, int32_t y_dim,
                           const flux_embed_weights* w, const float* z_t, const void* txt, const float* t,
                           const float* y, const float* guidance, const float* d_img, int64_t img_bstride,
                           const float* d_txt, int64_t txt_bstride, const float* dvec, const flux_embed_grads* g,
                           void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  REQUIRE(batch >= 1 && channels >= 1 && height >= 1 && width >= 1 && hidden >= 1, "sizes must be >= 1");
  REQUIRE(w && g && w->img_in_w && w->time_in1_w && w->time_in1_b && w->time_in2_w && w->time_in2_b,
          "image and time embedder weights and the gradient struct are required");
  REQUIRE(z_t && t && d_img && dvec && aligned16(z_t) && aligned16(d_img) && aligned16(dvec),
          "z_t, t, d_img and dvec are required (16-byte aligned)");
  REQUIRE(time_dim >= 8 && time_dim % 8 == 0 && time_dim <= 256, "time_dim must be a multiple of 8 in [8, 256]");
  if (channels % 64 != 0) return fail(FLUX_ERR_UNSUPPORTED, "channels must be a multiple of 64 (got %d)", channels);
  REQUIRE(hidden % 8 == 0 && hidden <= 4096, "hidden must be a multiple of 8, at most 4096");
  const int64_t B = batch, C = channels, HW = (int64_t)height * width, D = hidden;
  REQUIRE(img_bstride >= HW * D && img_bstride % 4 == 0, "img_bstride too small or not a multiple of 4");
  const bool has_txt = w->txt_in_w != nullptr, has_y = w->vector_in1_w != nullptr;
  float* const gp[] = {g->img_in_w, g->img_in_b, g->time_in1_w, g->time_in1_b, g->time_in2_w, g->time_in2_b};
  for (float* p : gp) REQUIRE(p && aligned16(p), "gradient pointers must be non-NULL and 16-byte aligned");
  if (has_txt) {
    REQUIRE(txt && d_txt && l_txt >= 1 && ctx_dim >= 1 && g->txt_in_w && g->txt_in_b, "txt_in needs txt, d_txt and its gradients");
    if (ctx_dim % 64 != 0) return fail(FLUX_ERR_UNSUPPORTED, "ctx_dim must be a multiple of 64");
    REQUIRE(txt_bstride >= (int64_t)l_txt * D && txt_bstride % 4 == 0, "txt_bstride too small");
    REQUIRE(aligned16(txt) && aligned16(d_txt) && aligned16(g->txt_in_w) && aligned16(g->txt_in_b),
            "pointers must be 16-byte aligned");
  }
  if (has_y)
    REQUIRE(y && y_dim >= 8 && y_dim % 8 == 0 && w->vector_in2_w && g->vector_in1_w && g->vector_in1_b &&
                g->vector_in2_w && g->vector_in2_b,
            "vector_in needs y (y_dim a multiple of 8) and its gradients");
  if (guidance)
    REQUIRE(w->guidance_in_w && g->guidance_in_w && g->guidance_in_b && aligned16(g->guidance_in_w) &&
                aligned16(g->guidance_in_b),
            "guidance needs the guidance embedding's weight and 16-byte aligned gradients");
  const int64_t Lt = has_txt ? l_txt : 0, ctx = has_txt ? ctx_dim : 0;
  flux_status s = check_workspace(workspace, workspace_bytes, embed_bwd_ws(B, C, HW, Lt, ctx, D, nullptr).bytes);
  if (s != FLUX_OK) return s;
  const EmbedBwdWs ws = embed_bwd_ws(B, C, HW, Lt, ctx, D, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const RowMap none = rmap(0, 1, 1);
  const int64_t Ti = tok_pad(B * HW);
  // image input linear: dW = d_img^T patchify(z_t), db = sum d_img
  FLUX_HIP(launch_patchify(z_t, (int)B, (int)C, (int)HW, ws.tok, kBF16, st), "patchify");
  FLUX_HIP(transpose_rows(ws.tok, kBF16, rmap(B * HW * C, C, B * HW), B * HW, C, ws.tokT, Ti, st), "tokens^T");
  FLUX_HIP(transpose_rows(d_img, kF32, rmap(img_bstride, D, HW), B * HW, D, ws.dT, Ti, st), "d_img^T");
  GemmBatch gb{};
  gb.count = 1;
  gb.p[0] = bf16_problem(ws.dT, rmap(D * Ti, Ti, D), ws.tokT, nullptr, D, C, Ti, g->img_in_w, rmap(D * C, C, D), true);
  FLUX_HIP(launch_gemm(gb, kBF16, st), "image input weight gradient");
  FLUX_HIP(colsum(d_img, kF32, rmap(img_bstride, D, HW), nullptr, none, B * HW, D, 1, g->img_in_b, 0, ws.pt.col, st),
           "image input bias gradient");
  if (has_txt) {
    const int64_t Tt = tok_pad(B * Lt);
    FLUX_HIP(transpose_rows(txt, kBF16, rmap(Lt * ctx, ctx, Lt), B * Lt, ctx, ws.txtT, Tt, st), "txt^T");
    FLUX_HIP(transpose_rows(d_txt, kF32, rmap(txt_bstride, D, Lt), B * Lt, D, ws.dT, Tt, st), "d_txt^T");
    gb.p[0] = bf16_problem(ws.dT, rmap(D * Tt, Tt, D), ws.txtT, nullptr, D, ctx, Tt, g->txt_in_w,
                           rmap(D * ctx, ctx, D), true);
    FLUX_HIP(launch_gemm(gb, kBF16, st), "text input weight gradient");
    FLUX_HIP(colsum(d_txt, kF32, rmap(txt_bstride, D, Lt), nullptr, none, B * Lt, D, 1, g->txt_in_b, 0, ws.pt.col,
                    st), "text input bias gradient");
  }
  // embedders: vec += W2 SiLU(W1 e + b1) + b2, e the timestep sinusoid or y
  FLUX_HIP(launch_timestep_embed(t, (int)B, time_dim, 1000.f, 10000.f, ws.emb, st), "timestep sinusoid");
  auto mlp_bwd = [&](const void* w1, const void* b1, const void* w2, const float* e, int64_t K, float* g1w, float* g1b,
                     float* g2w, float* g2b) -> flux_status {
    GemvBatch gv{};
    gv.count = 1;
    gv.p[0] = gemv_problem(w1, b1, (int)D, (int)K, e, K, ws.a1, D, 0, 0);
    FLUX_HIP(run_gemv(gv, (int)B, kBF16, st), "embedder layer 1");
    ModBwdArgs a{};
    a.w = w2; a.vec = ws.a1; a.dm = dvec; a.dm_bstride = D; a.dw = g2w; a.db = g2b; a.dvec = ws.da1;
    a.N = (int32_t)D; a.K = (int32_t)D; a.batch = (int32_t)B; a.nrc = kModParts; a.silu_in = 1; a.dvec_store = 1;
    a.part = ws.pt.mod;
    FLUX_HIP(launch_mod_bwd(a, kBF16, st), "embedder layer 2 backward");
    ModBwdArgs b{};
    b.w = w1; b.vec = e; b.dm = ws.da1; b.dm_bstride = D; b.dw = g1w; b.db = g1b; b.dvec = nullptr;
    b.N = (int32_t)D; b.K = (int32_t)K; b.batch = (int32_t)B; b.nrc = kModParts; b.silu_in = 0;
    b.part = ws.pt.mod;
    FLUX_HIP(launch_mod_bwd(b, kBF16, st), "embedder layer 1 backward");
    return FLUX_OK;
  };
  if ((s = mlp_bwd(w->time_in1_w, w->time_in1_b, w->time_in2_w, ws.emb, time_dim, g->time_in1_w, g->time_in1_b,
                   g->time_in2_w, g->time_in2_b)) != FLUX_OK)
    return s;
  if (has_y && (s = mlp_bwd(w->vector_in1_w, w->vector_in1_b, w->vector_in2_w, y, y_dim, g->vector_in1_w,
                            g->vector_in1_b, g->vector_in2_w, g->vector_in2_b)) != FLUX_OK)
    return s;
  if (guidance)
    FLUX_HIP(launch_guidance_bwd(dvec, guidance, (int)B, (int)D, g->guidance_in_w, g->guidance_in_b, st),
             "guidance embedding backward");
  return FLUX_OK;
}

}  // extern "C"
