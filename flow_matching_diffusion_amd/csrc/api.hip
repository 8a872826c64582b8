// libflux C ABI: argument validation, workspace layout and launch sequences
// of the Flux double block, single block, embeddings, output head and the
// rectified-flow objective.  Every check runs on the host before anything is
// enqueued; the library never allocates, frees or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/flux.h"
#include "api_common.h"
#include "common.h"
#include "kernels.h"

using namespace flux;
using namespace flux::api;

// Destination of the fused q|k|v epilogue: the attention operand layouts
// (head-major q, k; transposed v) with RMSNorm scales gq / gk and the RoPE
// table; tok0 is the joint position of the problem's first row of a sample.
static QkvOut qkv_out(const flux_dims* d, void* qh, void* kh, void* vt, const float* gq, const float* gk,
                      const float* rope, int64_t L, int64_t Lp, int64_t tok0) {
  QkvOut q{};
  q.qh = qh; q.kh = kh; q.vt = vt; q.gq = gq; q.gk = gk; q.rope = rope;
  q.heads = d->heads; q.seq = (int32_t)L; q.seq_pad = (int32_t)Lp; q.tok0 = (int32_t)tok0; q.eps = d->eps;
  return q;
}

// ================================ public API ================================
extern "C" {

const char* flux_status_string(flux_status s) {
  switch (s) {
    case FLUX_OK: return "ok";
    case FLUX_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FLUX_ERR_UNSUPPORTED: return "unsupported";
    case FLUX_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FLUX_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* flux_last_error(void) { return g_err; }

int32_t flux_gemm_stream_k(int32_t mode, int32_t spin) { return gemm_stream_k(mode, spin); }

size_t flux_workspace_bytes(const flux_dims* d, int32_t op) {
  if (check_dims(d) != FLUX_OK) return 0;
  if (op == 0 || op == 2) return block_ws(d, nullptr).bytes;   // the sequential block is a one-stream double block
  if (op == 1) return single_ws(d, nullptr).bytes;
  return 0;
}

// --------------------------------- double block --------------------------------
flux_status flux_block_fwd(const flux_dims* d, const flux_stream_weights* iw, const flux_stream_weights* tw,
                           float* img, int64_t img_bstride, float* txt, int64_t txt_bstride, const float* vec,
                           const float* rope, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  flux_status s = check_dims(d);
  if (s != FLUX_OK) return s;
  const int64_t B = d->batch, Li = d->l_img, Lt = d->l_txt, L = Li + Lt, D = d->hidden, F = d->mlp_hidden;
  const bool f32 = d->precision == FLUX_PREC_F32, fp8 = d->precision == FLUX_PREC_FP8_E4M3;
  const int dt = f32 ? kF32 : kBF16, es = esize(d->precision), aes = act_esize(d->precision);
  if ((s = check_stream_weights(iw, "image")) != FLUX_OK) return s;
  if (Lt > 0 && (s = check_stream_weights(tw, "text")) != FLUX_OK) return s;
  if (fp8 && (s = check_fp8_records(iw->fp8, "image weights")) != FLUX_OK) return s;
  if (fp8 && Lt > 0 && (s = check_fp8_records(tw->fp8, "text weights")) != FLUX_OK) return s;
  REQUIRE(img && aligned16(img), "img must be a non-NULL 16-byte aligned pointer");
  REQUIRE(img_bstride >= Li * D && img_bstride % 4 == 0, "img_bstride must be >= l_img*hidden and a multiple of 4");
  if (Lt > 0) {
    REQUIRE(txt && aligned16(txt), "txt must be a non-NULL 16-byte aligned pointer");
    REQUIRE(txt_bstride >= Lt * D && txt_bstride % 4 == 0,
            "txt_bstride must be >= l_txt*hidden and a multiple of 4");
  }
  REQUIRE(vec && aligned16(vec), "vec must be a non-NULL 16-byte aligned pointer");
  REQUIRE(rope && aligned16(rope), "rope must be a non-NULL 16-byte aligned pointer");
  const BlockWs need = block_ws(d, nullptr);
  if ((s = check_workspace(workspace, workspace_bytes, need.bytes)) != FLUX_OK) return s;
  const BlockWs w = block_ws(d, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // element types: fp32 workloads use float everywhere; bf16 workloads run the
  // linears on fp16 activations (bf16 weights converted in LDS, or fp16
  // weights) and attention on bf16 q, k, v; fp8 workloads run the linears on
  // E4M3 activations and weights, attention on bf16
  const int act = f32 ? kF32 : fp8 ? kFP8 : kF16, qkv_t = f32 ? kF32 : kBF16;
  const int lin = f32 ? kF32 : fp8 ? kFP8 : (d->weights_f16 ? kF16W : kF16);   // GEMM operand type
  const int ns = Lt > 0 ? 2 : 1;
  const flux_stream_weights* sw[2] = {iw, tw};
  // fp8 state records of a stream (null unless fp8)
  auto rec = [&](int i, int slot) -> flux_fp8_tensor* { return fp8 ? sw[i]->fp8 + slot : nullptr; };
  float* xs[2] = {img, txt};
  const int64_t xbs[2] = {img_bstride, txt_bstride};
  const int64_t seg[2] = {Li, Lt};
  const int64_t off[2] = {0, Li};   // first joint row of each stream

  // 1. adaLN modulation of both streams: Linear(SiLU(vec)) -> 6 chunks
  GemvBatch gv{};
  gv.count = ns;
  for (int i = 0; i < ns; ++i)
    gv.p[i] = gemv_problem(sw[i]->mod_w, sw[i]->mod_b, (int)(6 * D), (int)D, vec, D, w.mod[i], 6 * D, 1, 0);
  FLUX_HIP(run_gemv(gv, (int)B, dt, st), "modulation GEMV");

  auto ln_mod = [&](int chunk_shift) -> hipError_t {
    LnArgs a{};
    a.count = ns;
    a.dim = (int)D;
    a.eps = d->eps;
    for (int i = 0; i < ns; ++i) {
      a.s[i].x = xs[i];
      a.s[i].xmap = rmap(xbs[i], D, seg[i]);
      a.s[i].out = elem_ptr(w.h, off[i] * D, aes);
      a.s[i].omap = rmap(L * D, D, seg[i]);
      a.s[i].q = rec(i, chunk_shift == 0 ? FLUX_FP8_QKV_X : FLUX_FP8_FC1_X);
      a.s[i].shift = w.mod[i] + chunk_shift * D;
      a.s[i].scale = w.mod[i] + (chunk_shift + 1) * D;
      a.s[i].mod_bstride = 6 * D;
      a.s[i].rows = (int32_t)(B * seg[i]);
    }
    return launch_ln_mod(a, act, st);
  };
  // 2. h = LN(x)(1 + scale1) + shift1
  FLUX_HIP(ln_mod(0), "LayerNorm-modulate (attention)");

  // 3. q|k|v = Linear_qkv(h) per stream, one grouped launch
  GemmBatch g{};
  attach_sk(g, w.sk);
  g.count = ns;
  for (int i = 0; i < ns; ++i)
    g.p[i] = gemm_problem(elem_ptr(w.h, off[i] * D, aes), rmap(L * D, D, seg[i]), sw[i]->qkv_w, sw[i]->qkv_b,
                          (int)(B * seg[i]), (int)(3 * D), (int)D, kEpiStore, elem_ptr(w.big, off[i] * 3 * D, es),
                          rmap(L * 3 * D, 3 * D, seg[i]));
  for (int i = 0; i < ns; ++i) {
    g.p[i].out0_dt = qkv_t;
    g.p[i].qa = rec(i, FLUX_FP8_QKV_X);
    g.p[i].qw = rec(i, FLUX_FP8_QKV_W);
  }
  const int64_t Lp = seq_pad_of(L);
  // 3-4 fused: on the persistent GEMM the epilogue applies RMSNorm(q),
  // RMSNorm(k) and RoPE and writes the attention layouts itself
  if (!f32 && d->head_dim == 128 && gemm_is_persistent(g, lin)) {
    for (int i = 0; i < ns; ++i) {
      g.p[i].epi = kEpiQkv;
      g.p[i].qkv = qkv_out(d, w.qh, w.kh, w.vt, sw[i]->q_norm, sw[i]->k_norm, rope, L, Lp, off[i]);
    }
    FLUX_HIP(launch_attn_pad_zero(w.qh, w.kh, w.vt, (int)B, d->heads, (int)L, (int)Lp, st), "attention padding");
    FLUX_HIP(launch_gemm(g, lin, st), "qkv GEMM + q/k norm + RoPE");
  } else {
  FLUX_HIP(launch_gemm(g, lin, st), "qkv GEMM");

  // 4. RMSNorm(q), RMSNorm(k), RoPE, head-major layout
  PrepArgs pa{};
  pa.src_q = w.big;
  pa.src_k = elem_ptr(w.big, D, es);
  pa.src_v = elem_ptr(w.big, 2 * D, es);
  pa.src_bstride = L * 3 * D;
  pa.src_ld = 3 * D;
  pa.batch = (int)B; pa.seq = (int)L; pa.seq_pad = (int)Lp; pa.heads = d->heads; pa.head_dim = d->head_dim;
  pa.l_img = (int)Li;
  pa.gq_img = iw->q_norm; pa.gk_img = iw->k_norm;
  pa.gq_txt = Lt > 0 ? tw->q_norm : iw->q_norm;
  pa.gk_txt = Lt > 0 ? tw->k_norm : iw->k_norm;
  pa.rope = rope; pa.eps = d->eps;
  pa.qh = w.qh; pa.kh = w.kh; pa.vt = w.vt;
  FLUX_HIP(launch_prep(pa, qkv_t, st), "q/k norm + RoPE");
  }

  // 5. joint attention over image|text rows
  AttnArgs aa{};
  aa.qh = w.qh; aa.kh = w.kh; aa.vt = w.vt;
  aa.out = w.o; aa.out_bstride = L * D; aa.out_ld = D;
  aa.batch = (int)B; aa.seq = (int)L; aa.seq_pad = (int)Lp; aa.heads = d->heads; aa.head_dim = d->head_dim;
  aa.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d->head_dim));
  aa.oq[0] = rec(0, FLUX_FP8_PROJ_X);
  aa.oq[1] = ns > 1 ? rec(1, FLUX_FP8_PROJ_X) : nullptr;
  aa.l_img = (int)Li;
  FLUX_HIP(launch_attention(aa, qkv_t, act, st), "joint attention");

  // 6. x += gate1 * Linear_proj(O)
  for (int i = 0; i < ns; ++i) {
    g.p[i] = gemm_problem(elem_ptr(w.o, off[i] * D, aes), rmap(L * D, D, seg[i]), sw[i]->proj_w, sw[i]->proj_b,
                          (int)(B * seg[i]), (int)D, (int)D, kEpiResid, xs[i], rmap(xbs[i], D, seg[i]));
    g.p[i].gate = w.mod[i] + 2 * D;
    g.p[i].gate_bstride = 6 * D;
    g.p[i].qa = rec(i, FLUX_FP8_PROJ_X);
    g.p[i].qw = rec(i, FLUX_FP8_PROJ_W);
  }
  FLUX_HIP(launch_gemm(g, lin, st), "output projection GEMM");

  // 7. h = LN(x)(1 + scale2) + shift2
  FLUX_HIP(ln_mod(3), "LayerNorm-modulate (MLP)");

  // 8. u = GELU(fc1(h))
  for (int i = 0; i < ns; ++i)
    g.p[i] = gemm_problem(elem_ptr(w.h, off[i] * D, aes), rmap(L * D, D, seg[i]), sw[i]->fc1_w, sw[i]->fc1_b,
                          (int)(B * seg[i]), (int)F, (int)D, kEpiGelu, elem_ptr(w.big, off[i] * F, aes),
                          rmap(L * F, F, seg[i]));
  for (int i = 0; i < ns; ++i) {
    g.p[i].out0_dt = act;
    g.p[i].qa = rec(i, FLUX_FP8_FC1_X);
    g.p[i].qw = rec(i, FLUX_FP8_FC1_W);
    g.p[i].qo = rec(i, FLUX_FP8_FC2_X);
  }
  FLUX_HIP(launch_gemm(g, lin, st), "fc1 GEMM");

  // 9. x += gate2 * fc2(u)
  for (int i = 0; i < ns; ++i) {
    g.p[i] = gemm_problem(elem_ptr(w.big, off[i] * F, aes), rmap(L * F, F, seg[i]), sw[i]->fc2_w, sw[i]->fc2_b,
                          (int)(B * seg[i]), (int)D, (int)F, kEpiResid, xs[i], rmap(xbs[i], D, seg[i]));
    g.p[i].gate = w.mod[i] + 5 * D;
    g.p[i].gate_bstride = 6 * D;
    g.p[i].qa = rec(i, FLUX_FP8_FC2_X);
    g.p[i].qw = rec(i, FLUX_FP8_FC2_W);
  }
  FLUX_HIP(launch_gemm(g, lin, st), "fc2 GEMM");
  if (debug_checks_on())
    for (int i = 0; i < ns; ++i)
      FLUX_HIP(debug_check(xs[i], kF32, B, seg[i] * D, xbs[i], -kDbgBig, kDbgBig, FLUX_DBG_NONFINITE_RESIDUAL, st),
               "debug check of the residual");
  return FLUX_OK;
}

// --------------------------- sequential single block ---------------------------
flux_status flux_single_seq_fwd(const flux_dims* d, const flux_stream_weights* w, float* x, int64_t x_bstride,
                                const float* vec, const float* rope, void* workspace, size_t workspace_bytes,
                                void* stream) {
  g_err[0] = 0;
  flux_status s = check_dims(d);
  if (s != FLUX_OK) return s;
  // the whole joint sequence as the one (image) stream of a double block: same
  // L, same workspace layout, rope rows in the same order
  flux_dims one = *d;
  one.l_img = d->l_img + d->l_txt;
  one.l_txt = 0;
  return flux_block_fwd(&one, w, nullptr, x, x_bstride, nullptr, 0, vec, rope, workspace, workspace_bytes, stream);
}

// --------------------------------- single block --------------------------------
flux_status flux_single_fwd(const flux_dims* d, const flux_single_weights* sw, float* x, int64_t x_bstride,
                            const float* vec, const float* rope, void* workspace, size_t workspace_bytes,
                            void* stream) {
  g_err[0] = 0;
  flux_status s = check_dims(d);
  if (s != FLUX_OK) return s;
  const int64_t B = d->batch, L = (int64_t)d->l_img + d->l_txt, D = d->hidden, F = d->mlp_hidden;
  const bool f32 = d->precision == FLUX_PREC_F32, fp8 = d->precision == FLUX_PREC_FP8_E4M3;
  const int dt = f32 ? kF32 : kBF16, es = esize(d->precision), aes = act_esize(d->precision);
  REQUIRE(sw, "single-block weights are NULL");
  REQUIRE(sw->mod_w && sw->mod_b && sw->lin1_w && sw->lin1_b && sw->q_norm && sw->k_norm && sw->lin2_w &&
              sw->lin2_b,
          "single-block weights: a pointer is NULL");
  {
    const void* ps[] = {sw->mod_w, sw->mod_b, sw->lin1_w, sw->lin1_b, sw->q_norm, sw->k_norm, sw->lin2_w, sw->lin2_b};
    for (const void* p : ps) REQUIRE(aligned16(p), "single-block weights: pointers must be 16-byte aligned");
  }
  if (fp8 && (s = check_fp8_records(sw->fp8, "single-block weights")) != FLUX_OK) return s;
  REQUIRE(x && aligned16(x), "x must be a non-NULL 16-byte aligned pointer");
  REQUIRE(x_bstride >= L * D && x_bstride % 4 == 0, "x_bstride must be >= L*hidden and a multiple of 4");
  REQUIRE(vec && aligned16(vec), "vec must be a non-NULL 16-byte aligned pointer");
  REQUIRE(rope && aligned16(rope), "rope must be a non-NULL 16-byte aligned pointer");
  const SingleWs need = single_ws(d, nullptr);
  if ((s = check_workspace(workspace, workspace_bytes, need.bytes)) != FLUX_OK) return s;
  const SingleWs w = single_ws(d, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int act = f32 ? kF32 : fp8 ? kFP8 : kF16, qkv_t = f32 ? kF32 : kBF16;
  const int lin = f32 ? kF32 : fp8 ? kFP8 : (d->weights_f16 ? kF16W : kF16);   // GEMM operand type
  auto rec = [&](int slot) -> flux_fp8_tensor* { return fp8 ? sw->fp8 + slot : nullptr; };

  // 1. (shift, scale, gate) = Linear(SiLU(vec))
  GemvBatch gv{};
  gv.count = 1;
  gv.p[0] = gemv_problem(sw->mod_w, sw->mod_b, (int)(3 * D), (int)D, vec, D, w.mod, 3 * D, 1, 0);
  FLUX_HIP(run_gemv(gv, (int)B, dt, st), "modulation GEMV");

  // 2. h = LN(x)(1 + scale) + shift
  LnArgs la{};
  la.count = 1;
  la.dim = (int)D;
  la.eps = d->eps;
  la.s[0].x = x; la.s[0].xmap = rmap(x_bstride, D, L);
  la.s[0].out = w.h; la.s[0].omap = rmap(L * D, D, L);
  la.s[0].shift = w.mod; la.s[0].scale = w.mod + D; la.s[0].mod_bstride = 3 * D;
  la.s[0].q = rec(FLUX_FP8_LIN1_X);
  la.s[0].rows = (int32_t)(B * L);
  FLUX_HIP(launch_ln_mod(la, act, st), "LayerNorm-modulate");

  // 3. q|k|v -> qkv buffer; GELU(mlp_in) -> columns D.. of the linear2 input
  GemmBatch g{};
  attach_sk(g, w.sk);
  g.count = 1;
  g.p[0] = gemm_problem(w.h, rmap(L * D, D, L), sw->lin1_w, sw->lin1_b, (int)(B * L), (int)(3 * D + F), (int)D,
                        kEpiSplitGelu, w.qkv, rmap(L * 3 * D, 3 * D, L));
  g.p[0].out1 = elem_ptr(w.cat, D, aes);
  g.p[0].omap1 = rmap(L * (D + F), D + F, L);
  g.p[0].n_split = (int)(3 * D);
  g.p[0].out0_dt = qkv_t;
  g.p[0].out1_dt = act;
  g.p[0].qa = rec(FLUX_FP8_LIN1_X);
  g.p[0].qw = rec(FLUX_FP8_LIN1_W);
  g.p[0].qo = rec(FLUX_FP8_LIN2_X);
  const int64_t Lp = seq_pad_of(L);
  // 3-4 fused on the persistent GEMM: q|k|v columns go to the attention
  // layouts with RMSNorm and RoPE applied, the rest through GELU
  if (!f32 && d->head_dim == 128 && gemm_is_persistent(g, lin)) {
    g.p[0].epi = kEpiQkvSplitGelu;
    g.p[0].qkv = qkv_out(d, w.qh, w.kh, w.vt, sw->q_norm, sw->k_norm, rope, L, Lp, 0);
    FLUX_HIP(launch_attn_pad_zero(w.qh, w.kh, w.vt, (int)B, d->heads, (int)L, (int)Lp, st), "attention padding");
    FLUX_HIP(launch_gemm(g, lin, st), "linear1 GEMM + q/k norm + RoPE");
  } else {
  FLUX_HIP(launch_gemm(g, lin, st), "linear1 GEMM");

  // 4. RMSNorm(q), RMSNorm(k), RoPE
  PrepArgs pa{};
  pa.src_q = w.qkv;
  pa.src_k = elem_ptr(w.qkv, D, es);
  pa.src_v = elem_ptr(w.qkv, 2 * D, es);
  pa.src_bstride = L * 3 * D;
  pa.src_ld = 3 * D;
  pa.batch = (int)B; pa.seq = (int)L; pa.seq_pad = (int)Lp; pa.heads = d->heads; pa.head_dim = d->head_dim;
  pa.l_img = (int)L;
  pa.gq_img = pa.gq_txt = sw->q_norm;
  pa.gk_img = pa.gk_txt = sw->k_norm;
  pa.rope = rope; pa.eps = d->eps;
  pa.qh = w.qh; pa.kh = w.kh; pa.vt = w.vt;
  FLUX_HIP(launch_prep(pa, qkv_t, st), "q/k norm + RoPE");
  }

  // 5. attention -> columns 0..D of the linear2 input
  AttnArgs aa{};
  aa.qh = w.qh; aa.kh = w.kh; aa.vt = w.vt;
  aa.out = w.cat; aa.out_bstride = L * (D + F); aa.out_ld = D + F;
  aa.batch = (int)B; aa.seq = (int)L; aa.seq_pad = (int)Lp; aa.heads = d->heads; aa.head_dim = d->head_dim;
  aa.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d->head_dim));
  aa.oq[0] = aa.oq[1] = rec(FLUX_FP8_LIN2_X);   // O and GELU(m) form one quantized tensor
  aa.l_img = (int)L;
  FLUX_HIP(launch_attention(aa, qkv_t, act, st), "attention");

  // 6. x += gate * Linear2([O | GELU(m)])
  g.p[0] = gemm_problem(w.cat, rmap(L * (D + F), D + F, L), sw->lin2_w, sw->lin2_b, (int)(B * L), (int)D,
                        (int)(D + F), kEpiResid, x, rmap(x_bstride, D, L));
  g.p[0].gate = w.mod + 2 * D;
  g.p[0].gate_bstride = 3 * D;
  g.p[0].qa = rec(FLUX_FP8_LIN2_X);
  g.p[0].qw = rec(FLUX_FP8_LIN2_W);
  FLUX_HIP(launch_gemm(g, lin, st), "linear2 GEMM");
  if (debug_checks_on())
    FLUX_HIP(debug_check(x, kF32, B, L * D, x_bstride, -kDbgBig, kDbgBig, FLUX_DBG_NONFINITE_RESIDUAL, st),
             "debug check of the residual");
  return FLUX_OK;
}

// ------------------------------ rectified flow ------------------------------
size_t flux_rf_workspace_bytes(int32_t batch, int64_t n) {
  if (batch < 1 || n < 1) return 0;
  return (size_t)round_up((int64_t)batch * rf_parts_per_sample(n) * 8, 256);
}

static bool overlap(const void* a, const void* b, int64_t bytes) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + bytes && y < x + bytes;
}
// [a, a + la) and [b, b + lb) share a byte
static bool ranges_overlap(const void* a, int64_t la, const void* b, int64_t lb) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + lb && y < x + la;
}

// Host-side checks shared by rf_noise_loss and rf_noise_loss_noalloc (the
// workspace is checked by the caller).
static flux_status rf_check(const rf_args* a) {
  REQUIRE(a, "args is NULL");
  REQUIRE(a->batch >= 1, "batch must be >= 1 (got %d)", a->batch);
  REQUIRE(a->n_per_sample >= 1, "n_per_sample must be >= 1");
  REQUIRE((int64_t)a->batch * a->n_per_sample < ((int64_t)1 << 40), "problem too large");
  REQUIRE(a->z0 && a->z1 && a->t, "z0, z1 and t are required");
  const float* ptrs[] = {a->z0, a->z1, a->t, a->z_t, a->v_target, a->v_pred, a->loss, a->loss_per_sample};
  for (const float* p : ptrs) REQUIRE(!p || aligned16(p), "tensor pointers must be 16-byte aligned");
  const int64_t bytes = (int64_t)a->batch * a->n_per_sample * 4;
  const float* outs[] = {a->z_t, a->v_target};
  for (const float* o : outs) {
    if (!o) continue;
    REQUIRE(!overlap(o, a->z0, bytes) && !overlap(o, a->z1, bytes), "z_t / v_target must not alias z0 or z1");
  }
  if (a->z_t && a->v_target) REQUIRE(!overlap(a->z_t, a->v_target, bytes), "z_t and v_target must not alias");
  if (a->loss || a->loss_per_sample) REQUIRE(a->v_pred, "a loss output needs v_pred");
  return FLUX_OK;
}

// Enqueue noising and loss; `partials` holds batch * rf_parts_per_sample(n)
// doubles when a loss is asked for.
static flux_status rf_launch(const rf_args* a, double* partials, hipStream_t st) {
  const bool dbg = debug_checks_on();
  if (dbg) FLUX_HIP(debug_check(a->t, kF32, 1, a->batch, a->batch, 0.f, 1.f, FLUX_DBG_T_RANGE, st), "debug check of t");
  if (a->z_t || a->v_target)
    FLUX_HIP(launch_rf_noise(a->batch, a->n_per_sample, a->z0, a->z1, a->t, a->z_t, a->v_target, st), "rf noise");
  if (a->loss || a->loss_per_sample)
    FLUX_HIP(launch_rf_loss(a->batch, a->n_per_sample, a->z0, a->z1, a->v_pred, a->loss, a->loss_per_sample,
                            partials, rf_parts_per_sample(a->n_per_sample), st),
             "rf loss");
  if (dbg && (a->loss || a->loss_per_sample)) {
    const int64_t n = (int64_t)a->batch * a->n_per_sample;
    FLUX_HIP(debug_check(a->v_pred, kF32, 1, n, n, -kDbgBig, kDbgBig, FLUX_DBG_NONFINITE_LOSS, st), "debug check of v_pred");
    FLUX_HIP(debug_check(a->loss, kF32, 1, 1, 1, -kDbgBig, kDbgBig, FLUX_DBG_NONFINITE_LOSS, st), "debug check of the loss");
    FLUX_HIP(debug_check(a->loss_per_sample, kF32, 1, a->batch, a->batch, -kDbgBig, kDbgBig, FLUX_DBG_NONFINITE_LOSS, st),
             "debug check of the per-sample loss");
  }
  return FLUX_OK;
}

flux_status rf_noise_loss(const rf_args* a, void* stream) {
  g_err[0] = 0;
  flux_status s = rf_check(a);
  if (s != FLUX_OK) return s;
  if (a->loss || a->loss_per_sample) {
    s = check_workspace(a->workspace, a->workspace_bytes, flux_rf_workspace_bytes(a->batch, a->n_per_sample));
    if (s != FLUX_OK) return s;
  }
  return rf_launch(a, static_cast<double*>(a->workspace), static_cast<hipStream_t>(stream));
}

// ------------------------- rf_noise_loss without a workspace -------------------------
// The loss partials live in a file-scope device array instead of a caller
// workspace.  In host code `scratch` names a host-side stand-in, so its device
// address is looked up once per device (hipGetSymbolAddress with that device
// current) and only that address is ever passed to kernels.
constexpr int kRfScratchDoubles = 8192;   // 64 KiB: batch * parts <= 8192
constexpr int kMaxDevices = 64;
static __device__ __align__(256) double scratch[kRfScratchDoubles];

static std::mutex g_scratch_mu;
static double* g_scratch_ptr[kMaxDevices];

static flux_status scratch_for_current_device(double** out) {
  int dev = -1;
  FLUX_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FLUX_ERR_UNSUPPORTED, "device ordinal %d above %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    FLUX_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p) return fail(FLUX_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = static_cast<double*>(p);
  }
  *out = g_scratch_ptr[dev];
  return FLUX_OK;
}

int64_t flux_rf_noalloc_max_partials(void) { return kRfScratchDoubles; }

flux_status rf_noise_loss_noalloc(const rf_args* a, void* stream) {
  g_err[0] = 0;
  flux_status s = rf_check(a);
  if (s != FLUX_OK) return s;
  double* partials = nullptr;
  if (a->loss || a->loss_per_sample) {
    const int64_t need = (int64_t)a->batch * rf_parts_per_sample(a->n_per_sample);
    if (need > kRfScratchDoubles)
      return fail(FLUX_ERR_WORKSPACE_TOO_SMALL,
                  "batch %d needs %lld loss partials, above the static scratch of %d; use rf_noise_loss",
                  a->batch, (long long)need, kRfScratchDoubles);
    if ((s = scratch_for_current_device(&partials)) != FLUX_OK) return s;
  }
  return rf_launch(a, partials, static_cast<hipStream_t>(stream));
}

// --------------------------------- sampling ---------------------------------
flux_status flux_euler_step(const flux_euler_args* a, void* stream) {
  g_err[0] = 0;
  REQUIRE(a, "args is NULL");
  REQUIRE(a->batch >= 1, "batch must be >= 1 (got %d)", a->batch);
  REQUIRE(a->n_per_sample >= 1, "n_per_sample must be >= 1");
  REQUIRE((int64_t)a->batch * a->n_per_sample < ((int64_t)1 << 40), "problem too large");
  REQUIRE(a->v && a->z, "v and z are required");
  REQUIRE(aligned16(a->v) && aligned16(a->z) && (!a->z_model || aligned16(a->z_model)),
          "v, z and z_model must be 16-byte aligned");
  REQUIRE(isfinite(a->t_cur) && isfinite(a->t_next) && isfinite(a->guidance), "t_cur, t_next and guidance must be finite");
  const int copies = a->z_model ? a->copies : 0;
  REQUIRE(!a->z_model || copies == 1 || copies == 2, "copies must be 1 or 2 (got %d)", a->copies);
  REQUIRE(!a->t_model || a->t_model_n >= 1, "t_model_n must be >= 1");
  const int64_t zb = (int64_t)a->batch * a->n_per_sample * 4;
  const int64_t vb = zb * (a->cfg ? 2 : 1);
  REQUIRE(!ranges_overlap(a->z, zb, a->v, vb), "z must not overlap v");
  if (a->z_model) {
    const int64_t mb = zb * copies;
    REQUIRE(!ranges_overlap(a->z_model, mb, a->v, vb), "z_model must not overlap v");
    REQUIRE(!ranges_overlap(a->z_model, mb, a->z, zb), "z_model must not overlap z");
  }
  if (a->t_model) {
    const int64_t tb = (int64_t)a->t_model_n * 4;
    REQUIRE(!ranges_overlap(a->t_model, tb, a->v, vb) && !ranges_overlap(a->t_model, tb, a->z, zb),
            "t_model must not overlap v or z");
  }
  // dt is the fp32 difference, as on the device side of the reading
  const float dt = a->t_cur - a->t_next;
  FLUX_HIP(launch_euler_step(a->batch, a->n_per_sample, a->v, a->cfg ? 1 : 0, a->guidance, dt, a->z, a->z_model,
                             copies, a->t_next, a->t_model, a->t_model ? a->t_model_n : 0,
                             static_cast<hipStream_t>(stream)),
           "Euler step");
  return FLUX_OK;
}

// -------------------------------- RoPE table --------------------------------
flux_status flux_rope_table(const float* ids, int32_t batch, int32_t seq, const int32_t axes_dim[3], float theta,
                            float* table, void* stream) {
  g_err[0] = 0;
  REQUIRE(ids && table && axes_dim, "ids, table and axes_dim are required");
  REQUIRE(aligned16(table), "table must be 16-byte aligned");
  REQUIRE(batch >= 1 && seq >= 1, "batch and seq must be >= 1");
  for (int i = 0; i < 3; ++i) REQUIRE(axes_dim[i] >= 0 && axes_dim[i] % 2 == 0, "axes_dim must be even and >= 0");
  REQUIRE(axes_dim[0] + axes_dim[1] + axes_dim[2] >= 2, "axes_dim sum must be >= 2");
  REQUIRE(theta > 0.f && isfinite(theta), "theta must be positive");
  FLUX_HIP(launch_rope_table(ids, batch, seq, axes_dim, theta, table, static_cast<hipStream_t>(stream)),
           "RoPE table");
  return FLUX_OK;
}

flux_status flux_timestep_embed(const float* t, int32_t batch, int32_t dim, float time_factor, float* out,
                                void* stream) {
  g_err[0] = 0;
  REQUIRE(t && out, "t and out are required");
  REQUIRE(batch >= 1 && batch <= (1 << 20), "batch must be in [1, 2^20]");
  REQUIRE(dim >= 2 && dim % 2 == 0 && dim <= 4096, "dim must be even, in [2, 4096]");
  REQUIRE(isfinite(time_factor), "time_factor must be finite");
  FLUX_HIP(launch_timestep_embed(t, batch, dim, time_factor, 10000.f, out, static_cast<hipStream_t>(stream)),
           "timestep sinusoid");
  return FLUX_OK;
}

// -------------------------------- embeddings --------------------------------
size_t flux_embed_workspace_bytes(int32_t precision, int32_t batch, int32_t channels, int32_t height, int32_t width,
                                  int32_t hidden) {
  if (batch < 1 || channels < 1 || height < 1 || width < 1 || hidden < 1) return 0;
  Carve c(nullptr);
  c.take((size_t)batch * height * width * channels * esize(precision));   // patchified latents
  c.take((size_t)batch * 256 * 4);                                         // sinusoid, time_dim <= 256
  c.take((size_t)batch * hidden * 4 * 2);                                  // two hidden activations
  return (size_t)round_up((int64_t)c.off, 256);
}

flux_status flux_embed_fwd(int32_t precision, int32_t batch, int32_t channels, int32_t height, int32_t width,
                           int32_t l_txt, int32_t ctx_dim, int32_t hidden, int32_t time_dim, int32_t y_dim,
                           const flux_embed_weights* w, const float* z_t, const void* txt, const float* t,
                           const float* y, const float* guidance, float* x_img, int64_t img_bstride, float* x_txt,
                           int64_t txt_bstride, float* vec, void* workspace, size_t workspace_bytes,
                           void* stream) {
  g_err[0] = 0;
  REQUIRE(precision == FLUX_PREC_F32 || precision == FLUX_PREC_BF16, "precision %d unknown", precision);
  REQUIRE(batch >= 1 && channels >= 1 && height >= 1 && width >= 1 && hidden >= 1, "sizes must be >= 1");
  REQUIRE(w && w->img_in_w && w->img_in_b && w->time_in1_w && w->time_in1_b && w->time_in2_w && w->time_in2_b,
          "image and time embedder weights are required");
  REQUIRE(z_t && t && x_img && vec, "z_t, t, x_img and vec are required");
  REQUIRE(time_dim >= 2 && time_dim % 2 == 0 && time_dim <= 256, "time_dim must be even, in [2, 256]");
  const bool bf = precision == FLUX_PREC_BF16;
  const int dt = bf ? kBF16 : kF32, es = esize(precision);
  const int kq = bf ? 8 : 4;
  if (bf && channels % 64 != 0)
    return fail(FLUX_ERR_UNSUPPORTED, "bf16 image input needs channels %% 64 == 0 (got %d)", channels);
  REQUIRE(hidden % 4 == 0 && hidden % kq == 0 && time_dim % kq == 0, "hidden and time_dim must be multiples of %d",
          kq);
  REQUIRE(hidden <= 4096, "hidden must be <= 4096");
  const int64_t HW = (int64_t)height * width;
  REQUIRE(img_bstride >= HW * hidden && img_bstride % 4 == 0, "img_bstride too small or not a multiple of 4");
  REQUIRE(aligned16(x_img) && aligned16(vec) && aligned16(z_t), "pointers must be 16-byte aligned");
  const bool has_txt = w->txt_in_w != nullptr;
  const bool copy_txt = !has_txt && txt && x_txt;   // text already at the hidden width
  if (has_txt) {
    REQUIRE(w->txt_in_b && txt && x_txt && l_txt >= 1 && ctx_dim >= 1, "txt_in needs txt, x_txt, l_txt and ctx_dim");
    if (bf && ctx_dim % 64 != 0) return fail(FLUX_ERR_UNSUPPORTED, "bf16 txt_in needs ctx_dim %% 64 == 0");
  }
  if (copy_txt)
    REQUIRE(l_txt >= 1 && (ctx_dim == 0 || ctx_dim == hidden), "text without txt_in must be [B, l_txt, hidden]");
  if (has_txt || copy_txt) {
    REQUIRE(txt_bstride >= (int64_t)l_txt * hidden && txt_bstride % 4 == 0, "txt_bstride too small");
    REQUIRE(aligned16(x_txt) && aligned16(txt), "pointers must be 16-byte aligned");
  }
  const bool has_y = w->vector_in1_w != nullptr;
  if (has_y) {
    REQUIRE(w->vector_in1_b && w->vector_in2_w && w->vector_in2_b && y && y_dim >= 1 && y_dim % kq == 0,
            "vector_in needs both layers, y and y_dim (a multiple of %d)", kq);
  }
  const bool has_g = w->guidance_in_w != nullptr;
  if (has_g) REQUIRE(w->guidance_in_b && guidance, "guidance_in needs its bias and the guidance values");
  flux_status s = check_workspace(workspace, workspace_bytes,
                                  flux_embed_workspace_bytes(precision, batch, channels, height, width, hidden));
  if (s != FLUX_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carve c(workspace);
  void* tok = c.take((size_t)batch * HW * channels * es);
  float* emb = static_cast<float*>(c.take((size_t)batch * 256 * 4));
  float* a1 = static_cast<float*>(c.take((size_t)batch * hidden * 4));
  float* a2 = static_cast<float*>(c.take((size_t)batch * hidden * 4));

  // image tokens and (optionally) text tokens: one grouped GEMM into fp32 residual streams
  FLUX_HIP(launch_patchify(z_t, batch, channels, (int)HW, tok, dt, st), "patchify");
  GemmBatch g{};
  g.count = has_txt ? 2 : 1;
  g.p[0] = gemm_problem(tok, rmap(HW * channels, channels, HW), w->img_in_w, w->img_in_b, (int)(batch * HW), hidden,
                        channels, kEpiStoreF32, x_img, rmap(img_bstride, hidden, HW));
  if (has_txt)
    g.p[1] = gemm_problem(txt, rmap((int64_t)l_txt * ctx_dim, ctx_dim, l_txt), w->txt_in_w, w->txt_in_b,
                          batch * l_txt, hidden, ctx_dim, kEpiStoreF32, x_txt, rmap(txt_bstride, hidden, l_txt));
  FLUX_HIP(launch_gemm(g, dt, st), "input projection GEMM");
  if (copy_txt) FLUX_HIP(launch_rows_to_f32(txt, batch, l_txt, hidden, dt, x_txt, txt_bstride, st), "text rows");

  // conditioning vector
  FLUX_HIP(launch_timestep_embed(t, batch, time_dim, 1000.f, 10000.f, emb, st), "timestep sinusoid");
  GemvBatch gv{};
  gv.count = has_y ? 2 : 1;
  gv.p[0] = gemv_problem(w->time_in1_w, w->time_in1_b, hidden, time_dim, emb, time_dim, a1, hidden, 0, 0);
  if (has_y) gv.p[1] = gemv_problem(w->vector_in1_w, w->vector_in1_b, hidden, y_dim, y, y_dim, a2, hidden, 0, 0);
  FLUX_HIP(run_gemv(gv, batch, dt, st), "embedder layer 1");
  GemvBatch g2{};
  g2.count = 1;
  g2.p[0] = gemv_problem(w->time_in2_w, w->time_in2_b, hidden, hidden, a1, hidden, vec, hidden, 1, 0);
  FLUX_HIP(run_gemv(g2, batch, dt, st), "time embedder layer 2");
  if (has_y) {
    g2.p[0] = gemv_problem(w->vector_in2_w, w->vector_in2_b, hidden, hidden, a2, hidden, vec, hidden, 1, 1);
    FLUX_HIP(run_gemv(g2, batch, dt, st), "vector embedder layer 2");
  }
  if (has_g)
    FLUX_HIP(launch_guidance_embed(batch, hidden, guidance, w->guidance_in_w, w->guidance_in_b, dt, vec, st),
             "guidance embedding");
  return FLUX_OK;
}

// -------------------------------- output head --------------------------------
// the output linear's split-K partial sums need up to kGemmMaxSplit fp32
// copies of the [B*H*W, channels] output; channels is at most this many
constexpr int kFinalMaxChannels = 256;

size_t flux_final_workspace_bytes(int32_t precision, int32_t batch, int32_t height, int32_t width, int32_t hidden) {
  if (batch < 1 || height < 1 || width < 1 || hidden < 1) return 0;
  Carve c(nullptr);
  c.take((size_t)batch * 2 * hidden * 4);
  c.take((size_t)batch * height * width * hidden * esize(precision));
  c.take((size_t)kGemmMaxSplit * batch * height * width * kFinalMaxChannels * 4);
  return (size_t)round_up((int64_t)c.off, 256);
}

flux_status flux_final_fwd(int32_t precision, int32_t batch, int32_t channels, int32_t height, int32_t width,
                           int32_t hidden, float eps, const void* mod_w, const void* mod_b, const void* out_w,
                           const void* out_b, const float* x_img, int64_t bstride, const float* vec, float* v_pred,
                           void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  REQUIRE(precision == FLUX_PREC_F32 || precision == FLUX_PREC_BF16, "precision %d unknown", precision);
  REQUIRE(batch >= 1 && channels >= 1 && height >= 1 && width >= 1, "sizes must be >= 1");
  if (hidden % 256 != 0 || hidden > 4096)
    return fail(FLUX_ERR_UNSUPPORTED, "hidden %d unsupported (a multiple of 256, at most 4096)", hidden);
  if (channels % 4 != 0 || channels > kFinalMaxChannels)
    return fail(FLUX_ERR_UNSUPPORTED, "channels must be a multiple of 4, at most %d", kFinalMaxChannels);
  REQUIRE(eps > 0.f, "eps must be positive");
  REQUIRE(mod_w && mod_b && out_w && out_b && x_img && vec && v_pred, "a required pointer is NULL");
  REQUIRE(aligned16(x_img) && aligned16(vec) && aligned16(v_pred), "pointers must be 16-byte aligned");
  const int64_t HW = (int64_t)height * width;
  REQUIRE(bstride >= HW * hidden && bstride % 4 == 0, "bstride too small or not a multiple of 4");
  flux_status s =
      check_workspace(workspace, workspace_bytes, flux_final_workspace_bytes(precision, batch, height, width, hidden));
  if (s != FLUX_OK) return s;
  const int dt = precision == FLUX_PREC_BF16 ? kBF16 : kF32;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carve c(workspace);
  float* mod = static_cast<float*>(c.take((size_t)batch * 2 * hidden * 4));
  void* h = c.take((size_t)batch * HW * hidden * esize(precision));
  float* partials = static_cast<float*>(c.take((size_t)kGemmMaxSplit * batch * HW * kFinalMaxChannels * 4));
  GemvBatch gv{};
  gv.count = 1;
  gv.p[0] = gemv_problem(mod_w, mod_b, 2 * hidden, hidden, vec, hidden, mod, 2 * hidden, 1, 0);
  FLUX_HIP(run_gemv(gv, batch, dt, st), "final modulation GEMV");
  LnArgs la{};
  la.count = 1;
  la.dim = hidden;
  la.eps = eps;
  la.s[0].x = x_img; la.s[0].xmap = rmap(bstride, hidden, HW);
  la.s[0].out = h; la.s[0].omap = rmap(HW * hidden, hidden, HW);
  la.s[0].shift = mod; la.s[0].scale = mod + hidden; la.s[0].mod_bstride = 2 * hidden;
  la.s[0].rows = (int32_t)(batch * HW);
  const int act = dt == kBF16 ? kF16 : kF32;
  FLUX_HIP(launch_ln_mod(la, act, st), "final LayerNorm-modulate");
  // tok[b, l, c] lands at v_pred[b, c, l]: row l -> +l, column c -> +c*HW
  GemmBatch g{};
  g.count = 1;
  g.p[0] = gemm_problem(h, rmap(HW * hidden, hidden, HW), out_w, out_b, (int)(batch * HW), channels, hidden,
                        kEpiStoreF32, v_pred, rmap(channels * HW, 1, HW));
  g.p[0].col_stride0 = HW;
  g.partials = partials;
  FLUX_HIP(launch_gemm(g, act, st), "output GEMM");
  if (debug_checks_on()) {
    const int64_t n = (int64_t)batch * channels * HW;
    FLUX_HIP(debug_check(v_pred, kF32, 1, n, n, -kDbgBig, kDbgBig, FLUX_DBG_NONFINITE_OUTPUT, st), "debug check of v_pred");
  }
  return FLUX_OK;
}

// ------------------------------ weight conversion ------------------------------
flux_status flux_convert_bf16_to_f16(const void* src, void* dst, int64_t n, void* stream) {
  g_err[0] = 0;
  REQUIRE(src && dst, "src and dst are required");
  REQUIRE(aligned16(src) && aligned16(dst), "src and dst must be 16-byte aligned");
  REQUIRE(n >= 1, "n must be >= 1");
  REQUIRE(!overlap(src, dst, n * 2), "src and dst must not overlap");
  FLUX_HIP(launch_convert_bf16_f16(src, dst, n, static_cast<hipStream_t>(stream)), "bf16 -> fp16 conversion");
  return FLUX_OK;
}

// ------------------------------ standalone ops ------------------------------
flux_status flux_linear_fwd(int32_t precision, int32_t m, int32_t n, int32_t k, const void* x, int64_t lda,
                            const void* w, const void* b, float* y, int64_t ldy, void* stream) {
  g_err[0] = 0;
  REQUIRE(precision == FLUX_PREC_F32 || precision == FLUX_PREC_BF16, "precision %d unknown", precision);
  REQUIRE(m >= 1 && n >= 1 && k >= 1, "m, n, k must be >= 1");
  REQUIRE(x && w && y, "x, w and y are required");
  REQUIRE(aligned16(x) && aligned16(w) && aligned16(y) && (!b || aligned16(b)), "pointers must be 16-byte aligned");
  REQUIRE(lda >= k && ldy >= n, "lda >= k and ldy >= n required");
  if (precision == FLUX_PREC_BF16) {
    if (k % 64 != 0) return fail(FLUX_ERR_UNSUPPORTED, "bf16 linear needs k %% 64 == 0 (got %d)", k);
    REQUIRE(lda % 8 == 0, "bf16 lda must be a multiple of 8");
  }
  if (n % 4 != 0) return fail(FLUX_ERR_UNSUPPORTED, "n must be a multiple of 4 (got %d)", n);
  REQUIRE(ldy % 4 == 0, "ldy must be a multiple of 4");
  GemmBatch g{};
  g.count = 1;
  g.p[0] = gemm_problem(x, rmap((int64_t)m * lda, lda, m), w, b, m, n, k, kEpiStoreF32, y, rmap((int64_t)m * ldy, ldy, m));
  FLUX_HIP(launch_gemm(g, precision == FLUX_PREC_BF16 ? kBF16 : kF32, static_cast<hipStream_t>(stream)),
           "linear GEMM");
  return FLUX_OK;
}

// ------------------------------------ fp8 ------------------------------------
size_t flux_fp8_state_bytes(int32_t n_tensors) {
  return n_tensors >= 1 ? (size_t)n_tensors * sizeof(flux_fp8_tensor) : 0;
}

// ---------------------------------- MXFP8 ----------------------------------
size_t flux_mx_scale_bytes(int32_t rows, int32_t k) {
  if (rows < 1 || k < 64 || k % 64 != 0) return 0;
  return mx_scale_bytes(rows, k);
}

flux_status flux_mx_quantize(int32_t src_precision, const void* src, int32_t rows, int32_t k, uint8_t* codes,
                             uint8_t* scales, void* stream) {
  g_err[0] = 0;
  REQUIRE(src_precision == FLUX_PREC_F32 || src_precision == FLUX_PREC_BF16,
          "src_precision must be FLUX_PREC_F32 or FLUX_PREC_BF16 (got %d)", src_precision);
  REQUIRE(rows >= 1 && k >= 64 && k % 64 == 0, "rows must be >= 1 and k a positive multiple of 64");
  REQUIRE((int64_t)rows * k < ((int64_t)1 << 36), "problem too large");
  REQUIRE(src && codes && scales, "src, codes and scales are required");
  REQUIRE(aligned16(src) && aligned16(codes) && aligned16(scales), "pointers must be 16-byte aligned");
  const int64_t sbytes = (int64_t)rows * k * (src_precision == FLUX_PREC_F32 ? 4 : 2);
  REQUIRE(!ranges_overlap(codes, (int64_t)rows * k, src, sbytes) &&
              !ranges_overlap(scales, (int64_t)mx_scale_bytes(rows, k), src, sbytes) &&
              !ranges_overlap(scales, (int64_t)mx_scale_bytes(rows, k), codes, (int64_t)rows * k),
          "codes, scales and src must not overlap");
  FLUX_HIP(launch_mx_quantize(src, src_precision == FLUX_PREC_F32 ? kF32 : kBF16, rows, k, codes, scales,
                              static_cast<hipStream_t>(stream)),
           "MXFP8 quantize");
  return FLUX_OK;
}

flux_status flux_mxfp8_linear_fwd(int32_t m, int32_t n, int32_t k, const uint8_t* x, const uint8_t* x_scales,
                                  const uint8_t* w, const uint8_t* w_scales, const void* b, float* y, int64_t ldy,
                                  void* stream) {
  g_err[0] = 0;
  REQUIRE(m >= 1 && n >= 1 && k >= 1, "m, n, k must be >= 1");
  REQUIRE(x && x_scales && w && w_scales && y, "x, x_scales, w, w_scales and y are required");
  REQUIRE(aligned16(x) && aligned16(w) && aligned16(x_scales) && aligned16(w_scales) && aligned16(y) &&
              (!b || aligned16(b)),
          "pointers must be 16-byte aligned");
  if (k % 128 != 0 || k < 256)
    return fail(FLUX_ERR_UNSUPPORTED, "MXFP8 linear needs k %% 128 == 0 and k >= 256 (got %d)", k);
  if (n % 4 != 0) return fail(FLUX_ERR_UNSUPPORTED, "n must be a multiple of 4 (got %d)", n);
  REQUIRE(ldy >= n && ldy % 4 == 0, "ldy must be >= n and a multiple of 4");
  REQUIRE((int64_t)m * k < ((int64_t)1 << 32) && (int64_t)n * k < ((int64_t)1 << 32),
          "x and w must each span less than 4 GiB");
  GemmBatch g{};
  g.count = 1;
  g.p[0] = gemm_problem(x, rmap((int64_t)m * k, k, m), w, b, m, n, k, kEpiStoreF32, y, rmap((int64_t)m * ldy, ldy, m));
  g.p[0].ldw = k;
  g.p[0].sa = x_scales;
  g.p[0].sb = w_scales;
  FLUX_HIP(launch_gemm(g, kMXFP8, static_cast<hipStream_t>(stream)), "MXFP8 linear GEMM");
  return FLUX_OK;
}

flux_status flux_fp8_block_quantize(int32_t src_precision, const void* src, int32_t rows, int32_t k,
                                    int32_t tile_rows, uint8_t* codes, uint8_t* scales, void* stream) {
  g_err[0] = 0;
  REQUIRE(src_precision == FLUX_PREC_F32 || src_precision == FLUX_PREC_BF16,
          "src_precision must be FLUX_PREC_F32 or FLUX_PREC_BF16 (got %d)", src_precision);
  REQUIRE(tile_rows == 1 || tile_rows == 128, "tile_rows must be 1 (activations) or 128 (weights), got %d",
          tile_rows);
  REQUIRE(rows >= 1 && k >= 128 && k % 128 == 0, "rows must be >= 1 and k a positive multiple of 128");
  REQUIRE((int64_t)rows * k < ((int64_t)1 << 36), "problem too large");
  // one block per 128-row tile along the grid's y dimension (at most 65535)
  REQUIRE((int64_t)(rows + 255) / 256 * 2 <= 65535, "rows must be at most 8388480");
  REQUIRE(src && codes && scales, "src, codes and scales are required");
  REQUIRE(aligned16(src) && aligned16(codes) && aligned16(scales), "pointers must be 16-byte aligned");
  const int64_t sbytes = (int64_t)rows * k * (src_precision == FLUX_PREC_F32 ? 4 : 2);
  const int64_t scb = (int64_t)mx_scale_bytes(rows, k);
  REQUIRE(!ranges_overlap(codes, (int64_t)rows * k, src, sbytes) && !ranges_overlap(scales, scb, src, sbytes) &&
              !ranges_overlap(scales, scb, codes, (int64_t)rows * k),
          "codes, scales and src must not overlap");
  FLUX_HIP(launch_fp8_block_quantize(src, src_precision == FLUX_PREC_F32 ? kF32 : kBF16, rows, k, tile_rows, codes,
                                     scales, static_cast<hipStream_t>(stream)),
           "blockwise fp8 quantize");
  return FLUX_OK;
}

// ---------------------------------- MXFP4 ----------------------------------
size_t flux_mxfp4_scale_bytes(int32_t rows, int32_t k) {
  if (rows < 1 || k < 128 || k % 128 != 0) return 0;
  return mx_scale_bytes(rows, k);
}

flux_status flux_mxfp4_quantize(int32_t src_precision, const void* src, int32_t rows, int32_t k, uint8_t* codes,
                                uint8_t* scales, void* stream) {
  g_err[0] = 0;
  REQUIRE(src_precision == FLUX_PREC_F32 || src_precision == FLUX_PREC_BF16,
          "src_precision must be FLUX_PREC_F32 or FLUX_PREC_BF16 (got %d)", src_precision);
  REQUIRE(rows >= 1 && k >= 128 && k % 128 == 0, "rows must be >= 1 and k a positive multiple of 128");
  REQUIRE((int64_t)rows * k < ((int64_t)1 << 36), "problem too large");
  REQUIRE(src && codes && scales, "src, codes and scales are required");
  REQUIRE(aligned16(src) && aligned16(codes) && aligned16(scales), "pointers must be 16-byte aligned");
  const int64_t sbytes = (int64_t)rows * k * (src_precision == FLUX_PREC_F32 ? 4 : 2);
  const int64_t cbytes = (int64_t)rows * (k / 2), scb = (int64_t)mx_scale_bytes(rows, k);
  REQUIRE(!ranges_overlap(codes, cbytes, src, sbytes) && !ranges_overlap(scales, scb, src, sbytes) &&
              !ranges_overlap(scales, scb, codes, cbytes),
          "codes, scales and src must not overlap");
  FLUX_HIP(launch_mxfp4_quantize(src, src_precision == FLUX_PREC_F32 ? kF32 : kBF16, rows, k, codes, scales,
                                 static_cast<hipStream_t>(stream)),
           "MXFP4 quantize");
  return FLUX_OK;
}

flux_status flux_mxfp4_linear_fwd(int32_t m, int32_t n, int32_t k, const uint8_t* x, const uint8_t* x_scales,
                                  const uint8_t* w, const uint8_t* w_scales, const void* b, float* y, int64_t ldy,
                                  void* stream) {
  g_err[0] = 0;
  REQUIRE(m >= 1 && n >= 1 && k >= 1, "m, n, k must be >= 1");
  REQUIRE(x && x_scales && w && w_scales && y, "x, x_scales, w, w_scales and y are required");
  REQUIRE(aligned16(x) && aligned16(w) && aligned16(x_scales) && aligned16(w_scales) && aligned16(y) &&
              (!b || aligned16(b)),
          "pointers must be 16-byte aligned");
  if (k % 256 != 0 || k < 512)
    return fail(FLUX_ERR_UNSUPPORTED, "MXFP4 linear needs k %% 256 == 0 and k >= 512 (got %d)", k);
  if (n % 4 != 0) return fail(FLUX_ERR_UNSUPPORTED, "n must be a multiple of 4 (got %d)", n);
  REQUIRE(ldy >= n && ldy % 4 == 0, "ldy must be >= n and a multiple of 4");
  REQUIRE((int64_t)m * (k / 2) < ((int64_t)1 << 32) && (int64_t)n * (k / 2) < ((int64_t)1 << 32),
          "x and w must each span less than 4 GiB");
  GemmBatch g{};
  g.count = 1;
  g.p[0] = gemm_problem(x, rmap((int64_t)m * (k / 2), k / 2, m), w, b, m, n, k, kEpiStoreF32, y,
                        rmap((int64_t)m * ldy, ldy, m));
  g.p[0].ldw = k / 2;
  g.p[0].sa = x_scales;
  g.p[0].sb = w_scales;
  FLUX_HIP(launch_gemm(g, kMXFP4, static_cast<hipStream_t>(stream)), "MXFP4 linear GEMM");
  return FLUX_OK;
}

flux_status flux_fp8_quantize_current(int32_t src_precision, const void* src, int64_t n, flux_fp8_tensor* rec,
                                      uint8_t* dst, void* stream) {
  g_err[0] = 0;
  REQUIRE(src_precision == FLUX_PREC_F32 || src_precision == FLUX_PREC_BF16,
          "src_precision must be FLUX_PREC_F32 or FLUX_PREC_BF16 (got %d)", src_precision);
  REQUIRE(n >= 1 && n < ((int64_t)1 << 40), "n must be in [1, 2^40)");
  REQUIRE(src && dst && rec, "src, rec and dst are required");
  REQUIRE(aligned16(src) && aligned16(dst) && aligned16(rec), "pointers must be 16-byte aligned");
  const int64_t sbytes = n * (src_precision == FLUX_PREC_F32 ? 4 : 2);
  REQUIRE(!ranges_overlap(dst, n, src, sbytes), "src and dst must not overlap");
  const int sdt = src_precision == FLUX_PREC_F32 ? kF32 : kBF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  FLUX_HIP(launch_fp8_current_scale(src, sdt, n, rec, st), "fp8 current scale");
  FLUX_HIP(launch_fp8_quantize(src, sdt, n, rec, dst, st), "fp8 quantize");
  return FLUX_OK;
}

flux_status flux_fp8_quantize(int32_t src_precision, const void* src, int64_t n, flux_fp8_tensor* rec, uint8_t* dst,
                              void* stream) {
  g_err[0] = 0;
  REQUIRE(src_precision == FLUX_PREC_F32 || src_precision == FLUX_PREC_BF16,
          "src_precision must be FLUX_PREC_F32 or FLUX_PREC_BF16 (got %d)", src_precision);
  REQUIRE(n >= 1 && n < ((int64_t)1 << 40), "n must be in [1, 2^40)");
  REQUIRE(src && dst && rec, "src, rec and dst are required");
  REQUIRE(aligned16(src) && aligned16(dst) && aligned16(rec), "pointers must be 16-byte aligned");
  const int64_t sbytes = n * (src_precision == FLUX_PREC_F32 ? 4 : 2);
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = reinterpret_cast<const char*>(dst);
  REQUIRE(!(s0 < d0 + n && d0 < s0 + sbytes), "src and dst must not overlap");
  FLUX_HIP(launch_fp8_quantize(src, src_precision == FLUX_PREC_F32 ? kF32 : kBF16, n, rec, dst,
                               static_cast<hipStream_t>(stream)),
           "fp8 quantize");
  return FLUX_OK;
}

flux_status flux_fp8_update(flux_fp8_tensor* recs, int32_t n_tensors, int32_t algo, int32_t margin, void* stream) {
  g_err[0] = 0;
  REQUIRE(recs && aligned16(recs), "recs must be a non-NULL 16-byte aligned pointer");
  REQUIRE(n_tensors >= 1, "n_tensors must be >= 1");
  REQUIRE(algo == 0 || algo == 1, "algo must be 0 (most_recent) or 1 (max)");
  REQUIRE(margin >= 0 && margin <= 32, "margin must be in [0, 32]");
  FLUX_HIP(launch_fp8_update(recs, n_tensors, algo, margin, static_cast<hipStream_t>(stream)), "fp8 scale update");
  return FLUX_OK;
}

flux_status flux_fp8_linear_fwd(int32_t m, int32_t n, int32_t k, const uint8_t* x, int64_t ldx, const uint8_t* w,
                                int64_t ldw, const flux_fp8_tensor* rx, const flux_fp8_tensor* rw, const void* b,
                                float* y, int64_t ldy, void* stream) {
  g_err[0] = 0;
  REQUIRE(m >= 1 && n >= 1 && k >= 1, "m, n, k must be >= 1");
  REQUIRE(x && w && rx && rw && y, "x, w, rx, rw and y are required");
  REQUIRE(aligned16(x) && aligned16(w) && aligned16(y) && aligned16(rx) && aligned16(rw) && (!b || aligned16(b)),
          "pointers must be 16-byte aligned");
  if (k % 64 != 0) return fail(FLUX_ERR_UNSUPPORTED, "fp8 linear needs k %% 64 == 0 (got %d)", k);
  if (n % 4 != 0) return fail(FLUX_ERR_UNSUPPORTED, "n must be a multiple of 4 (got %d)", n);
  REQUIRE(ldx >= k && ldw >= k && ldx % 16 == 0 && ldw % 16 == 0, "ldx, ldw must be >= k and multiples of 16");
  REQUIRE(ldy >= n && ldy % 4 == 0, "ldy must be >= n and a multiple of 4");
  GemmBatch g{};
  g.count = 1;
  g.p[0] = gemm_problem(x, rmap((int64_t)m * ldx, ldx, m), w, b, m, n, k, kEpiStoreF32, y,
                        rmap((int64_t)m * ldy, ldy, m));
  g.p[0].ldw = ldw;
  g.p[0].qa = rx;
  g.p[0].qw = rw;
  FLUX_HIP(launch_gemm(g, kFP8, static_cast<hipStream_t>(stream)), "fp8 linear GEMM");
  return FLUX_OK;
}

size_t flux_attention_workspace_bytes(int32_t precision, int32_t batch, int32_t seq, int32_t heads,
                                      int32_t head_dim) {
  if (batch < 1 || seq < 1 || heads < 1 || head_dim < 1) return 0;
  Carve c(nullptr);
  const int64_t per = (int64_t)batch * heads * seq_pad_of(seq) * head_dim * esize(precision);
  c.take(per);
  c.take(per);
  c.take(per);
  return (size_t)round_up((int64_t)c.off, 256);
}

flux_status flux_attention_fwd(int32_t precision, int32_t batch, int32_t seq, int32_t heads, int32_t head_dim,
                               const void* q, const void* k, const void* v, int64_t ld_in, void* o, int64_t ld_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  REQUIRE(precision == FLUX_PREC_F32 || precision == FLUX_PREC_BF16, "precision %d unknown", precision);
  REQUIRE(batch >= 1 && seq >= 1 && heads >= 1, "batch, seq and heads must be >= 1");
  if (head_dim != 64 && head_dim != 128)
    return fail(FLUX_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", head_dim);
  if (seq_pad_of(seq) * head_dim * 2 >= (int64_t)1 << 31)
    return fail(FLUX_ERR_UNSUPPORTED, "seq %d too long (one head's keys must stay under 2 GiB)", seq);
  REQUIRE(q && k && v && o, "q, k, v and o are required");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o), "pointers must be 16-byte aligned");
  const int64_t D = (int64_t)heads * head_dim;
  REQUIRE(ld_in >= D && ld_out >= D && ld_in % 8 == 0 && ld_out % 8 == 0,
          "row strides must be >= heads*head_dim and multiples of 8");
  flux_status s = check_workspace(workspace, workspace_bytes,
                                  flux_attention_workspace_bytes(precision, batch, seq, heads, head_dim));
  if (s != FLUX_OK) return s;
  const int dt = precision == FLUX_PREC_BF16 ? kBF16 : kF32;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t Lp = seq_pad_of(seq), es = esize(precision);
  Carve c(workspace);
  const int64_t per = (int64_t)batch * heads * Lp * head_dim * es;
  PrepArgs pa{};
  pa.src_q = q; pa.src_k = k; pa.src_v = v;
  pa.src_bstride = (int64_t)seq * ld_in; pa.src_ld = ld_in;
  pa.batch = batch; pa.seq = seq; pa.seq_pad = (int)Lp; pa.heads = heads; pa.head_dim = head_dim; pa.l_img = seq;
  pa.eps = 1e-6f;
  pa.qh = c.take(per); pa.kh = c.take(per); pa.vt = c.take(per);
  FLUX_HIP(launch_prep(pa, dt, st), "attention layout");
  AttnArgs aa{};
  aa.qh = pa.qh; aa.kh = pa.kh; aa.vt = pa.vt;
  aa.out = o; aa.out_bstride = (int64_t)seq * ld_out; aa.out_ld = ld_out;
  aa.batch = batch; aa.seq = seq; aa.seq_pad = (int)Lp; aa.heads = heads; aa.head_dim = head_dim;
  aa.scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
  FLUX_HIP(launch_attention(aa, dt, dt, st), "attention");
  return FLUX_OK;
}

// ---------------------------------- fp8 attention ----------------------------------
size_t flux_attention_fp8_workspace_bytes(int32_t batch, int32_t seq, int32_t heads) {
  if (batch < 1 || seq < 1 || heads < 1) return 0;
  Carve c(nullptr);
  const int64_t n = (int64_t)batch * heads * seq_pad_of(seq) * 128;
  for (int i = 0; i < 3; ++i) c.take(n * 2);
  for (int i = 0; i < 3; ++i) c.take(n);
  return (size_t)round_up((int64_t)c.off, 256);
}

flux_status flux_attention_fp8_fwd(int32_t batch, int32_t seq, int32_t heads, const void* q, const void* k,
                                   const void* v, int64_t ld_in, void* o, int64_t ld_out, flux_fp8_tensor* recs,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  REQUIRE(batch >= 1 && seq >= 1 && heads >= 1, "batch, seq and heads must be >= 1");
  REQUIRE(q && k && v && o && recs, "q, k, v, o and recs are required");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o) && aligned16(recs),
          "pointers must be 16-byte aligned");
  const int64_t D = (int64_t)heads * 128;
  REQUIRE(ld_in >= D && ld_out >= D && ld_in % 8 == 0 && ld_out % 8 == 0,
          "row strides must be >= heads*128 and multiples of 8");
  flux_status s = check_workspace(workspace, workspace_bytes, flux_attention_fp8_workspace_bytes(batch, seq, heads));
  if (s != FLUX_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t Lp = seq_pad_of(seq), n = (int64_t)batch * heads * Lp * 128;
  Carve c(workspace);
  PrepArgs pa{};
  pa.src_q = q; pa.src_k = k; pa.src_v = v;
  pa.src_bstride = (int64_t)seq * ld_in; pa.src_ld = ld_in;
  pa.batch = batch; pa.seq = seq; pa.seq_pad = (int)Lp; pa.heads = heads; pa.head_dim = 128; pa.l_img = seq;
  pa.eps = 1e-6f;
  pa.qh = c.take(n * 2); pa.kh = c.take(n * 2); pa.vt = c.take(n * 2);
  FLUX_HIP(launch_prep(pa, kBF16, st), "attention layout");
  // per-tensor current scaling of Q, K and V (padding rows are zero)
  void* src[3] = {pa.qh, pa.kh, pa.vt};
  uint8_t* codes[3];
  for (int i = 0; i < 3; ++i) {
    codes[i] = static_cast<uint8_t*>(c.take(n));
    FLUX_HIP(launch_fp8_current_scale(src[i], kBF16, n, recs + i, st), "fp8 current scale");
    FLUX_HIP(launch_fp8_quantize(src[i], kBF16, n, recs + i, codes[i], st), "fp8 quantize");
  }
  AttnArgs aa{};
  aa.qh = codes[0]; aa.kh = codes[1]; aa.vt = codes[2];
  aa.sq = recs; aa.sk = recs + 1; aa.sv = recs + 2;
  aa.out = o; aa.out_bstride = (int64_t)seq * ld_out; aa.out_ld = ld_out;
  aa.batch = batch; aa.seq = seq; aa.seq_pad = (int)Lp; aa.heads = heads; aa.head_dim = 128;
  aa.scale_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  FLUX_HIP(launch_attention(aa, kFP8, kBF16, st), "fp8 attention");
  return FLUX_OK;
}

}  // extern "C"
