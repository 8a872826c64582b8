// Host-side helpers shared by the C ABI translation units: error text,
// argument checks, workspace carving and GEMM / GEMV problem descriptions.
#pragma once
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/flux.h"
#include "common.h"
#include "kernels.h"

namespace flux {
namespace api {

inline thread_local char g_err[512] = "";

inline flux_status fail(flux_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

inline flux_status hip_fail(hipError_t e, const char* what) {
  return fail(FLUX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define FLUX_HIP(call, what)                  \
  do {                                        \
    hipError_t e_ = (call);                   \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

#define REQUIRE(cond, ...)                                                  \
  do {                                                                      \
    if (!(cond)) return fail(FLUX_ERR_INVALID_ARGUMENT, __VA_ARGS__);       \
  } while (0)

// Device checks (FLUX_DEBUG_CHECKS): whether they are on, and a read-only pass
// that ORs `bit` into the device's status word if any value of `rows` rows of
// `cols` elements (dtype kF32 / kBF16 / kF16, rows `row_stride` elements
// apart) is outside [lo, hi] or NaN.
bool debug_checks_on();
hipError_t debug_check(const void* p, int dt, int64_t rows, int64_t cols, int64_t row_stride, float lo, float hi,
                       uint32_t bit, hipStream_t st);
constexpr float kDbgBig = 3.402823466e38f;   // [-kDbgBig, kDbgBig]: finite

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// bytes of a q/k/v or attention element (bf16 unless fp32)
inline int esize(int prec) { return prec == FLUX_PREC_F32 ? 4 : 2; }
// bytes of a block-linear activation operand: fp32, fp16 (bf16 workloads) or E4M3
inline int act_esize(int prec) { return prec == FLUX_PREC_F32 ? 4 : prec == FLUX_PREC_FP8_E4M3 ? 1 : 2; }
inline int64_t seq_pad_of(int64_t seq) { return round_up(seq, 256); }   // attention: 256 queries per block

// Bump allocator over the caller's workspace (256-byte aligned regions).
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    off = (size_t)round_up((int64_t)off, 256);
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

inline flux_status check_dims(const flux_dims* d) {
  REQUIRE(d, "dims is NULL");
  REQUIRE(d->precision == FLUX_PREC_F32 || d->precision == FLUX_PREC_BF16 || d->precision == FLUX_PREC_FP8_E4M3,
          "precision %d unknown", d->precision);
  REQUIRE(d->batch >= 1, "batch must be >= 1 (got %d)", d->batch);
  REQUIRE(d->l_img >= 1, "l_img must be >= 1 (got %d)", d->l_img);
  REQUIRE(d->l_txt >= 0, "l_txt must be >= 0 (got %d)", d->l_txt);
  REQUIRE(d->heads >= 1 && d->head_dim >= 1, "heads and head_dim must be >= 1");
  REQUIRE((int64_t)d->heads * d->head_dim == d->hidden, "hidden (%d) != heads (%d) * head_dim (%d)", d->hidden,
          d->heads, d->head_dim);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(FLUX_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", d->head_dim);
  if (d->hidden % 256 != 0 || d->hidden > 4096)
    return fail(FLUX_ERR_UNSUPPORTED, "hidden %d unsupported (a multiple of 256, at most 4096)", d->hidden);
  if (d->mlp_hidden < 64 || d->mlp_hidden % 64 != 0)
    return fail(FLUX_ERR_UNSUPPORTED, "mlp_hidden %d unsupported (a positive multiple of 64)", d->mlp_hidden);
  int sum = 0;
  for (int i = 0; i < 3; ++i) {
    REQUIRE(d->axes_dim[i] >= 0 && d->axes_dim[i] % 2 == 0, "axes_dim[%d] = %d must be even and >= 0", i,
            d->axes_dim[i]);
    sum += d->axes_dim[i];
  }
  REQUIRE(sum == d->head_dim, "axes_dim sum %d != head_dim %d", sum, d->head_dim);
  REQUIRE(d->theta > 0.f && isfinite(d->theta), "theta must be positive");
  REQUIRE(d->eps > 0.f && isfinite(d->eps), "eps must be positive");
  REQUIRE(d->weights_f16 == 0 || (d->weights_f16 == 1 && d->precision == FLUX_PREC_BF16),
          "weights_f16 must be 0, or 1 with FLUX_PREC_BF16");
  const int64_t L = (int64_t)d->l_img + d->l_txt;
  if ((L + 255) / 256 * 256 * d->head_dim * 2 >= (int64_t)1 << 31)
    return fail(FLUX_ERR_UNSUPPORTED, "l_img + l_txt = %lld too long (one head's keys must stay under 2 GiB)",
                (long long)L);
  REQUIRE(L * d->batch < (int64_t)1 << 31 && (int64_t)d->batch * L * (3 * d->hidden + d->mlp_hidden) < (int64_t)1 << 40,
          "problem too large");
  return FLUX_OK;
}

// ------------------------------ workspace layouts ------------------------------
struct BlockWs {
  float* mod[2];
  void* h;
  void* big;
  void* o;
  void* qh;
  void* kh;
  void* vt;
  void* sk;   // stream-K partial sums and flags of the persistent GEMM (16-bit workloads)
  size_t bytes;
};

// The stream-K area of a block workspace (kGemmSkBytes) attached to a GEMM batch.
inline void attach_sk(GemmBatch& g, void* sk) {
  g.sk_part = static_cast<float*>(sk);
  g.sk_flag = sk ? reinterpret_cast<int32_t*>(static_cast<char*>(sk) + kGemmSkMaxGrid * kGemmSkSlotFloats * 4)
                 : nullptr;
}

inline BlockWs block_ws(const flux_dims* d, void* base) {
  Carve c(base);
  BlockWs w{};
  const int64_t B = d->batch, L = (int64_t)d->l_img + d->l_txt, D = d->hidden, F = d->mlp_hidden;
  const int64_t Lp = seq_pad_of(L), es = esize(d->precision), aes = act_esize(d->precision);
  w.mod[0] = static_cast<float*>(c.take(B * 6 * D * 4));
  w.mod[1] = static_cast<float*>(c.take(B * 6 * D * 4));
  w.h = c.take(B * L * D * aes);
  w.big = c.take(B * L * (3 * D * es > F * aes ? 3 * D * es : F * aes));   // q|k|v, later GELU(fc1)
  w.o = c.take(B * L * D * aes);
  w.qh = c.take(B * d->heads * Lp * d->head_dim * es);
  w.kh = c.take(B * d->heads * Lp * d->head_dim * es);
  w.vt = c.take(B * d->heads * Lp * d->head_dim * es);
  w.sk = d->precision == FLUX_PREC_BF16 ? c.take(kGemmSkBytes) : nullptr;
  w.bytes = (size_t)round_up((int64_t)c.off, 256);
  return w;
}

struct SingleWs {
  float* mod;
  void* h;
  void* qkv;
  void* cat;
  void* qh;
  void* kh;
  void* vt;
  void* sk;   // stream-K partial sums and flags of the persistent GEMM (16-bit workloads)
  size_t bytes;
};

inline SingleWs single_ws(const flux_dims* d, void* base) {
  Carve c(base);
  SingleWs w{};
  const int64_t B = d->batch, L = (int64_t)d->l_img + d->l_txt, D = d->hidden, F = d->mlp_hidden;
  const int64_t Lp = seq_pad_of(L), es = esize(d->precision), aes = act_esize(d->precision);
  w.mod = static_cast<float*>(c.take(B * 3 * D * 4));
  w.h = c.take(B * L * D * aes);
  w.qkv = c.take(B * L * 3 * D * es);
  w.cat = c.take(B * L * (D + F) * aes);
  w.qh = c.take(B * d->heads * Lp * d->head_dim * es);
  w.kh = c.take(B * d->heads * Lp * d->head_dim * es);
  w.vt = c.take(B * d->heads * Lp * d->head_dim * es);
  w.sk = d->precision == FLUX_PREC_BF16 ? c.take(kGemmSkBytes) : nullptr;
  w.bytes = (size_t)round_up((int64_t)c.off, 256);
  return w;
}

inline flux_status check_workspace(void* ws, size_t have, size_t need) {
  REQUIRE(ws, "workspace is NULL");
  REQUIRE((reinterpret_cast<uintptr_t>(ws) & 255u) == 0, "workspace must be 256-byte aligned");
  if (have < need)
    return fail(FLUX_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", have, need);
  return FLUX_OK;
}

inline RowMap rmap(int64_t bstride, int64_t ld, int64_t seg) { return RowMap{bstride, ld, (int32_t)seg}; }

// ------------------------------ launch helpers ------------------------------
inline hipError_t run_gemv(GemvBatch g, int batch, int dtype, hipStream_t st) {
  for (int b0 = 0; b0 < batch; b0 += 4) {
    GemvBatch c = g;
    c.batch = batch - b0 < 4 ? batch - b0 : 4;
    for (int i = 0; i < c.count; ++i) {
      c.p[i].x += (int64_t)b0 * c.p[i].x_bstride;
      c.p[i].y += (int64_t)b0 * c.p[i].y_bstride;
    }
    hipError_t e = launch_gemv(c, dtype, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

inline GemvProblem gemv_problem(const void* W, const void* b, int N, int K, const float* x, int64_t xbs, float* y,
                         int64_t ybs, int silu, int acc) {
  GemvProblem p{};
  p.W = W; p.bias = b; p.N = N; p.K = K; p.x = x; p.x_bstride = xbs; p.y = y; p.y_bstride = ybs;
  p.act_silu = silu; p.accumulate = acc;
  return p;
}

inline GemmProblem gemm_problem(const void* A, RowMap am, const void* W, const void* bias, int M, int N, int K, int epi,
                         void* out0, RowMap om0) {
  GemmProblem p{};
  p.A = A; p.amap = am; p.W = W; p.ldw = K; p.bias = bias; p.M = M; p.N = N; p.K = K; p.epi = epi;
  p.out0 = out0; p.omap0 = om0; p.col_stride0 = 1;
  p.omap1 = rmap(0, 1, 1);
  return p;
}

inline const char* elem_ptr(const void* p, int64_t elems, int es) { return static_cast<const char*>(p) + elems * es; }
inline char* elem_ptr(void* p, int64_t elems, int es) { return static_cast<char*>(p) + elems * es; }

inline flux_status check_stream_weights(const flux_stream_weights* w, const char* name) {
  REQUIRE(w, "%s weights are NULL", name);
  REQUIRE(w->mod_w && w->mod_b && w->qkv_w && w->qkv_b && w->q_norm && w->k_norm && w->proj_w && w->proj_b &&
              w->fc1_w && w->fc1_b && w->fc2_w && w->fc2_b,
          "%s weights: a pointer is NULL", name);
  const void* ps[] = {w->mod_w, w->mod_b, w->qkv_w, w->qkv_b, w->proj_w, w->proj_b,
                      w->fc1_w, w->fc1_b, w->fc2_w, w->fc2_b, w->q_norm, w->k_norm};
  for (const void* p : ps) REQUIRE(aligned16(p), "%s weights: pointers must be 16-byte aligned", name);
  return FLUX_OK;
}

inline flux_status check_fp8_records(const flux_fp8_tensor* r, const char* name) {
  REQUIRE(r && aligned16(r), "%s: fp8 state records are required (16-byte aligned) with FLUX_PREC_FP8_E4M3", name);
  return FLUX_OK;
}


}  // namespace api
}  // namespace flux
