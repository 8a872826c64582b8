/*
 * libflux -- Flux MMDiT block forward and rectified-flow objective on
 * AMD Instinct MI355X (gfx950).  Plain C ABI.
 *
 * What the library computes is defined by three pages:
 *   "Flux architecture deep dive" (sections Flow matching framework, Model
 *     components, Mathematical formulation, Implementation details),
 *   "Flux model API reference" (FluxConfig key parameters, AdaLN, RMSNorm,
 *     EmbedND, JointSelfAttention, MMDiTLayer, FluxSingleTransformerBlock,
 *     apply_flow_matching_noise, compute_flow_matching_loss), and
 *   "FP8 training for Flux models" (Configuration: E4M3 linears with delayed
 *     scaling) for FLUX_PREC_FP8_E4M3.
 *
 * Conventions common to every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers unless stated otherwise; the
 *    caller allocates and owns every buffer (the library never allocates,
 *    frees or synchronises).  Struct arguments themselves live in host memory
 *    and are read before the call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued on it in order; results are ready when the stream is.
 *  - Token layout is batch-major [B, L, D]; within a projection the feature
 *    index is head * head_dim + d.  The joint sequence is image rows first,
 *    then text rows.
 *  - Element types: with FLUX_PREC_F32 every weight and activation operand is
 *    float.  With FLUX_PREC_BF16 weights and biases are bf16 (raw 16-bit
 *    patterns); attention runs on bf16 q, k, v with fp32 softmax and
 *    accumulation; the block linears multiply fp16 activations by the bf16
 *    weights, converted to fp16 (round toward zero) inside the kernel or once
 *    beforehand (exact for magnitudes in fp16's normal range, error below
 *    2^-24 under it), with fp32 accumulation.  The fp16 activation stores
 *    (LayerNorm-modulate output, attention output, GELU output) round to
 *    nearest even and saturate at +-65504, so a value beyond fp16's range is
 *    clipped rather than turned into infinity; NaN stays NaN.  fp16
 *    activations keep 3 more mantissa bits than bf16 at
 *    the same matrix-core rate, which the max-abs error bound of the block
 *    outputs needs at Flux-12B widths.  With FLUX_PREC_FP8_E4M3 the token-path
 *    linears of the blocks (qkv, proj, fc1, fc2; lin1, lin2) take OCP E4M3FN
 *    operands (bytes) quantized with per-tensor delayed scales (see
 *    flux_fp8_tensor); their biases, the modulation linears and attention
 *    stay bf16.  Residual streams, modulation vectors,
 *    RMSNorm scales, RoPE tables, latents and losses are always float.
 *  - Errors: every argument is validated on the host BEFORE anything is
 *    enqueued.  A failed check returns a non-zero flux_status and enqueues
 *    nothing; flux_last_error() then returns a thread-local message.  A HIP
 *    launch error returns FLUX_ERR_HIP.  Faults inside kernels surface at the
 *    caller's next synchronisation.
 *  - Pointers passed as tensors must be 16-byte aligned; row strides are in
 *    elements.
 */
#ifndef FLUX_H
#define FLUX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLUX_OK = 0,
  FLUX_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, misalignment, aliasing */
  FLUX_ERR_UNSUPPORTED = 2,        /* valid but not implemented (e.g. head_dim not 64/128) */
  FLUX_ERR_WORKSPACE_TOO_SMALL = 3,
  FLUX_ERR_HIP = 4                 /* a HIP runtime call failed */
} flux_status;

typedef enum {
  FLUX_PREC_F32 = 0,
  FLUX_PREC_BF16 = 1,
  FLUX_PREC_FP8_E4M3 = 2          /* block token-path linears in E4M3, everything else as BF16 */
} flux_precision;

/*
 * Delayed-scaling state of one fp8 tensor ("FP8 training for Flux models",
 * Configuration: fp8 "e4m3", recipe "delayed", margin, amax history length
 * 1024, amax compute algorithm "most_recent" or "max").  Caller-allocated
 * device memory; an all-zero record is valid and means scale 1 with an empty
 * history.
 *
 * Quantization of a value v: q = e4m3(fp32(v * scale)), rounded to the nearest
 * E4M3FN value with ties to even, magnitudes above 448 (infinities included)
 * saturated to +-448, NaN kept.  Every kernel that quantizes a tensor raises
 * amax_bits to the largest |v| it saw.  flux_fp8_update then appends that
 * amax to the history, selects the amax (the new entry, or the history
 * maximum), sets scale = fp32(448 / amax) * 2^-margin when that amax is finite
 * and positive (otherwise the scale is kept and FLUX_FP8_NONFINITE is set when
 * the entry was not finite), and clears amax_bits.  The scale a forward uses
 * is therefore derived from the amaxes of earlier forwards.
 */
#define FLUX_FP8_HISTORY 1024
#define FLUX_FP8_SCALE_SET 1u     /* flags: scale holds an updated value (else 1 is used) */
#define FLUX_FP8_NONFINITE 2u     /* flags: a non-finite amax was seen (sticky) */
typedef struct {
  float scale;                    /* multiplier applied before rounding; 1 until FLUX_FP8_SCALE_SET */
  float scale_inv;                /* 1 / scale */
  uint32_t amax_bits;             /* fp32 bit pattern of the amax since the last update */
  uint32_t flags;
  uint32_t hist_len;              /* valid entries of amax_history (<= FLUX_FP8_HISTORY) */
  uint32_t hist_pos;              /* slot the next entry goes to (ring) */
  uint32_t reserved[2];
  float amax_history[FLUX_FP8_HISTORY];
} flux_fp8_tensor;

/* Record slots.  A double-block stream uses 8 consecutive records, a single
 * block 4: the input (X) and the weight (W) of each token-path linear. */
enum {
  FLUX_FP8_QKV_X = 0, FLUX_FP8_QKV_W = 1, FLUX_FP8_PROJ_X = 2, FLUX_FP8_PROJ_W = 3,
  FLUX_FP8_FC1_X = 4, FLUX_FP8_FC1_W = 5, FLUX_FP8_FC2_X = 6, FLUX_FP8_FC2_W = 7,
  FLUX_FP8_STREAM_TENSORS = 8,
  FLUX_FP8_LIN1_X = 0, FLUX_FP8_LIN1_W = 1, FLUX_FP8_LIN2_X = 2, FLUX_FP8_LIN2_W = 3,
  FLUX_FP8_SINGLE_TENSORS = 4
};

/* Shapes of one block call ("Flux model API reference", FluxConfig). */
typedef struct {
  int32_t batch;          /* B >= 1 */
  int32_t l_img;          /* image tokens per sample (H*W of the latent), >= 1 */
  int32_t l_txt;          /* text tokens per sample, >= 0; joint L = l_img + l_txt */
  int32_t hidden;         /* D == heads * head_dim, a multiple of 256, at most 4096 */
  int32_t heads;
  int32_t head_dim;       /* 64 or 128 */
  int32_t mlp_hidden;     /* F (4 * D for Flux), multiple of 64 */
  int32_t axes_dim[3];    /* 3D RoPE widths, even, sum == head_dim; Flux: 16, 56, 56 */
  float theta;            /* RoPE base, 10000 */
  float eps;              /* LayerNorm and RMSNorm epsilon, 1e-6 */
  int32_t precision;      /* flux_precision */
  int32_t weights_f16;    /* FLUX_PREC_BF16 only.  0: the block linears' weights (qkv, proj, fc1,
                             fc2; lin1, lin2) are bf16 and are converted to fp16 inside the GEMM.
                             1: those weights were converted once to fp16 with
                             flux_convert_bf16_to_f16 (biases and modulation weights stay bf16). */
} flux_dims;

/* Weights of one stream of a double block (torch Linear layout W [out, in]).
 * Element type of W and b follows dims.precision; q_norm / k_norm are float. */
typedef struct {
  const void* mod_w;  const void* mod_b;    /* [6D, D], [6D]: shift1|scale1|gate1|shift2|scale2|gate2 */
  const void* qkv_w;  const void* qkv_b;    /* [3D, D], [3D]: rows q|k|v */
  const float* q_norm; const float* k_norm; /* [head_dim] RMSNorm scales, shared by the heads */
  const void* proj_w; const void* proj_b;   /* [D, D], [D] */
  const void* fc1_w;  const void* fc1_b;    /* [F, D], [F] */
  const void* fc2_w;  const void* fc2_b;    /* [D, F], [D] */
  flux_fp8_tensor* fp8;                     /* FLUX_PREC_FP8_E4M3: FLUX_FP8_STREAM_TENSORS records of
                                               this stream, and qkv_w, proj_w, fc1_w, fc2_w are E4M3
                                               bytes quantized (flux_fp8_quantize) with the W records'
                                               current scales; NULL otherwise */
} flux_stream_weights;

/* Weights of a single block, fused parallel form. */
typedef struct {
  const void* mod_w;  const void* mod_b;    /* [3D, D], [3D]: shift|scale|gate */
  const void* lin1_w; const void* lin1_b;   /* [3D+F, D], [3D+F]: rows q|k|v|mlp_in */
  const float* q_norm; const float* k_norm; /* [head_dim] */
  const void* lin2_w; const void* lin2_b;   /* [D, D+F], [D]: input columns attn|gelu(mlp_in) */
  flux_fp8_tensor* fp8;                     /* FLUX_PREC_FP8_E4M3: FLUX_FP8_SINGLE_TENSORS records,
                                               lin1_w / lin2_w are E4M3 bytes; NULL otherwise.  The
                                               attention output and GELU(mlp_in) are one tensor (the
                                               input of lin2) with one scale. */
} flux_single_weights;

/*
 * flux_block_fwd -- one MMDiT double block ("Flux architecture deep dive",
 * Model components / MMDiT layer (double block); "Flux model API reference",
 * MMDiTLayer and JointSelfAttention).
 *
 * Per stream s (image, text): (shift1, scale1, gate1, shift2, scale2, gate2) =
 * Linear_mod,s(SiLU(vec)); h = LayerNorm(x_s)(1 + scale1) + shift1 (no affine,
 * eps); q|k|v = Linear_qkv,s(h); q, k <- RMSNorm over head_dim with the
 * stream's scales.  Joint softmax attention over the image rows followed by
 * the text rows, 3D RoPE applied to q and k, scale 1/sqrt(head_dim), no mask.
 * x_s += gate1 * Linear_proj,s(O_s); x_s += gate2 * fc2_s(GELU(fc1_s(
 * LayerNorm(x_s)(1 + scale2) + shift2))).
 *
 *  img   [B, l_img, D] float, sample b at img + b*img_bstride; updated in place.
 *  txt   [B, l_txt, D] float, sample b at txt + b*txt_bstride; updated in place
 *        (may be NULL when l_txt == 0).  img and txt rows must not overlap.
 *  vec   [B, D] float conditioning vector.
 *  rope  [B, L, head_dim/2, 2] float (cos, sin) per token and pair, image
 *        rows first, as written by flux_rope_table.
 *  workspace  device scratch of at least flux_workspace_bytes(dims, 0) bytes,
 *        256-byte aligned; its content on entry is ignored.  With
 *        FLUX_PREC_BF16 it includes a 64 MB stream-K area (see
 *        flux_gemm_stream_k); calls that run at the same time need workspaces
 *        of their own.
 */
flux_status flux_block_fwd(const flux_dims* dims, const flux_stream_weights* img_w,
                           const flux_stream_weights* txt_w, float* img, int64_t img_bstride,
                           float* txt, int64_t txt_bstride, const float* vec, const float* rope,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * flux_single_fwd -- one single-stream block over the joint sequence
 * ("Flux architecture deep dive", Model components / Flux single block, in the
 * fused parallel form: one adaLN, one linear D -> 3D+F, attention and GELU
 * side by side, one linear D+F -> D, one gated residual).
 *
 * (shift, scale, gate) = Linear_mod(SiLU(vec)); h = LayerNorm(x)(1+scale)+shift;
 * q|k|v|m = Linear1(h); q, k <- RMSNorm, RoPE; O = softmax attention;
 * x += gate * Linear2([O | GELU(m)]).
 *
 *  x     [B, L, D] float (image rows then text rows), sample b at x + b*x_bstride;
 *        updated in place.
 *  vec, rope, workspace as for flux_block_fwd (workspace op 1).
 */
flux_status flux_single_fwd(const flux_dims* dims, const flux_single_weights* w, float* x,
                            int64_t x_bstride, const float* vec, const float* rope,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * flux_single_seq_fwd -- one single-stream block over the joint sequence in
 * the sequential form the architecture page writes out step by step ("Flux
 * architecture deep dive", Model components / Flux single block: adaLN,
 * self-attention, gated residual, then adaLN, MLP, gated residual).
 *
 * (shift1, scale1, gate1, shift2, scale2, gate2) = Linear_mod(SiLU(vec));
 * h = LayerNorm(x)(1 + scale1) + shift1; q|k|v = Linear_qkv(h); q, k <- RMSNorm
 * over head_dim, RoPE; O = softmax attention over all L = l_img + l_txt rows;
 * x += gate1 * Linear_proj(O); x += gate2 * fc2(GELU(fc1(LayerNorm(x)(1 +
 * scale2) + shift2))).  This is the double block's per-stream computation
 * with the whole joint sequence as its one stream, and it runs the same
 * kernels.
 *
 *  w     one stream's weights (flux_stream_weights: mod [6D, D], qkv [3D, D],
 *        q/k norms, proj, fc1, fc2; fp8: FLUX_FP8_STREAM_TENSORS records).
 *  x     [B, L, D] float (image rows then text rows), sample b at
 *        x + b*x_bstride; updated in place.
 *  vec, rope as for flux_block_fwd; workspace of at least
 *        flux_workspace_bytes(dims, 2) bytes.
 * Errors as for flux_block_fwd.
 */
flux_status flux_single_seq_fwd(const flux_dims* dims, const flux_stream_weights* w, float* x,
                                int64_t x_bstride, const float* vec, const float* rope,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * rf_noise_loss -- rectified-flow noising and velocity MSE ("Flux architecture
 * deep dive", Flow matching framework and Mathematical formulation / Flow
 * matching objective; "Flux model API reference", apply_flow_matching_noise
 * and compute_flow_matching_loss).
 *
 *  z_t = (1 - t_b) z0 + t_b z1, evaluated as two rounded fp32 products and one
 *        rounded sum (so t = 0 and t = 1 reproduce z0 and z1 exactly);
 *  v_target = z1 - z0;
 *  loss = mean over all B*n elements of (v_pred - (z1 - z0))^2, accumulated in
 *        fp64 in a fixed order (bitwise reproducible), stored as float;
 *  loss_per_sample[b] = the same mean over sample b.
 * Outputs that are NULL are skipped; the loss outputs need v_pred.  z_t and
 * v_target must not alias z0, z1 or each other.
 */
typedef struct {
  int32_t batch;              /* B >= 1 */
  int64_t n_per_sample;       /* C*H*W >= 1 */
  const float* z0;            /* [B, n] clean latents */
  const float* z1;            /* [B, n] noise */
  const float* t;             /* [B] flow time in [0, 1] (not checked on the device) */
  float* z_t;                 /* [B, n] out, nullable */
  float* v_target;            /* [B, n] out, nullable */
  const float* v_pred;        /* [B, n] in, nullable (needed for the loss) */
  float* loss;                /* [1] out, nullable */
  float* loss_per_sample;     /* [B] out, nullable */
  void* workspace;            /* >= flux_rf_workspace_bytes(batch, n) bytes when a loss is asked */
  size_t workspace_bytes;
} rf_args;

flux_status rf_noise_loss(const rf_args* args, void* stream);

/*
 * rf_noise_loss_noalloc -- rf_noise_loss for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, results
 * and errors as rf_noise_loss; args->workspace and workspace_bytes are
 * ignored.  The loss partials go to a static 64 KiB device array (8192
 * doubles) that each GPU holds until the process ends; a loss over more than
 * flux_rf_noalloc_max_partials() partials (batch * min(256, ceil(n / 4096)))
 * returns FLUX_ERR_WORKSPACE_TOO_SMALL with nothing enqueued.  The array's
 * device address is looked up on the first call on each device (the device
 * current on the calling thread).  Every call on one GPU shares that array
 * and no clearing is needed (each call writes every partial it reads), so
 * calls that overlap in time on one GPU (different streams, or threads
 * without ordering) race and must be serialised by the caller.  Never calls
 * hipMalloc or hipFree.
 */
flux_status rf_noise_loss_noalloc(const rf_args* args, void* stream);
int64_t flux_rf_noalloc_max_partials(void);

/*
 * flux_euler_step -- one step of the Euler sampler with optional
 * classifier-free guidance ("Flux architecture deep dive", Sampling
 * (inference) / Euler integration and Classifier-free guidance).
 *
 *  g = v_uncond + guidance * (v_cond - v_uncond)   when cfg != 0,
 *  g = v                                           otherwise;
 *  z <- z - (t_cur - t_next) * g.
 * Every operation is one rounded fp32 operation in the order written (d =
 * v_c - v_u; w*d; v_u + w*d; dt = t_cur - t_next; dt*g; z - dt*g), so the
 * result is bit-reproducible.
 *
 *  v        model velocity: [B, n] (cfg == 0) or [2B, n] (cfg != 0: rows
 *           0..B-1 from the conditional, rows B..2B-1 from the unconditional
 *           evaluation of one batched forward).
 *  z        [B, n] current sample, updated in place.
 *  z_model  nullable [copies*B, n]: the next forward's input, z written into
 *           each of its `copies` batch-halves (copies 1 or 2).
 *  t_model  nullable [t_model_n]: the next forward's timesteps, set to t_next.
 * z and z_model must not overlap v or each other.
 */
typedef struct {
  int32_t batch;              /* B >= 1 samples */
  int64_t n_per_sample;       /* C*H*W >= 1 */
  const float* v;
  int32_t cfg;
  float guidance;             /* w */
  float t_cur, t_next;
  float* z;
  float* z_model;
  int32_t copies;
  float* t_model;
  int32_t t_model_n;
} flux_euler_args;

flux_status flux_euler_step(const flux_euler_args* args, void* stream);

/*
 * flux_rope_table -- 3D RoPE angles ("Flux architecture deep dive", 3D RoPE
 * mathematics; "Flux model API reference", EmbedND with rotary_interleaved).
 * For token position ids (p0, p1, p2) and axis a of width d_a (axes in order,
 * contiguous head-dim slices), pair j < d_a/2 turns by p_a * theta^(-2j/d_a);
 * interleaved pairs (2m, 2m+1).  Angles are evaluated in fp64 and stored as
 * float cos/sin.
 *  ids   [B, L, 3] float position ids;  table [B, L, head_dim/2, 2] float out.
 */
flux_status flux_rope_table(const float* ids, int32_t batch, int32_t seq, const int32_t axes_dim[3],
                            float theta, float* table, void* stream);

/*
 * flux_timestep_embed -- sinusoidal encoding of the flow time ("Flux
 * architecture deep dive", Conditioning / Timestep embedding; "Flux model API
 * reference", TimeStepEmbedder): tau = time_factor * t_b (1000 in the model),
 * f_j = 10000^(-j / (dim/2)) for j < dim/2, out[b] = [cos(tau f_j) | sin(tau f_j)],
 * evaluated in fp64 and stored as float.  flux_embed_fwd applies it itself;
 * this call exposes the step alone.
 *  t [batch] float; out [batch, dim] float (dim even, at most 4096).
 */
flux_status flux_timestep_embed(const float* t, int32_t batch, int32_t dim, float time_factor, float* out,
                                void* stream);

/*
 * flux_embed_fwd -- inputs of the transformer ("Flux architecture deep dive",
 * Model components / Input embeddings and Conditioning; Implementation
 * details / Memory layout):
 *   x_img = Linear_img_in(patchify(z_t)), patchify [B,C,H,W] -> [B,H*W,C];
 *   x_txt = Linear_txt_in(txt) if txt_in_w is not NULL; else, when txt and
 *           x_txt are both given, the text is already at the hidden width
 *           (txt [B, l_txt, hidden], ctx_dim 0 or hidden) and x_txt = txt as
 *           float; else x_txt is not written;
 *   vec   = Linear(SiLU(Linear(sinusoid(t)))) [+ Linear(SiLU(Linear(y)))]
 *           [+ Linear_guidance(g)],
 *   sinusoid(t) = [cos(1000 t f_j) | sin(1000 t f_j)], f_j = 1e4^(-j/half),
 *   j < half = time_dim/2.  The guidance term (Conditioning: the optional
 *   guidance scale g through a Linear 1 -> D) is added when guidance_in_w is
 *   not NULL; `guidance` is then [B] float.
 * Element type of the weights and of txt follows `precision`.
 */
typedef struct {
  const void* img_in_w;  const void* img_in_b;     /* [D, C], [D] */
  const void* txt_in_w;  const void* txt_in_b;     /* [D, ctx], [D] or NULL */
  const void* time_in1_w; const void* time_in1_b;  /* [D, time_dim], [D] */
  const void* time_in2_w; const void* time_in2_b;  /* [D, D], [D] */
  const void* vector_in1_w; const void* vector_in1_b;  /* [D, y_dim], [D] or NULL */
  const void* vector_in2_w; const void* vector_in2_b;  /* [D, D], [D] or NULL */
  const void* guidance_in_w; const void* guidance_in_b; /* [D, 1], [D] or NULL */
} flux_embed_weights;

flux_status flux_embed_fwd(int32_t precision, int32_t batch, int32_t channels, int32_t height, int32_t width,
                           int32_t l_txt, int32_t ctx_dim, int32_t hidden, int32_t time_dim, int32_t y_dim,
                           const flux_embed_weights* w, const float* z_t, const void* txt, const float* t,
                           const float* y, const float* guidance, float* x_img, int64_t img_bstride, float* x_txt,
                           int64_t txt_bstride, float* vec, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * flux_final_fwd -- output head ("Flux architecture deep dive", Model
 * components / Output processing): (shift, scale) = Linear_mod(SiLU(vec));
 * tok = Linear_out(LayerNorm(x_img)(1 + scale) + shift) [B, H*W, C];
 * v_pred[b, c, h, w] = tok[b, h*W + w, c].
 *  x_img [B, H*W, D] float, sample b at x_img + b*bstride;  v_pred [B, C, H, W] float out.
 *  channels: a multiple of 4, at most 256 (FLUX_ERR_UNSUPPORTED otherwise).
 *  The workspace also holds the output linear's split-K partial sums, which
 *  are added in a fixed order (results do not depend on the split).
 */
flux_status flux_final_fwd(int32_t precision, int32_t batch, int32_t channels, int32_t height, int32_t width,
                           int32_t hidden, float eps, const void* mod_w, const void* mod_b,
                           const void* out_w, const void* out_b, const float* x_img, int64_t bstride,
                           const float* vec, float* v_pred, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * flux_linear_fwd -- y = x W^T + b, the linear layer used throughout the
 * blocks, exposed on its own ("Flux architecture deep dive", Model components:
 * the q|k|v, projection and MLP linears of the MMDiT layer and the linear1 /
 * linear2 of the single block; weights in the [out, in] layout of a torch
 * Linear).  x [M, K] (row stride lda), W [N, K], b [N] or
 * NULL, all of element type `precision`; y [M, N] float (row stride ldy).
 * K must be a multiple of 64 for bf16.
 */
flux_status flux_linear_fwd(int32_t precision, int32_t m, int32_t n, int32_t k, const void* x, int64_t lda,
                            const void* w, const void* b, float* y, int64_t ldy, void* stream);

/*
 * flux_attention_fwd -- softmax(q k^T / sqrt(head_dim)) v per head, no mask
 * ("Flux architecture deep dive", Implementation details / Attention
 * implementation), exposed on its own (no RMSNorm, no RoPE).
 *  q, k, v [B, L, heads*head_dim] of element type `precision`, row stride ld_in;
 *  o [B, L, heads*head_dim] same type, row stride ld_out.
 *  workspace >= flux_attention_workspace_bytes(...) bytes.
 *  FLUX_ERR_UNSUPPORTED when round_up(seq, 256) * head_dim * 2 bytes (one
 *  head's keys) reach 2 GiB; the block calls apply the same limit to
 *  l_img + l_txt.
 */
flux_status flux_attention_fwd(int32_t precision, int32_t batch, int32_t seq, int32_t heads, int32_t head_dim,
                               const void* q, const void* k, const void* v, int64_t ld_in, void* o,
                               int64_t ld_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * flux_convert_bf16_to_f16 -- dst[i] = fp16(src[i]) for n elements, rounded
 * toward zero, the rule the GEMM applies when it converts bf16 weights itself
 * (exact for magnitudes in [2^-14, 65504]; a weight under 2^-14 keeps an
 * error below 2^-24; finite magnitudes above 65504 saturate to +-65504;
 * infinities and NaN pass through).  For the one-time conversion of static
 * linear weights used with flux_dims.weights_f16 = 1.  src and dst are device
 * pointers, 16-byte aligned, not overlapping.
 */
flux_status flux_convert_bf16_to_f16(const void* src, void* dst, int64_t n, void* stream);

/*
 * FP8 (E4M3) delayed scaling ("FP8 training for Flux models", Configuration).
 *
 * flux_fp8_state_bytes -- bytes of n consecutive flux_fp8_tensor records.
 *
 * flux_fp8_quantize -- dst[i] = e4m3(src[i] * scale(rec)) for n elements and
 *   rec->amax_bits raised to max |src[i]| (the weight cast of a forward).
 *   src_precision FLUX_PREC_F32 (float) or FLUX_PREC_BF16; src, dst 16-byte
 *   aligned, not overlapping; n >= 1.
 *
 * flux_fp8_update -- the update described at flux_fp8_tensor for n
 *   consecutive records; algo 0 = most_recent, 1 = max; 0 <= margin <= 32.
 *   Run it after a forward, on the same stream.
 *
 * flux_fp8_quantize_current -- the current ("tensorwise") scaling recipe the
 *   page lists beside delayed scaling: rec->amax_bits = max |src| of this
 *   tensor, then, when that amax is finite and positive, rec->scale =
 *   fp32(448 / amax), rec->scale_inv = 1 / scale and FLUX_FP8_SCALE_SET (a
 *   non-finite amax keeps the scale and sets FLUX_FP8_NONFINITE); then dst as
 *   flux_fp8_quantize with that scale.  The history is not touched.
 *
 * flux_fp8_linear_fwd -- y = (x_q w_q^T) * scale_inv(rx) * scale_inv(rw) + b:
 *   x_q [M, K] E4M3 bytes (row stride ldx), w_q [N, K] E4M3 bytes (row stride
 *   ldw), quantized with the records rx and rw; b [N] bf16 or NULL; y [M, N]
 *   float (row stride ldy).  K a multiple of 64, N a multiple of 4.
 */
size_t flux_fp8_state_bytes(int32_t n_tensors);
flux_status flux_fp8_quantize(int32_t src_precision, const void* src, int64_t n, flux_fp8_tensor* rec,
                              uint8_t* dst, void* stream);
flux_status flux_fp8_quantize_current(int32_t src_precision, const void* src, int64_t n, flux_fp8_tensor* rec,
                                      uint8_t* dst, void* stream);
flux_status flux_fp8_update(flux_fp8_tensor* recs, int32_t n_tensors, int32_t algo, int32_t margin,
                            void* stream);
flux_status flux_fp8_linear_fwd(int32_t m, int32_t n, int32_t k, const uint8_t* x, int64_t ldx,
                                const uint8_t* w, int64_t ldw, const flux_fp8_tensor* rx,
                                const flux_fp8_tensor* rw, const void* b, float* y, int64_t ldy,
                                void* stream);

/*
 * MXFP8 linears (the "mxfp8" recipe named in "FP8 training for Flux models",
 * Configuration; block-scaled E4M3 in the OCP MX v1.0 format): each 32
 * consecutive values along K share one power-of-two scale stored as an E8M0
 * byte, applied inside gfx950's scaled fp8 MFMA.
 *
 * flux_mx_scale_bytes -- bytes of the scale array of a [rows, k] operand:
 *   rows rounded up to a multiple of 256, times k / 32.
 *
 * flux_mx_quantize -- codes [rows, k] (row-major E4M3 bytes) and scales of
 *   src [rows, k] (FLUX_PREC_F32 float or FLUX_PREC_BF16, row-major): block
 *   exponent X = floor(log2 max|v|) - 8 clamped to [-127, 127] (-127 for an
 *   all-zero block), scale byte X + 127 (0xFF, the E8M0 NaN, for a block
 *   holding a non-finite value, whose elements are then encoded unscaled),
 *   code = e4m3(v * 2^-X) rounded to nearest even with saturation to +-448.
 *   The scale array has the layout the GEMM reads: the byte of (row, block
 *   kb) is at (((row/128)*(k/64) + kb/2)*2 + kb%2)*128 + (row%32)*4 + (row/32)%4,
 *   pad rows get the all-zero block's byte.  k a multiple of 64; pointers
 *   16-byte aligned; codes and scales must not overlap src.
 *
 * flux_mxfp8_linear_fwd -- y = sum over K blocks of 2^(X_x + X_w) (x_q w_q^T)
 *   + b: x [M, K] and w [N, K] as written by flux_mx_quantize (row stride K),
 *   b [N] bf16 or NULL, y [M, N] float (row stride ldy).  K a multiple of 128
 *   and at least 256, N a multiple of 4.
 */
size_t flux_mx_scale_bytes(int32_t rows, int32_t k);
flux_status flux_mx_quantize(int32_t src_precision, const void* src, int32_t rows, int32_t k, uint8_t* codes,
                             uint8_t* scales, void* stream);
flux_status flux_mxfp8_linear_fwd(int32_t m, int32_t n, int32_t k, const uint8_t* x, const uint8_t* x_scales,
                                  const uint8_t* w, const uint8_t* w_scales, const void* b, float* y, int64_t ldy,
                                  void* stream);

/*
 * Blockwise E4M3 (the "blockwise" recipe listed in "FP8 training for Flux
 * models", Configuration, which the page does not define; read here as one
 * power-of-two scale per tile along K).
 *
 * flux_fp8_block_quantize -- codes [rows, k] (row-major E4M3 bytes) and scales
 *   of src [rows, k] (FLUX_PREC_F32 float or FLUX_PREC_BF16, row-major) in
 *   tiles of tile_rows x 128 values (tile_rows 1 for activations, 128 for
 *   weights; the last row tile of a ragged row count holds the rows that
 *   exist).  A tile's exponent e is the largest integer with
 *   amax * 2^e <= 448, clamped to [-127, 127] (0 for an all-zero tile);
 *   code = e4m3(v * 2^e) rounded to nearest even.  The scale array
 *   (flux_mx_scale_bytes(rows, k) bytes) holds the E8M0 byte 127 - e of each
 *   tile, repeated for its four 32-value blocks, in the layout of
 *   flux_mx_quantize (0xFF for a tile holding a non-finite value, whose
 *   elements are then encoded unscaled), so flux_mxfp8_linear_fwd computes
 *   y = sum over 128-wide k blocks of 2^-(e_x + e_w) (x_q w_q^T) + b from an
 *   activation quantized with tile_rows 1 and a weight quantized with
 *   tile_rows 128.  k a multiple of 128, rows at most 8388480; pointers 16-byte aligned; codes and
 *   scales must not overlap src.
 */
flux_status flux_fp8_block_quantize(int32_t src_precision, const void* src, int32_t rows, int32_t k,
                                    int32_t tile_rows, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * MXFP4 linears (OCP MX v1.0 with E2M1 elements: the fp4 member of the
 * microscaling family whose fp8 member is the "mxfp8" recipe of "FP8 training
 * for Flux models", Configuration): each 32 consecutive values along K share
 * one E8M0 power-of-two scale, applied inside gfx950's scaled MFMA in its fp4
 * form.
 *
 * flux_mxfp4_scale_bytes -- bytes of the scale array of a [rows, k] operand
 *   (rows rounded up to a multiple of 256, times k / 32); 0 unless rows >= 1
 *   and k is a positive multiple of 128.
 *
 * flux_mxfp4_quantize -- codes [rows, k / 2] (row-major bytes, two E2M1 codes
 *   each, the even-indexed element in the low nibble; code bit 3 is the sign,
 *   bits 2-1 the exponent with bias 1, bit 0 the mantissa) and scales of src
 *   [rows, k] (FLUX_PREC_F32 float or FLUX_PREC_BF16, row-major): block
 *   exponent X = floor(log2 max|v|) - 2 clamped to [-127, 127] (-127 for an
 *   all-zero block), scale byte X + 127 (0xFF for a block holding a
 *   non-finite value, whose elements are then encoded unscaled), code =
 *   e2m1(v * 2^-X) rounded to nearest with ties to the even code and
 *   saturation to +-6.  The scale byte of (row, block kb) is at
 *   ((row/128)*(k/128) + kb/4)*512 + (kb%2)*256 + (row%32)*8 + ((kb%4)/2)*4
 *   + (row/32)%4; pad rows get the all-zero block's byte.  k a multiple of
 *   128; pointers 16-byte aligned; codes and scales must not overlap src.
 *
 * flux_mxfp4_linear_fwd -- y = sum over K blocks of 2^(X_x + X_w) (x_q w_q^T)
 *   + b: x [M, K / 2 bytes] and w [N, K / 2 bytes] as written by
 *   flux_mxfp4_quantize, b [N] bf16 or NULL, y [M, N] float (row stride ldy).
 *   K counts values: a multiple of 256 and at least 512 (else
 *   FLUX_ERR_UNSUPPORTED); N a multiple of 4.
 */
size_t flux_mxfp4_scale_bytes(int32_t rows, int32_t k);
flux_status flux_mxfp4_quantize(int32_t src_precision, const void* src, int32_t rows, int32_t k, uint8_t* codes,
                                uint8_t* scales, void* stream);
flux_status flux_mxfp4_linear_fwd(int32_t m, int32_t n, int32_t k, const uint8_t* x, const uint8_t* x_scales,
                                  const uint8_t* w, const uint8_t* w_scales, const void* b, float* y, int64_t ldy,
                                  void* stream);

/* Workspace sizes (bytes).  op: 0 double block, 1 single block, 2 sequential single block;
 * 0 for invalid dims or op. */
size_t flux_workspace_bytes(const flux_dims* dims, int32_t op);
size_t flux_rf_workspace_bytes(int32_t batch, int64_t n_per_sample);
size_t flux_embed_workspace_bytes(int32_t precision, int32_t batch, int32_t channels, int32_t height,
                                  int32_t width, int32_t hidden);
size_t flux_final_workspace_bytes(int32_t precision, int32_t batch, int32_t height, int32_t width,
                                  int32_t hidden);
size_t flux_attention_workspace_bytes(int32_t precision, int32_t batch, int32_t seq, int32_t heads,
                                      int32_t head_dim);

/*
 * Training: the backward pass of the blocks under the rectified-flow
 * objective ("Flux architecture deep dive", Flow matching framework: the
 * velocity MSE is backpropagated through the network; the gradients follow
 * from the forward definitions of the double and single blocks by the chain
 * rule).  Training runs with precision FLUX_PREC_BF16, weights_f16 = 0 and
 * head_dim 128 (anything else: FLUX_ERR_UNSUPPORTED).  The forward's block
 * linears multiply fp16 activations (LayerNorm-modulate, attention and GELU
 * outputs, saturating at +-65504) by the bf16 weights converted to fp16 per
 * tile, accumulating in fp32, as flux_block_fwd does; the q|k|v projection is
 * rounded to bf16 before the q / k norm.  The backward runs on the bf16 MFMA
 * with bf16 gradient operands (the saved fp16 activations rounded to bf16 for
 * the weight gradients), fp32 accumulation, fp32 residual stream and fp32
 * parameter gradients.
 *
 * A training forward computes the same block output as flux_block_fwd /
 * flux_single_fwd (up to the rounding of its activations) and keeps in
 * `saved` (caller-allocated, 256-byte aligned, flux_train_saved_bytes(dims,
 * op) bytes; op 0 double block, 1 single block) everything its backward
 * reads: the residual before each half, the modulation vectors, the
 * LayerNorm-modulate outputs, the linear outputs before GELU and before each
 * gate, the attention operands, output and per-query log-sum-exp.
 *
 * A backward takes the gradient of the objective with respect to the
 * block's output, in the residual buffers (d_img / d_txt, or dx; same layout
 * and strides as the forward's residual), and overwrites it in place with
 * the gradient with respect to the block's input.  It writes (=) every
 * parameter gradient into the caller's fp32 buffers (same shapes as the
 * weights: W [out, in], b [out], norm scales [head_dim]) and ADDS (+=) the
 * gradient with respect to vec into dvec [B, hidden] (several blocks share
 * one vec).  `saved` must hold the training forward of the same block on the
 * same inputs and weights; workspace: flux_bwd_workspace_bytes(dims, op)
 * bytes, 256-byte aligned.  Sums over tokens run in a fixed order, so the
 * results are bitwise repeatable.  Errors as elsewhere: checked on the host
 * before anything is enqueued.
 */
typedef struct {
  float *mod_w, *mod_b, *qkv_w, *qkv_b, *q_norm, *k_norm, *proj_w, *proj_b, *fc1_w, *fc1_b, *fc2_w, *fc2_b;
} flux_stream_grads;
typedef struct {
  float *mod_w, *mod_b, *lin1_w, *lin1_b, *q_norm, *k_norm, *lin2_w, *lin2_b;
} flux_single_grads;

/* op 2: the sequential single block (flux_single_seq_fwd's one-stream form:
 * weights in a flux_stream_weights, gradients in a flux_stream_grads). */
size_t flux_train_saved_bytes(const flux_dims* dims, int32_t op);
size_t flux_bwd_workspace_bytes(const flux_dims* dims, int32_t op);
flux_status flux_block_fwd_train(const flux_dims* dims, const flux_stream_weights* img_w,
                                 const flux_stream_weights* txt_w, float* img, int64_t img_batch_stride, float* txt,
                                 int64_t txt_batch_stride, const float* vec, const float* rope, void* saved,
                                 size_t saved_bytes, void* stream);
flux_status flux_block_bwd(const flux_dims* dims, const flux_stream_weights* img_w, const flux_stream_weights* txt_w,
                           float* d_img, int64_t img_batch_stride, float* d_txt, int64_t txt_batch_stride,
                           const float* vec, const float* rope, const void* saved, size_t saved_bytes,
                           const flux_stream_grads* img_grads, const flux_stream_grads* txt_grads, float* dvec,
                           void* workspace, size_t workspace_bytes, void* stream);
flux_status flux_single_fwd_train(const flux_dims* dims, const flux_single_weights* w, float* x,
                                  int64_t x_batch_stride, const float* vec, const float* rope, void* saved,
                                  size_t saved_bytes, void* stream);
flux_status flux_single_bwd(const flux_dims* dims, const flux_single_weights* w, float* dx, int64_t x_batch_stride,
                            const float* vec, const float* rope, const void* saved, size_t saved_bytes,
                            const flux_single_grads* grads, float* dvec, void* workspace, size_t workspace_bytes,
                            void* stream);

flux_status flux_single_seq_fwd_train(const flux_dims* dims, const flux_stream_weights* w, float* x,
                                      int64_t x_batch_stride, const float* vec, const float* rope, void* saved,
                                      size_t saved_bytes, void* stream);
flux_status flux_single_seq_bwd(const flux_dims* dims, const flux_stream_weights* w, float* dx,
                                int64_t x_batch_stride, const float* vec, const float* rope, const void* saved,
                                size_t saved_bytes, const flux_stream_grads* grads, float* dvec, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * The rest of a rectified-flow training step (bf16 weights):
 * flux_rf_loss_grad writes dv = 2 (v_pred - (z1 - z0)) / N, the gradient of
 * the velocity MSE over all N = batch * n_per_sample elements, fp32.
 * flux_final_bwd differentiates the output head of flux_final_fwd (its
 * AdaLN modulation and LayerNorm-modulate are recomputed from x_img and vec):
 * it ADDS the image-row input gradient into dx_img (rows like x_img) and the
 * vec gradient into dvec, and writes the fp32 gradients of the head's
 * weights.  flux_embed_bwd writes (=) the fp32 gradients of the image and
 * text input linears and of the time and pooled-vector embedders, given the
 * gradients d_img, d_txt of the embedded token rows and dvec of the
 * conditioning vector; with guidance [B] float (the values the forward's
 * guidance embedding took, or NULL when it had none) it also writes the
 * gradients of that Linear 1 -> D: guidance_in_w[d] = sum_b g_b dvec[b, d],
 * guidance_in_b[d] = sum_b dvec[b, d] (the guidance values themselves are
 * inputs and get no gradient).
 * channels and ctx_dim multiples of 64; workspaces from the *_bytes calls,
 * 256-byte aligned.
 */
typedef struct {
  float *img_in_w, *img_in_b, *txt_in_w, *txt_in_b, *time_in1_w, *time_in1_b, *time_in2_w, *time_in2_b;
  float *vector_in1_w, *vector_in1_b, *vector_in2_w, *vector_in2_b;
  float *guidance_in_w, *guidance_in_b; /* [D] each; used when guidance is given */
} flux_embed_grads;

flux_status flux_rf_loss_grad(int32_t batch, int64_t n_per_sample, const float* v_pred, const float* z0,
                              const float* z1, float* dv, void* stream);
size_t flux_final_bwd_workspace_bytes(int32_t batch, int32_t channels, int32_t height, int32_t width,
                                      int32_t hidden);
flux_status flux_final_bwd(int32_t batch, int32_t channels, int32_t height, int32_t width, int32_t hidden, float eps,
                           const void* mod_w, const void* mod_b, const void* out_w, const float* x_img,
                           int64_t bstride, const float* vec, const float* dv, float* dx_img, float* dvec,
                           float* g_mod_w, float* g_mod_b, float* g_out_w, float* g_out_b, void* workspace,
                           size_t workspace_bytes, void* stream);
size_t flux_embed_bwd_workspace_bytes(int32_t batch, int32_t channels, int32_t height, int32_t width,
                                      int32_t l_txt, int32_t ctx_dim, int32_t hidden);
flux_status flux_embed_bwd(int32_t batch, int32_t channels, int32_t height, int32_t width, int32_t l_txt,
                           int32_t ctx_dim, int32_t hidden, int32_t time_dim, int32_t y_dim,
                           const flux_embed_weights* w, const float* z_t, const void* txt, const float* t,
                           const float* y, const float* guidance, const float* d_img, int64_t img_batch_stride,
                           const float* d_txt, int64_t txt_batch_stride, const float* dvec,
                           const flux_embed_grads* grads,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Softmax attention alone, training form (bf16, head_dim 128, no mask):
 * q, k, v, o, dout bf16 [B, seq, heads*128] token rows (q, k, v with row
 * stride ld; o and dout with row stride ldo).  flux_attention_fwd_train
 * writes o and lse [B, heads, round_up(seq, 256)] fp32 (log2-domain
 * log-sum-exp of the scaled scores per query).  flux_attention_bwd
 * recomputes the probabilities from q, k and lse and writes dq | dk | dv as
 * bf16 [B, seq, 3*heads*128] (dq at column 0, dk at heads*128, dv at
 * 2*heads*128).  Workspace: flux_attention_train_workspace_bytes bytes,
 * 256-byte aligned, for either call.
 */
size_t flux_attention_train_workspace_bytes(int32_t batch, int32_t seq, int32_t heads);
flux_status flux_attention_fwd_train(int32_t batch, int32_t seq, int32_t heads, const void* q, const void* k,
                                     const void* v, int64_t ld, void* o, int64_t ldo, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream);
flux_status flux_attention_bwd(int32_t batch, int32_t seq, int32_t heads, const void* q, const void* k, const void* v,
                               int64_t ld, const void* o, const void* dout, int64_t ldo, const float* lse, void* dqkv,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Softmax attention with E4M3 operands ("FP8 training for Flux models": fp8
 * attention, off by default), head_dim 128: q, k, v bf16 [B, seq, heads*128]
 * token rows (row stride ld_in) are quantized to E4M3 with per-tensor
 * current scaling -- recs[0..2] (Q, K, V; flux_fp8_tensor records) receive
 * amax, scale = fp32(448 / amax) and scale_inv as flux_fp8_quantize_current
 * sets them -- then S = q k^T / sqrt(128) and O = P v run on the fp8 MFMA,
 * with the probabilities P packed to E4M3; o bf16 (row stride ld_out).
 * Workspace: flux_attention_fp8_workspace_bytes bytes, 256-byte aligned.
 */
size_t flux_attention_fp8_workspace_bytes(int32_t batch, int32_t seq, int32_t heads);
flux_status flux_attention_fp8_fwd(int32_t batch, int32_t seq, int32_t heads, const void* q, const void* k,
                                   const void* v, int64_t ld_in, void* o, int64_t ld_out, flux_fp8_tensor* recs,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel timing (diagnostics, off by default).  While enabled, each kernel
 * launch made by the library is bracketed by two hipEvents recorded on that
 * launch's stream.  flux_timing_read waits for the recorded events, writes
 * per kernel class (the first n classes, n <= flux_timing_classes(); any
 * array may be NULL) the summed milliseconds, the launch count and the summed
 * algorithmic work of those launches -- FLOPs (2*M*N*K per GEMM problem,
 * 4*B*H*L*L*head_dim per attention call) for the GEMM and attention classes,
 * bytes that must cross HBM for the other classes -- and forgets them.
 * flux_timing_class_name names a class ("" when out of range).  The hook is
 * process-wide and serialised by a lock.
 */
flux_status flux_timing_enable(int32_t on);
int32_t flux_timing_classes(void);
const char* flux_timing_class_name(int32_t cls);
flux_status flux_timing_read(double* ms, int64_t* launches, double* work, int32_t n);

/*
 * Measurement helpers (diagnostics).
 *
 * flux_timing_flush -- while timing is enabled and `buffer` is not NULL,
 *   every timed launch is preceded, on its stream and outside its events, by
 *   a kernel that overwrites `bytes` of `buffer` (device memory the caller
 *   owns; 16-byte aligned, bytes >= 16; 512 MB evicts the 4 MB L2 of every
 *   XCD and the 256 MB Infinity Cache), so the timed kernel reads its inputs
 *   from HBM.  NULL turns the flush off.  The library keeps the pointer, not
 *   a copy: it must stay valid while set.
 *
 * flux_stream_copy -- dst[0, bytes) = src[0, bytes), device pointers,
 *   16-byte aligned, not overlapping: a streaming copy (16 bytes per lane,
 *   four loads in flight per lane) whose bandwidth is the practical HBM
 *   ceiling the row-wise kernels are compared with.  Timed as the class
 *   "hbm_copy" with 2 * bytes of traffic.
 */
flux_status flux_timing_flush(void* buffer, int64_t bytes);
flux_status flux_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * Device checks, off by default.  Two preconditions are not checked on the
 * device in normal runs: timesteps lie in [0, 1] ("Flux model API
 * reference", Common issues: the timestep range) and the values the model
 * computes are finite.  With checks on -- the environment variable
 * FLUX_DEBUG_CHECKS set to anything but "" or "0" when the library is first
 * used, or flux_debug_checks(1) -- the entry points below enqueue, on the
 * caller's stream after their own work, read-only passes over the named
 * tensors that OR a bit into a status word of the current device:
 *   FLUX_DBG_T_RANGE             rf_noise_loss(_noalloc): a t outside [0, 1] or NaN
 *   FLUX_DBG_NONFINITE_RESIDUAL  flux_block_fwd, flux_single_fwd, flux_single_seq_fwd
 *                                and the training forwards: a non-finite residual
 *                                value after the block
 *   FLUX_DBG_NONFINITE_LOSS      rf_noise_loss(_noalloc): a non-finite v_pred, loss or
 *                                per-sample loss
 *   FLUX_DBG_NONFINITE_OUTPUT    flux_final_fwd: a non-finite velocity
 *   FLUX_DBG_NONFINITE_GRAD      the block backwards: a non-finite input gradient
 * The word persists until cleared; the checks never change a result.  Each
 * check is one extra read of the tensor (about as long as a copy of it).
 *
 * flux_debug_checks -- on = 1 turns the checks on, 0 off, a negative value
 *   leaves the setting; returns the setting before the call (1 on, 0 off).
 * flux_debug_status -- synchronizes the current device, writes its status
 *   word to *status and, when clear != 0, resets it to 0.
 */
#define FLUX_DBG_T_RANGE 1u
#define FLUX_DBG_NONFINITE_RESIDUAL 2u
#define FLUX_DBG_NONFINITE_LOSS 4u
#define FLUX_DBG_NONFINITE_OUTPUT 8u
#define FLUX_DBG_NONFINITE_GRAD 16u
int32_t flux_debug_checks(int32_t on);
flux_status flux_debug_status(uint32_t* status, int32_t clear);

/*
 * Stream-K tail of the block linears (16-bit workloads, off by default).  A
 * persistent GEMM launch covers its 256 x 256 output tiles in rounds of 256
 * (one block per compute unit); when the last round is partial (64 tiles or
 * more), the K range of its tiles is shared out evenly over all 256 blocks
 * instead.  A block that computes only part of a tile's K range writes its
 * fp32 partial sums to the stream-K area of the block workspace and raises a
 * flag; the block that finishes the tile adds them, in a fixed order, before
 * the epilogue, so results are bitwise repeatable (they differ from the
 * whole-tile order only by rounding).  If a partial has not arrived after
 * `spin` polls, the finishing block computes that K range itself, so a launch
 * always completes.
 *
 * flux_gemm_stream_k -- mode 1 on, 0 off, a negative value leaves the
 *   setting; spin > 0 sets the poll limit, 0 restores the default.  Returns
 *   the mode before the call.  Process-wide; meant for tuning and tests.
 *   Off by default: on the 12B block linears the tail split alone would save
 *   at most about 3% of the block time, and the finishing blocks' waits for
 *   the partial sums cost more than that.
 */
int32_t flux_gemm_stream_k(int32_t mode, int32_t spin);

/* Static text for a status code; thread-local detail of the last failure on
 * this thread ("" when none). */
const char* flux_status_string(flux_status s);
const char* flux_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FLUX_H */
