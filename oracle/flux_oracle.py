"""fp64 reference of the Flux MMDiT forward and the rectified-flow objective.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy float64:
inputs are upcast, no intermediate is rounded.  Tensor layout is batch-major
[B, L, D] with feature index head * head_dim + d inside a projection.

Readings of the pages taken here (each repeated at its function):
  R1 single block = one adaLN (shift, scale, gate), one fused linear
     D -> 3D + F (q|k|v|mlp), attention and GELU in parallel, one fused output
     linear (D + F) -> D, one gated residual.
  R2 joint sequence order is image rows then text rows.
  R3 RoPE rotates interleaved pairs (2m, 2m+1); axis a owns the contiguous
     head-dim slice of width axes_dim[a] in axis order; pair j < d_a/2 of axis
     a turns by p_a * theta^(-2j/d_a).
  R4 QK RMSNorm per token and head over head_dim, eps 1e-6, learnable scale,
     after the qkv bias and before RoPE; separate scales per stream.
  R5 the LayerNorm inside modulate has no affine part, biased variance, eps 1e-6.
  R6 adaLN modulation = one Linear over SiLU(vec); chunks in the order
     shift, scale, gate (, shift_mlp, scale_mlp, gate_mlp); the final
     AdaLNContinuous uses (shift, scale).
  R7 attention scale 1/sqrt(head_dim), no mask, no dropout.
  R8 GELU is the erf form.
  R9 timestep sinusoid of tau = 1000 t, layout [cos | sin], max period 1e4.
  R10 loss = mean over every element; per-sample means are also reported.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "f64", "rf_noise", "rf_noise_f32_order", "rf_loss",
    "timestep_embedding", "silu", "gelu", "linear", "layernorm", "modulate",
    "rmsnorm", "adaln", "rope_angles", "apply_rope", "attention_probs",
    "attention", "double_block", "single_block", "single_block_sequential", "final_layer",
    "conditioning_vector", "patchify", "unpatchify", "flux_forward", "euler_timesteps",
    "cfg_combine", "euler_step", "euler_cfg_step_f32_order", "euler_sample", "flux_sample_cfg",
    "param_count",
]


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- #
# Rectified flow
# ("Flux architecture deep dive", Flow matching framework and Mathematical
#  formulation / Flow matching objective; "Flux model API reference",
#  apply_flow_matching_noise and compute_flow_matching_loss)
# --------------------------------------------------------------------------- #
def _per_sample(t, ndim: int) -> np.ndarray:
    t = f64(t)
    return t.reshape((-1,) + (1,) * (ndim - 1))


def rf_noise(z0, z1, t) -> Tuple[np.ndarray, np.ndarray]:
    """Noisy latent z_t = (1 - t) z0 + t z1 (z0 clean latent, z1 noise, one t
    per sample) and the velocity target v* = z1 - z0."""
    z0, z1 = f64(z0), f64(z1)
    tb = _per_sample(t, z0.ndim)
    return (1.0 - tb) * z0 + tb * z1, z1 - z0


def rf_noise_f32_order(z0, z1, t) -> Tuple[np.ndarray, np.ndarray]:
    """The same two formulas evaluated in float32 in one fixed order: the two
    products (1 - t) * z0 and t * z1 each rounded, then their rounded sum; and
    the rounded difference z1 - z0.  This order keeps z_t(0) == z0 and
    z_t(1) == z1 exactly; it is the reading used for bit-exact comparison."""
    z0 = np.asarray(z0, dtype=np.float32)
    z1 = np.asarray(z1, dtype=np.float32)
    tb = np.asarray(t, dtype=np.float32).reshape((-1,) + (1,) * (z0.ndim - 1))
    one_minus_t = (np.float32(1.0) - tb).astype(np.float32)
    a = (one_minus_t * z0).astype(np.float32)
    b = (tb * z1).astype(np.float32)
    return (a + b).astype(np.float32), (z1 - z0).astype(np.float32)


def rf_loss(v_pred, z0, z1) -> Tuple[float, np.ndarray]:
    """Velocity MSE: mean over all elements of (v_pred - (z1 - z0))^2 and the
    per-sample means (reading R10)."""
    d = f64(v_pred) - (f64(z1) - f64(z0))
    sq = d * d
    per = sq.reshape(sq.shape[0], -1).mean(axis=1)
    return float(sq.mean()), per


# --------------------------------------------------------------------------- #
# Elementwise pieces
# --------------------------------------------------------------------------- #
def silu(x) -> np.ndarray:
    x = f64(x)
    return x / (1.0 + np.exp(-x))


def gelu(x) -> np.ndarray:
    """GELU, erf form (reading R8): x * Phi(x)."""
    x = f64(x)
    return 0.5 * x * (1.0 + _erf(x / np.sqrt(2.0)))


def linear(x, w, b=None) -> np.ndarray:
    """x W^T + b with W in [out, in] layout."""
    y = f64(x) @ f64(w).T
    if b is not None:
        y = y + f64(b)
    return y


def timestep_embedding(t, dim: int = 256, time_factor: float = 1000.0,
                       max_period: float = 10000.0) -> np.ndarray:
    """Sinusoidal encoding of the flow time (reading R9): tau = 1000 t,
    frequencies f_j = max_period^(-j / (dim/2)), j < dim/2, output
    [cos(tau f_j) | sin(tau f_j)]  ("Flux architecture deep dive",
    Conditioning; "Flux model API reference", TimeStepEmbedder)."""
    tau = time_factor * f64(t).reshape(-1)
    half = dim // 2
    freqs = np.exp(-np.log(max_period) * np.arange(half, dtype=np.float64) / half)
    args = tau[:, None] * freqs[None, :]
    return np.concatenate([np.cos(args), np.sin(args)], axis=-1)


def layernorm(x, eps: float) -> np.ndarray:
    """LayerNorm over the last axis, no affine part, biased variance (R5)."""
    x = f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(x, shift, scale, eps: float) -> np.ndarray:
    """LN(x) * (1 + scale) + shift; shift and scale are per sample [B, D] and
    broadcast over tokens ("Flux architecture deep dive", Adaptive layer
    normalization)."""
    return layernorm(x, eps) * (1.0 + f64(scale)[:, None, :]) + f64(shift)[:, None, :]


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis ("Flux model API
    reference", RMSNorm; reading R4)."""
    x = f64(x)
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * f64(gamma)


def adaln(vec, w, b, n_chunks: int) -> Sequence[np.ndarray]:
    """Modulation parameters: Linear(SiLU(vec)) split into n_chunks [B, D]
    pieces, in the order shift, scale, gate, ... (reading R6; "Flux model API
    reference", AdaLN with n_adaln_chunks=6)."""
    m = linear(silu(vec), w, b)
    return np.split(m, n_chunks, axis=-1)


# --------------------------------------------------------------------------- #
# 3D RoPE ("Flux architecture deep dive", Position embeddings and 3D RoPE
# mathematics; "Flux model API reference", EmbedND and rotary_interleaved)
# --------------------------------------------------------------------------- #
def rope_angles(ids, axes_dim: Sequence[int], theta: float) -> np.ndarray:
    """Rotation angle of every head-dim pair: ids [B, L, 3] -> [B, L, Dh/2].

    Axis a contributes d_a/2 pairs with angle p_a * theta^(-2j/d_a),
    j = 0 .. d_a/2 - 1, placed in axis order (reading R3)."""
    ids = f64(ids)
    parts = []
    for a, d in enumerate(axes_dim):
        j = np.arange(d // 2, dtype=np.float64)
        omega = float(theta) ** (-2.0 * j / d)
        parts.append(ids[..., a:a + 1] * omega)
    return np.concatenate(parts, axis=-1)


def apply_rope(x, angles) -> np.ndarray:
    """Rotate interleaved pairs: x [B, L, H, Dh], angles [B, L, Dh/2];
    (u, w) at dims (2m, 2m+1) -> (u cos - w sin, u sin + w cos) in every head."""
    x = f64(x)
    c = np.cos(f64(angles))[:, :, None, :]
    s = np.sin(f64(angles))[:, :, None, :]
    u, w = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = u * c - w * s
    out[..., 1::2] = u * s + w * c
    return out


# --------------------------------------------------------------------------- #
# Attention ("Flux architecture deep dive", Attention implementation and the
# joint attention trick; reading R7)
# --------------------------------------------------------------------------- #
def attention_probs(q, k) -> np.ndarray:
    """softmax over keys of q k^T / sqrt(Dh): q [B, Lq, H, Dh], k [B, Lk, H, Dh]
    -> [B, H, Lq, Lk]."""
    q, k = f64(q), f64(k)
    dh = q.shape[-1]
    s = np.matmul(q.transpose(0, 2, 1, 3), k.transpose(0, 2, 3, 1)) / np.sqrt(dh)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def attention(q, k, v) -> np.ndarray:
    """softmax(q k^T / sqrt(Dh)) v, heads merged back: -> [B, Lq, H * Dh]."""
    a = attention_probs(q, k)
    o = np.matmul(a, f64(v).transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)
    b_, lq, h, dh = o.shape
    return np.ascontiguousarray(o).reshape(b_, lq, h * dh)


def _heads(y: np.ndarray, heads: int) -> np.ndarray:
    b_, l_, d = y.shape
    return y.reshape(b_, l_, heads, d // heads)


# --------------------------------------------------------------------------- #
# Blocks ("Flux architecture deep dive", MMDiT layer (double block) and Flux
# single block; "Flux model API reference", MMDiTLayer, JointSelfAttention,
# FluxSingleTransformerBlock)
# --------------------------------------------------------------------------- #
def _plain_linear(name, x, w, b):
    return linear(x, w, b)


def double_block(x_img, x_txt, vec, angles, w: Dict[str, np.ndarray], heads: int,
                 eps: float = 1e-6, rows: Optional[Dict[str, np.ndarray]] = None,
                 taps: Optional[dict] = None, lin=None):
    """One MMDiT double block.

    Per stream s: (shift1, scale1, gate1, shift2, scale2, gate2) = adaLN(vec);
    h = LN(x_s)(1 + scale1) + shift1; q|k|v = Linear(h); q, k <- RMSNorm.
    Joint: Q, K, V = concatenation over the sequence of the image then text
    rows (R2), RoPE on Q and K with the joint angles, O = softmax attention.
    Split O back; x_s += gate1 * Linear_proj(O_s);
    x_s += gate2 * fc2(GELU(fc1(LN(x_s)(1 + scale2) + shift2))).

    angles: [B, L_img + L_txt, Dh/2] joint RoPE angles (image rows first).
    rows: optional {"img": idx, "txt": idx}; when given only those token rows
    of the outputs are evaluated (keys and values still cover every token) and
    the returned arrays hold just those rows.
    lin: optional hook lin(name, x, W, b) for the token-path linears, named
    "<stream>_qkv", "<stream>_proj", "<stream>_fc1", "<stream>_fc2" (the fp8
    linears plug in here); plain linear() when omitted.
    """
    lin = lin or _plain_linear
    xs = {"img": f64(x_img), "txt": f64(x_txt)}
    l_img = xs["img"].shape[1]
    seg = {"img": slice(0, l_img), "txt": slice(l_img, l_img + xs["txt"].shape[1])}
    sel = rows if rows is not None else {s: np.arange(xs[s].shape[1]) for s in xs}
    D = xs["img"].shape[-1]
    mods, qs, ks, vs = {}, {}, {}, {}
    for s in ("img", "txt"):
        m = adaln(vec, w[s + "_mod.w"], w[s + "_mod.b"], 6)
        mods[s] = m
        h = modulate(xs[s], m[0], m[1], eps)
        qkv = lin(s + "_qkv", h, w[s + "_qkv.w"], w[s + "_qkv.b"])
        q, k, v = qkv[..., :D], qkv[..., D:2 * D], qkv[..., 2 * D:]
        qs[s] = rmsnorm(_heads(q[:, sel[s]], heads), w[s + "_q_norm"], eps)
        ks[s] = rmsnorm(_heads(k, heads), w[s + "_k_norm"], eps)
        vs[s] = _heads(v, heads)
        if taps is not None:
            taps[s + "_mod"] = np.concatenate(m, axis=-1)
            taps[s + "_h1"] = h
    ang = f64(angles)
    k_all = apply_rope(np.concatenate([ks["img"], ks["txt"]], axis=1), ang)
    v_all = np.concatenate([vs["img"], vs["txt"]], axis=1)
    out = {}
    for s in ("img", "txt"):
        q_rot = apply_rope(qs[s], ang[:, seg[s]][:, sel[s]])
        o = attention(q_rot, k_all, v_all)
        if taps is not None:
            taps[s + "_attn"] = o
        m = mods[s]
        x = xs[s][:, sel[s]] + m[2][:, None, :] * lin(s + "_proj", o, w[s + "_proj.w"], w[s + "_proj.b"])
        h2 = modulate(x, m[3], m[4], eps)
        u = gelu(lin(s + "_fc1", h2, w[s + "_fc1.w"], w[s + "_fc1.b"]))
        out[s] = x + m[5][:, None, :] * lin(s + "_fc2", u, w[s + "_fc2.w"], w[s + "_fc2.b"])
    return out["img"], out["txt"]


def single_block(x, vec, angles, w: Dict[str, np.ndarray], heads: int, eps: float = 1e-6,
                 rows: Optional[np.ndarray] = None, taps: Optional[dict] = None, lin=None) -> np.ndarray:
    """One single-stream block in the fused parallel form (reading R1).

    (shift, scale, gate) = adaLN(vec); h = LN(x)(1 + scale) + shift;
    q|k|v|m = Linear1(h) with widths D, D, D, F; q, k <- RMSNorm, RoPE;
    O = attention(q, k, v); x += gate * Linear2([O | GELU(m)]).
    x covers the whole joint sequence (image rows then text rows).
    rows: optional token indices; only those output rows are evaluated.
    lin: optional hook lin(name, x, W, b) for the two token-path linears,
    named "lin1" and "lin2"; plain linear() when omitted.
    """
    lin = lin or _plain_linear
    x = f64(x)
    D = x.shape[-1]
    sel = rows if rows is not None else np.arange(x.shape[1])
    shift, scale, gate = adaln(vec, w["mod.w"], w["mod.b"], 3)
    h = modulate(x, shift, scale, eps)
    y = lin("lin1", h, w["lin1.w"], w["lin1.b"])
    q = rmsnorm(_heads(y[:, sel, :D], heads), w["q_norm"], eps)
    k = rmsnorm(_heads(y[..., D:2 * D], heads), w["k_norm"], eps)
    v = _heads(y[..., 2 * D:3 * D], heads)
    ang = f64(angles)
    o = attention(apply_rope(q, ang[:, sel]), apply_rope(k, ang), v)
    if taps is not None:
        taps["mod"] = np.concatenate([shift, scale, gate], axis=-1)
        taps["h"] = h
        taps["attn"] = o
    cat = np.concatenate([o, gelu(y[:, sel, 3 * D:])], axis=-1)
    return x[:, sel] + gate[:, None, :] * lin("lin2", cat, w["lin2.w"], w["lin2.b"])


def single_block_sequential(x, vec, angles, w: Dict[str, np.ndarray], heads: int, eps: float = 1e-6,
                            rows: Optional[np.ndarray] = None, lin=None) -> np.ndarray:
    """One single-stream block in the sequential form the architecture page
    writes out step by step ("Flux architecture deep dive", Model components /
    Flux single block): the whole joint sequence is one stream with two
    adaLN-modulated sub-blocks, each closed by its own gated residual.

    (shift1, scale1, gate1, shift2, scale2, gate2) = adaLN(vec) (six chunks);
    h = LN(x)(1 + scale1) + shift1; q|k|v = Linear_qkv(h); q, k <- RMSNorm;
    RoPE on q, k; O = softmax attention over every token;
    x <- x + gate1 * Linear_proj(O);
    h2 = LN(x)(1 + scale2) + shift2; x <- x + gate2 * fc2(GELU(fc1(h2))).
    Weights: "mod" [6D, D], "qkv" [3D, D], "q_norm"/"k_norm" [Dh], "proj"
    [D, D], "fc1" [F, D], "fc2" [D, F].  The text rows stay in the output
    (reading S2 of the fused form applies here too: text leaves the sequence
    only after the last block).
    rows: optional token indices; only those output rows are evaluated.
    lin: optional hook lin(name, x, W, b) for the token-path linears, named
    "qkv", "proj", "fc1", "fc2".
    """
    lin = lin or _plain_linear
    x = f64(x)
    D = x.shape[-1]
    sel = rows if rows is not None else np.arange(x.shape[1])
    sh1, sc1, g1, sh2, sc2, g2 = adaln(vec, w["mod.w"], w["mod.b"], 6)
    h = modulate(x, sh1, sc1, eps)
    qkv = lin("qkv", h, w["qkv.w"], w["qkv.b"])
    q = rmsnorm(_heads(qkv[:, sel, :D], heads), w["q_norm"], eps)
    k = rmsnorm(_heads(qkv[..., D:2 * D], heads), w["k_norm"], eps)
    v = _heads(qkv[..., 2 * D:], heads)
    ang = f64(angles)
    o = attention(apply_rope(q, ang[:, sel]), apply_rope(k, ang), v)
    x1 = x[:, sel] + g1[:, None, :] * lin("proj", o, w["proj.w"], w["proj.b"])
    h2 = modulate(x1, sh2, sc2, eps)
    u = gelu(lin("fc1", h2, w["fc1.w"], w["fc1.b"]))
    return x1 + g2[:, None, :] * lin("fc2", u, w["fc2.w"], w["fc2.b"])


# --------------------------------------------------------------------------- #
# Embeddings and output head ("Flux architecture deep dive", Input
# embeddings, Conditioning, Output processing, Implementation details /
# Memory layout)
# --------------------------------------------------------------------------- #
def patchify(z) -> np.ndarray:
    """[B, C, H, W] -> [B, H*W, C] (token index h*W + w)."""
    z = f64(z)
    b_, c, hh, ww = z.shape
    return z.reshape(b_, c, hh * ww).transpose(0, 2, 1)


def unpatchify(tok, hh: int, ww: int) -> np.ndarray:
    """[B, H*W, C] -> [B, C, H, W]."""
    tok = f64(tok)
    b_, l_, c = tok.shape
    return tok.transpose(0, 2, 1).reshape(b_, c, hh, ww)


def conditioning_vector(t, y, w: Dict[str, np.ndarray], model_channels: int = 256,
                        guidance=None) -> np.ndarray:
    """vec = time_in(sinusoid(t)) [+ vector_in(y)] [+ guidance_in(g)], the
    first two embedders being Linear -> SiLU -> Linear.  The guidance scale g
    (one per sample) goes through one Linear 1 -> D ("Flux architecture deep
    dive", Conditioning: the optional guidance scale enters the combined
    vector through a Linear); W "guidance_in.w" [D, 1], b [D]."""
    e = timestep_embedding(t, model_channels)
    vec = linear(silu(linear(e, w["time_in1.w"], w["time_in1.b"])), w["time_in2.w"], w["time_in2.b"])
    if y is not None:
        vec = vec + linear(silu(linear(y, w["vector_in1.w"], w["vector_in1.b"])),
                           w["vector_in2.w"], w["vector_in2.b"])
    if guidance is not None:
        vec = vec + linear(f64(guidance).reshape(-1, 1), w["guidance_in.w"], w["guidance_in.b"])
    return vec


def final_layer(x_img, vec, w: Dict[str, np.ndarray], hh: int, ww: int, eps: float = 1e-6) -> np.ndarray:
    """AdaLNContinuous (shift, scale from Linear(SiLU(vec))), Linear D -> C,
    reshape to the velocity field [B, C, H, W]."""
    shift, scale = adaln(vec, w["final_mod.w"], w["final_mod.b"], 2)
    tok = linear(modulate(x_img, shift, scale, eps), w["final_out.w"], w["final_out.b"])
    return unpatchify(tok, hh, ww)


def flux_forward(z_t, txt, y, t, ids, emb_w: Dict[str, np.ndarray],
                 double_ws: Sequence[Dict[str, np.ndarray]], single_ws: Sequence[Dict[str, np.ndarray]],
                 heads: int, axes_dim: Sequence[int], theta: float, eps: float = 1e-6,
                 model_channels: int = 256, taps: Optional[dict] = None, guidance=None) -> np.ndarray:
    """Whole forward ("Flux architecture deep dive", Data flow / Complete
    forward pass): image tokens = Linear(patchify(z_t)); text tokens =
    Linear(txt) when a txt_in projection exists, else txt as given; vec
    (with the guidance embedding when guidance is given); double blocks;
    concatenation image|text; single blocks (the sequential form when a
    block's weights hold "qkv.w"); image rows -> final layer -> velocity
    [B, C, H, W]."""
    z_t = f64(z_t)
    _, _, hh, ww = z_t.shape
    x_img = linear(patchify(z_t), emb_w["img_in.w"], emb_w["img_in.b"])
    x_txt = linear(txt, emb_w["txt_in.w"], emb_w["txt_in.b"]) if "txt_in.w" in emb_w else f64(txt)
    vec = conditioning_vector(t, y, emb_w, model_channels, guidance)
    angles = rope_angles(ids, axes_dim, theta)
    for w in double_ws:
        x_img, x_txt = double_block(x_img, x_txt, vec, angles, w, heads, eps)
    x = np.concatenate([x_img, x_txt], axis=1)
    for w in single_ws:
        if "qkv.w" in w:
            x = single_block_sequential(x, vec, angles, w, heads, eps)
        else:
            x = single_block(x, vec, angles, w, heads, eps)
    if taps is not None:
        taps["vec"] = vec
        taps["x_final"] = x
    return final_layer(x[:, :x_img.shape[1]], vec, emb_w, hh, ww, eps)


# --------------------------------------------------------------------------- #
# Sampling ("Flux architecture deep dive", Sampling (inference) / Euler
# integration and Classifier-free guidance)
# --------------------------------------------------------------------------- #
def euler_timesteps(n_steps: int) -> np.ndarray:
    """The uniform grid from t = 1 (noise) down to t = 0: n_steps + 1 points
    1 - i / n_steps.  Step i evaluates the velocity at grid point i and moves
    to grid point i + 1 (reading: the page's loop over 1.0, 0.9, ..., 0.0
    names the grid, its last point being where integration ends)."""
    return 1.0 - np.arange(n_steps + 1, dtype=np.float64) / n_steps


def cfg_combine(v_cond, v_uncond, w: float) -> np.ndarray:
    """Classifier-free guidance: v_uncond + w (v_cond - v_uncond)."""
    vc, vu = f64(v_cond), f64(v_uncond)
    return vu + w * (vc - vu)


def euler_step(z, v, t_cur: float, t_next: float) -> np.ndarray:
    """One Euler step of dz/dt = v from t_cur down to t_next:
    z - (t_cur - t_next) v."""
    return f64(z) - (t_cur - t_next) * f64(v)


def euler_cfg_step_f32_order(z, v_cond, v_uncond, w, t_cur, t_next) -> np.ndarray:
    """The CFG combination and the Euler step evaluated in float32 in one fixed
    order, each operation rounded: d = v_c - v_u; g = v_u + w d (product then
    sum); dt = t_cur - t_next; z - dt g (product then difference).  With
    v_uncond None the combination is skipped (g = v_cond).  This order is the
    reading used for the bit-exact comparison."""
    f = np.float32
    z = np.asarray(z, dtype=f)
    vc = np.asarray(v_cond, dtype=f)
    if v_uncond is None:
        g = vc
    else:
        vu = np.asarray(v_uncond, dtype=f)
        d = (vc - vu).astype(f)
        g = (vu + (f(w) * d).astype(f)).astype(f)
    dt = f(f(t_cur) - f(t_next))
    return (z - (dt * g).astype(f)).astype(f)


def euler_sample(z1, n_steps: int, velocity) -> np.ndarray:
    """Integrate from noise z1 at t = 1 to t = 0 with n_steps Euler steps on
    the uniform grid; velocity(z, t) returns the model's velocity at (z, t)."""
    ts = euler_timesteps(n_steps)
    z = f64(z1)
    for i in range(n_steps):
        z = euler_step(z, velocity(z, ts[i]), ts[i], ts[i + 1])
    return z


def flux_sample_cfg(z1, n_steps: int, guidance_w: float, cond: dict, uncond: Optional[dict], ids,
                    emb_w: Dict[str, np.ndarray], double_ws, single_ws, heads: int, axes_dim, theta: float,
                    eps: float = 1e-6, model_channels: int = 256, guidance=None) -> np.ndarray:
    """Euler sampling of the Flux velocity model with classifier-free guidance:
    at each step v = v_uncond + w (v_cond - v_uncond), v_cond from the
    conditioning cond = {"txt", "y"} and v_uncond from the null conditioning
    uncond (None: no guidance, v = v_cond).  guidance: optional [B] values
    for the guidance embedding (passed to both evaluations)."""
    B = f64(z1).shape[0]

    def velocity(z, t):
        tb = np.full(B, t)
        vc = flux_forward(z, cond["txt"], cond.get("y"), tb, ids, emb_w, double_ws, single_ws, heads, axes_dim,
                          theta, eps, model_channels, guidance=guidance)
        if uncond is None:
            return vc
        vu = flux_forward(z, uncond["txt"], uncond.get("y"), tb, ids, emb_w, double_ws, single_ws, heads,
                          axes_dim, theta, eps, model_channels, guidance=guidance)
        return cfg_combine(vc, vu, guidance_w)

    return euler_sample(z1, n_steps, velocity)


# --------------------------------------------------------------------------- #
# Structure
# --------------------------------------------------------------------------- #
def param_count(hidden: int, heads: int, mlp_hidden: int, n_double: int, n_single: int,
                in_channels: int = 64, context_dim: int = 4096, vec_in_dim: int = 768,
                model_channels: int = 256) -> int:
    """Number of parameters of the weight structure the blocks above consume
    (every Linear with a bias; one RMSNorm scale of head_dim for q and for k
    per stream)."""
    D, F, dh = hidden, mlp_hidden, hidden // heads

    def lin(o, i):
        return o * i + o

    stream = lin(6 * D, D) + lin(3 * D, D) + 2 * dh + lin(D, D) + lin(F, D) + lin(D, F)
    double = 2 * stream
    single = lin(3 * D, D) + lin(3 * D + F, D) + 2 * dh + lin(D, D + F)
    embed = (lin(D, in_channels) + lin(D, context_dim) + lin(D, model_channels) + lin(D, D)
             + lin(D, vec_in_dim) + lin(D, D))
    head = lin(2 * D, D) + lin(in_channels, D)
    return embed + n_double * double + n_single * single + head
