"""fp64 reference of the backward pass of the Flux blocks under the
rectified-flow objective.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Flux architecture deep dive" trains the blocks on the flow-matching loss
(Flow matching framework / the training step: noise, predict the velocity,
mean squared error, backpropagate).  The pages print no backward formulas, so
every function below is the chain rule applied to the forward definitions of
flux_oracle (vector-Jacobian products, written out by hand, no automatic
differentiation).  Each *_vjp function takes the forward's inputs and the
gradient of a scalar objective with respect to the forward's output, and
returns the gradients with respect to every input and parameter; forward
intermediates are recomputed from the inputs.

Readings taken here:
  G1 the objective is the mean over every element of (v_pred - (z1 - z0))^2
     (reading R10 of flux_oracle), so dJ/dv_pred = 2 (v_pred - v*) / N with
     N the element count.
  G2 weights enter as the forward uses them; gradients of W [out, in] have the
     same layout, biases [out].  Gradients are sums over batch and tokens.
  G3 the softmax backward uses the plain form dS = P * (dP - rowsum(P * dP)).
Parity status: every function is pinned by central finite differences of the
forward in tests/test_backward_oracle_pins.py.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np
from scipy.special import erf as _erf

from .flux_oracle import (_heads, adaln, apply_rope, attention_probs, double_block, f64, final_layer, gelu, layernorm,
                          linear, modulate, patchify, rf_loss, rf_noise, rmsnorm, rope_angles, silu, single_block,
                          timestep_embedding)

__all__ = [
    "rf_loss_grad", "linear_vjp", "silu_grad", "gelu_grad", "modulate_vjp", "rmsnorm_vjp", "rope_vjp",
    "attention_vjp", "adaln_vjp", "single_block_vjp", "double_block_vjp", "final_layer_vjp", "conditioning_vjp",
    "flux_train_vjp", "single_block_sequential_vjp",
]


def rf_loss_grad(v_pred, z0, z1) -> np.ndarray:
    """dJ/dv_pred of J = mean((v_pred - (z1 - z0))^2) (reading G1)."""
    v_pred = f64(v_pred)
    return 2.0 * (v_pred - (f64(z1) - f64(z0))) / v_pred.size


def linear_vjp(x, w, dy) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """y = x W^T + b: dx = dy W, dW = sum over rows of dy^T x, db = sum of dy."""
    x, w, dy = f64(x), f64(w), f64(dy)
    x2 = x.reshape(-1, x.shape[-1])
    dy2 = dy.reshape(-1, dy.shape[-1])
    return dy @ w, dy2.T @ x2, dy2.sum(axis=0)


def silu_grad(x) -> np.ndarray:
    """d/dx of x sigmoid(x) = sigmoid(x) (1 + x (1 - sigmoid(x)))."""
    x = f64(x)
    s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def gelu_grad(x) -> np.ndarray:
    """d/dx of x Phi(x) = Phi(x) + x phi(x) (erf form)."""
    x = f64(x)
    return 0.5 * (1.0 + _erf(x / np.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)


def modulate_vjp(x, shift, scale, dh, eps: float):
    """h = LN(x)(1 + scale) + shift, shift / scale per sample [B, D]:
    returns (dx, dshift [B, D], dscale [B, D])."""
    x, dh = f64(x), f64(dh)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * rstd
    dxhat = dh * (1.0 + f64(scale)[:, None, :])
    dx = rstd * (dxhat - dxhat.mean(axis=-1, keepdims=True) - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True))
    return dx, dh.sum(axis=1), (dh * xhat).sum(axis=1)


def rmsnorm_vjp(x, gamma, dy, eps: float):
    """y = x / sqrt(mean(x^2) + eps) * gamma over the last axis: returns
    (dx, dgamma) with dgamma summed over every leading axis."""
    x, dy, gamma = f64(x), f64(dy), f64(gamma)
    rstd = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    n = x * rstd
    dn = dy * gamma
    dx = rstd * (dn - n * (dn * n).mean(axis=-1, keepdims=True))
    return dx, (dy * n).reshape(-1, x.shape[-1]).sum(axis=0)


def rope_vjp(dy, angles) -> np.ndarray:
    """The rotation is orthogonal: its transpose turns every pair back by the
    same angle."""
    return apply_rope(dy, -f64(angles))


def attention_vjp(q, k, v, do):
    """O = softmax(q k^T / sqrt(Dh)) v per (batch, head); q, k, v [B, L, H, Dh],
    do [B, Lq, H * Dh].  Returns dq, dk, dv in the layout of q, k, v (G3)."""
    q, k, v = f64(q), f64(k), f64(v)
    b_, lq, h, dh = q.shape
    p = attention_probs(q, k)                                     # [B, H, Lq, Lk]
    dO = f64(do).reshape(b_, lq, h, dh).transpose(0, 2, 1, 3)    # [B, H, Lq, Dh]
    vt = v.transpose(0, 2, 1, 3)                                  # [B, H, Lk, Dh]
    dv = np.matmul(p.transpose(0, 1, 3, 2), dO)
    dp = np.matmul(dO, vt.transpose(0, 1, 3, 2))
    ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
    c = 1.0 / np.sqrt(dh)
    dq = np.matmul(ds, k.transpose(0, 2, 1, 3)) * c
    dk = np.matmul(ds.transpose(0, 1, 3, 2), q.transpose(0, 2, 1, 3)) * c
    back = lambda a: a.transpose(0, 2, 1, 3)
    return back(dq), back(dk), back(dv)


def adaln_vjp(vec, w, dm):
    """m = Linear(SiLU(vec)) (all chunks concatenated, [B, k D]): returns
    (dvec, dW, db)."""
    vec = f64(vec)
    dsv, dW, db = linear_vjp(silu(vec), w, dm)
    return dsv * silu_grad(vec), dW, db


def _cat(chunks):
    return np.concatenate(chunks, axis=-1)


def single_block_vjp(x, vec, angles, w: Dict[str, np.ndarray], heads: int, eps: float, dout):
    """Gradients of the fused single block (flux_oracle.single_block, reading
    R1) for the output gradient dout [B, L, D].  Returns (dx, dvec, grads)
    with grads keyed like w."""
    x, ang = f64(x), f64(angles)
    D = x.shape[-1]
    shift, scale, gate = adaln(vec, w["mod.w"], w["mod.b"], 3)
    h = modulate(x, shift, scale, eps)
    y1 = linear(h, w["lin1.w"], w["lin1.b"])
    qr, kr, v = _heads(y1[..., :D], heads), _heads(y1[..., D:2 * D], heads), _heads(y1[..., 2 * D:3 * D], heads)
    a = y1[..., 3 * D:]
    qn, kn = rmsnorm(qr, w["q_norm"], eps), rmsnorm(kr, w["k_norm"], eps)
    q, k = apply_rope(qn, ang), apply_rope(kn, ang)
    p = attention_probs(q, k)
    o = np.matmul(p, v.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3).reshape(x.shape[0], x.shape[1], D)
    cat = _cat([o, gelu(a)])
    y2 = linear(cat, w["lin2.w"], w["lin2.b"])

    g: Dict[str, np.ndarray] = {}
    dout = f64(dout)
    dgate = (y2 * dout).sum(axis=1)
    dy2 = gate[:, None, :] * dout
    dcat, g["lin2.w"], g["lin2.b"] = linear_vjp(cat, w["lin2.w"], dy2)
    do, du = dcat[..., :D], dcat[..., D:]
    da = du * gelu_grad(a)
    dq, dk, dv = attention_vjp(q, k, v, do)
    dqn, dkn = rope_vjp(dq, ang), rope_vjp(dk, ang)
    dqr, g["q_norm"] = rmsnorm_vjp(qr, w["q_norm"], dqn, eps)
    dkr, g["k_norm"] = rmsnorm_vjp(kr, w["k_norm"], dkn, eps)
    flat = lambda t: t.reshape(t.shape[0], t.shape[1], -1)
    dy1 = _cat([flat(dqr), flat(dkr), flat(dv), da])
    dh, g["lin1.w"], g["lin1.b"] = linear_vjp(h, w["lin1.w"], dy1)
    dx_ln, dshift, dscale = modulate_vjp(x, shift, scale, dh, eps)
    dx = dout + dx_ln
    dvec, g["mod.w"], g["mod.b"] = adaln_vjp(vec, w["mod.w"], _cat([dshift, dscale, dgate]))
    return dx, dvec, g


def double_block_vjp(x_img, x_txt, vec, angles, w: Dict[str, np.ndarray], heads: int, eps: float, d_img, d_txt):
    """Gradients of the MMDiT double block (flux_oracle.double_block) for the
    output gradients d_img [B, L_img, D], d_txt [B, L_txt, D].  Returns
    (dx_img, dx_txt, dvec, grads) with grads keyed like w."""
    xs = {"img": f64(x_img), "txt": f64(x_txt)}
    dout = {"img": f64(d_img), "txt": f64(d_txt)}
    ang = f64(angles)
    l_img = xs["img"].shape[1]
    seg = {"img": slice(0, l_img), "txt": slice(l_img, l_img + xs["txt"].shape[1])}
    D = xs["img"].shape[-1]
    f = {}
    for s in ("img", "txt"):
        m = adaln(vec, w[s + "_mod.w"], w[s + "_mod.b"], 6)
        h1 = modulate(xs[s], m[0], m[1], eps)
        qkv = linear(h1, w[s + "_qkv.w"], w[s + "_qkv.b"])
        qr, kr, v = _heads(qkv[..., :D], heads), _heads(qkv[..., D:2 * D], heads), _heads(qkv[..., 2 * D:], heads)
        f[s] = dict(m=m, h1=h1, qr=qr, kr=kr, v=v,
                    qn=rmsnorm(qr, w[s + "_q_norm"], eps), kn=rmsnorm(kr, w[s + "_k_norm"], eps))
    q = apply_rope(np.concatenate([f["img"]["qn"], f["txt"]["qn"]], axis=1), ang)
    k = apply_rope(np.concatenate([f["img"]["kn"], f["txt"]["kn"]], axis=1), ang)
    v = np.concatenate([f["img"]["v"], f["txt"]["v"]], axis=1)
    p = attention_probs(q, k)
    o = np.matmul(p, v.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3).reshape(q.shape[0], q.shape[1], D)

    g: Dict[str, np.ndarray] = {}
    dx, do_parts, dm = {}, {}, {}
    for s in ("img", "txt"):
        m, os_ = f[s]["m"], o[:, seg[s]]
        y1 = linear(os_, w[s + "_proj.w"], w[s + "_proj.b"])
        x1 = xs[s] + m[2][:, None, :] * y1
        h2 = modulate(x1, m[3], m[4], eps)
        a = linear(h2, w[s + "_fc1.w"], w[s + "_fc1.b"])
        u = gelu(a)
        y2 = linear(u, w[s + "_fc2.w"], w[s + "_fc2.b"])
        d = dout[s]
        dm5 = (y2 * d).sum(axis=1)
        du, g[s + "_fc2.w"], g[s + "_fc2.b"] = linear_vjp(u, w[s + "_fc2.w"], m[5][:, None, :] * d)
        dh2, g[s + "_fc1.w"], g[s + "_fc1.b"] = linear_vjp(h2, w[s + "_fc1.w"], du * gelu_grad(a))
        dx1_ln, dm3, dm4 = modulate_vjp(x1, m[3], m[4], dh2, eps)
        dx1 = d + dx1_ln
        dm2 = (y1 * dx1).sum(axis=1)
        do_parts[s], g[s + "_proj.w"], g[s + "_proj.b"] = linear_vjp(os_, w[s + "_proj.w"], m[2][:, None, :] * dx1)
        dx[s] = dx1
        dm[s] = [None, None, dm2, dm3, dm4, dm5]
    dq, dk, dv = attention_vjp(q, k, v, np.concatenate([do_parts["img"], do_parts["txt"]], axis=1))
    dqn, dkn = rope_vjp(dq, ang), rope_vjp(dk, ang)
    dvec = np.zeros_like(f64(vec))
    flat = lambda t: t.reshape(t.shape[0], t.shape[1], -1)
    for s in ("img", "txt"):
        dqr, g[s + "_q_norm"] = rmsnorm_vjp(f[s]["qr"], w[s + "_q_norm"], dqn[:, seg[s]], eps)
        dkr, g[s + "_k_norm"] = rmsnorm_vjp(f[s]["kr"], w[s + "_k_norm"], dkn[:, seg[s]], eps)
        dqkv = _cat([flat(dqr), flat(dkr), flat(dv[:, seg[s]])])
        dh1, g[s + "_qkv.w"], g[s + "_qkv.b"] = linear_vjp(f[s]["h1"], w[s + "_qkv.w"], dqkv)
        m = f[s]["m"]
        dx_ln, dm[s][0], dm[s][1] = modulate_vjp(xs[s], m[0], m[1], dh1, eps)
        dx[s] = dx[s] + dx_ln
        dv_s, g[s + "_mod.w"], g[s + "_mod.b"] = adaln_vjp(vec, w[s + "_mod.w"], _cat(dm[s]))
        dvec = dvec + dv_s
    return dx["img"], dx["txt"], dvec, g


def final_layer_vjp(x_img, vec, w: Dict[str, np.ndarray], eps: float, dv):
    """Gradients of flux_oracle.final_layer (AdaLNContinuous, Linear D -> C,
    unpatchify) for the velocity gradient dv [B, C, H, W].  unpatchify is a
    permutation, so its transpose is patchify.  Returns (dx_img, dvec, grads)."""
    x_img = f64(x_img)
    shift, scale = adaln(vec, w["final_mod.w"], w["final_mod.b"], 2)
    h = modulate(x_img, shift, scale, eps)
    g: Dict[str, np.ndarray] = {}
    dh, g["final_out.w"], g["final_out.b"] = linear_vjp(h, w["final_out.w"], patchify(dv))
    dx, dsh, dsc = modulate_vjp(x_img, shift, scale, dh, eps)
    dvec, g["final_mod.w"], g["final_mod.b"] = adaln_vjp(vec, w["final_mod.w"], _cat([dsh, dsc]))
    return dx, dvec, g


def conditioning_vjp(t, y, w: Dict[str, np.ndarray], dvec, model_channels: int = 256,
                     guidance=None) -> Dict[str, np.ndarray]:
    """Gradients of the two Linear -> SiLU -> Linear embedders of
    flux_oracle.conditioning_vector (time, and the pooled vector when y is
    given) and, when guidance [B] is given, of its Linear 1 -> D, for the vec
    gradient dvec [B, D]."""
    g: Dict[str, np.ndarray] = {}
    if guidance is not None:
        _, g["guidance_in.w"], g["guidance_in.b"] = linear_vjp(f64(guidance).reshape(-1, 1), w["guidance_in.w"], dvec)
    pairs = [("time_in", timestep_embedding(t, model_channels))]
    if y is not None:
        pairs.append(("vector_in", f64(y)))
    for name, e in pairs:
        a1 = linear(e, w[name + "1.w"], w[name + "1.b"])
        ds1, g[name + "2.w"], g[name + "2.b"] = linear_vjp(silu(a1), w[name + "2.w"], dvec)
        _, g[name + "1.w"], g[name + "1.b"] = linear_vjp(e, w[name + "1.w"], ds1 * silu_grad(a1))
    return g


def flux_train_vjp(z0, z1, t, txt, y, ids, emb_w: Dict[str, np.ndarray], double_ws, single_ws, heads: int,
                   axes_dim, theta: float, eps: float = 1e-6, model_channels: int = 256, guidance=None):
    """One rectified-flow training step of the model of flux_oracle.flux_forward
    (fused single blocks; the guidance embedding when guidance [B] is given,
    the guidance values themselves being inputs): z_t = (1 - t) z0 + t z1, the
    velocity prediction, J = mean((v_pred - (z1 - z0))^2), then the gradient of
    J with respect to every weight.  Returns (J, emb_grads, [double grads],
    [single grads])."""
    z_t, _ = rf_noise(z0, z1, t)
    _, _, hh, ww = z_t.shape
    patches = patchify(z_t)
    x_img = linear(patches, emb_w["img_in.w"], emb_w["img_in.b"])
    has_txt_in = "txt_in.w" in emb_w
    x_txt = linear(txt, emb_w["txt_in.w"], emb_w["txt_in.b"]) if has_txt_in else f64(txt)
    e = timestep_embedding(t, model_channels)
    vec = linear(silu(linear(e, emb_w["time_in1.w"], emb_w["time_in1.b"])), emb_w["time_in2.w"], emb_w["time_in2.b"])
    if y is not None:
        vec = vec + linear(silu(linear(y, emb_w["vector_in1.w"], emb_w["vector_in1.b"])),
                           emb_w["vector_in2.w"], emb_w["vector_in2.b"])
    if guidance is not None:
        vec = vec + linear(f64(guidance).reshape(-1, 1), emb_w["guidance_in.w"], emb_w["guidance_in.b"])
    angles = rope_angles(ids, axes_dim, theta)
    l_img = x_img.shape[1]
    d_in = []
    for w in double_ws:
        d_in.append((x_img, x_txt))
        x_img, x_txt = double_block(x_img, x_txt, vec, angles, w, heads, eps)
    x = np.concatenate([x_img, x_txt], axis=1)
    s_in = []
    for w in single_ws:
        s_in.append(x)
        x = single_block(x, vec, angles, w, heads, eps)
    v_pred = final_layer(x[:, :l_img], vec, emb_w, hh, ww, eps)
    loss, _ = rf_loss(v_pred, z0, z1)

    dv = rf_loss_grad(v_pred, z0, z1)
    dx_img, dvec, g_emb = final_layer_vjp(x[:, :l_img], vec, emb_w, eps, dv)
    dx = np.zeros_like(x)
    dx[:, :l_img] = dx_img
    g_single = [None] * len(single_ws)
    for i in reversed(range(len(single_ws))):
        dx, dv_b, g_single[i] = single_block_vjp(s_in[i], vec, angles, single_ws[i], heads, eps, dx)
        dvec = dvec + dv_b
    d_img, d_txt = dx[:, :l_img], dx[:, l_img:]
    g_double = [None] * len(double_ws)
    for i in reversed(range(len(double_ws))):
        xi, xt = d_in[i]
        d_img, d_txt, dv_b, g_double[i] = double_block_vjp(xi, xt, vec, angles, double_ws[i], heads, eps, d_img, d_txt)
        dvec = dvec + dv_b
    _, g_emb["img_in.w"], g_emb["img_in.b"] = linear_vjp(patches, emb_w["img_in.w"], d_img)
    if has_txt_in:
        _, g_emb["txt_in.w"], g_emb["txt_in.b"] = linear_vjp(txt, emb_w["txt_in.w"], d_txt)
    g_emb.update(conditioning_vjp(t, y, emb_w, dvec, model_channels, guidance))
    return loss, g_emb, g_double, g_single


def single_block_sequential_vjp(x, vec, angles, w: Dict[str, np.ndarray], heads: int, eps: float, dout):
    """Gradients of flux_oracle.single_block_sequential (one stream: two
    adaLN halves with qkv / proj / fc1 / fc2, attention over every token) for
    the output gradient dout [B, L, D].  Returns (dx, dvec, grads) keyed like w."""
    x, ang = f64(x), f64(angles)
    D = x.shape[-1]
    m = adaln(vec, w["mod.w"], w["mod.b"], 6)
    h1 = modulate(x, m[0], m[1], eps)
    qkv = linear(h1, w["qkv.w"], w["qkv.b"])
    qr, kr, v = _heads(qkv[..., :D], heads), _heads(qkv[..., D:2 * D], heads), _heads(qkv[..., 2 * D:], heads)
    q = apply_rope(rmsnorm(qr, w["q_norm"], eps), ang)
    k = apply_rope(rmsnorm(kr, w["k_norm"], eps), ang)
    p = attention_probs(q, k)
    o = np.matmul(p, v.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3).reshape(x.shape[0], x.shape[1], D)
    y1 = linear(o, w["proj.w"], w["proj.b"])
    x1 = x + m[2][:, None, :] * y1
    h2 = modulate(x1, m[3], m[4], eps)
    a = linear(h2, w["fc1.w"], w["fc1.b"])
    u = gelu(a)
    y2 = linear(u, w["fc2.w"], w["fc2.b"])

    g: Dict[str, np.ndarray] = {}
    d = f64(dout)
    dm5 = (y2 * d).sum(axis=1)
    du, g["fc2.w"], g["fc2.b"] = linear_vjp(u, w["fc2.w"], m[5][:, None, :] * d)
    dh2, g["fc1.w"], g["fc1.b"] = linear_vjp(h2, w["fc1.w"], du * gelu_grad(a))
    dx1_ln, dm3, dm4 = modulate_vjp(x1, m[3], m[4], dh2, eps)
    dx1 = d + dx1_ln
    dm2 = (y1 * dx1).sum(axis=1)
    do, g["proj.w"], g["proj.b"] = linear_vjp(o, w["proj.w"], m[2][:, None, :] * dx1)
    dq, dk, dv = attention_vjp(q, k, v, do)
    dqr, g["q_norm"] = rmsnorm_vjp(qr, w["q_norm"], rope_vjp(dq, ang), eps)
    dkr, g["k_norm"] = rmsnorm_vjp(kr, w["k_norm"], rope_vjp(dk, ang), eps)
    flat = lambda t: t.reshape(t.shape[0], t.shape[1], -1)
    dh1, g["qkv.w"], g["qkv.b"] = linear_vjp(h1, w["qkv.w"], _cat([flat(dqr), flat(dkr), flat(dv)]))
    dx_ln, dm0, dm1 = modulate_vjp(x, m[0], m[1], dh1, eps)
    dvec, g["mod.w"], g["mod.b"] = adaln_vjp(vec, w["mod.w"], _cat([dm0, dm1, dm2, dm3, dm4, dm5]))
    return dx1 + dx_ln, dvec, g
