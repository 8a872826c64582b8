"""Pins of oracle/backward_oracle.py: every vector-Jacobian product against a
central finite difference of the forward it differentiates (flux_oracle, itself
pinned in test_oracle_pins.py).  For a scalar J = sum(G * f(theta)) with a
random upstream gradient G and a random direction U, the directional
derivative (J(theta + e U) - J(theta - e U)) / 2e must equal <grad, U>; in
float64 with e = 1e-6 the two agree to about 1e-8 relative, so a dropped term,
a wrong sign or a transposed operand anywhere in a backward fails here."""
import numpy as np
import pytest

import oracle as O
from oracle import backward_oracle as G

EPS_FD = 1e-6


def _dir_check(fwd, theta, grad, upstream, rng, tol=2e-7):
    """fwd(theta) -> array; grad = d(sum(upstream * fwd))/d theta."""
    u = rng.standard_normal(np.shape(theta))
    jp = np.sum(upstream * fwd(theta + EPS_FD * u))
    jm = np.sum(upstream * fwd(theta - EPS_FD * u))
    fd = (jp - jm) / (2 * EPS_FD)
    an = float(np.sum(grad * u))
    assert abs(fd - an) <= tol * max(1.0, abs(fd)), (fd, an)


def test_rf_loss_grad():
    rng = np.random.default_rng(0)
    z0, z1, v = (rng.standard_normal((2, 4, 3, 5)) for _ in range(3))
    g = G.rf_loss_grad(v, z0, z1)
    _dir_check(lambda vv: np.array(O.rf_loss(vv, z0, z1)[0]), v, g, 1.0, rng)


def test_activation_grads():
    x = np.linspace(-6, 6, 241)
    h = 1e-6
    np.testing.assert_allclose(G.gelu_grad(x), (O.gelu(x + h) - O.gelu(x - h)) / (2 * h), atol=1e-8)
    np.testing.assert_allclose(G.silu_grad(x), (O.silu(x + h) - O.silu(x - h)) / (2 * h), atol=1e-8)
    # closed forms: GELU'(0) = 1/2, SiLU'(0) = 1/2, both tend to 1 for large x
    assert G.gelu_grad(0.0) == 0.5 and G.silu_grad(0.0) == 0.5
    assert abs(G.gelu_grad(8.0) - 1.0) < 1e-12


def test_linear_vjp():
    rng = np.random.default_rng(1)
    x, w, b = rng.standard_normal((2, 5, 7)), rng.standard_normal((4, 7)), rng.standard_normal(4)
    dy = rng.standard_normal((2, 5, 4))
    dx, dw, db = G.linear_vjp(x, w, dy)
    _dir_check(lambda t: O.linear(t, w, b), x, dx, dy, rng)
    _dir_check(lambda t: O.linear(x, t, b), w, dw, dy, rng)
    _dir_check(lambda t: O.linear(x, w, t), b, db, dy, rng)


def test_modulate_vjp():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 5, 16)) * 3 + 1
    sh, sc = rng.standard_normal((2, 16)), rng.standard_normal((2, 16))
    dh = rng.standard_normal((2, 5, 16))
    dx, dsh, dsc = G.modulate_vjp(x, sh, sc, dh, 1e-6)
    _dir_check(lambda t: O.modulate(t, sh, sc, 1e-6), x, dx, dh, rng)
    _dir_check(lambda t: O.modulate(x, t, sc, 1e-6), sh, dsh, dh, rng)
    _dir_check(lambda t: O.modulate(x, sh, t, 1e-6), sc, dsc, dh, rng)
    # LayerNorm's output is invariant to a shift of x: dx sums to zero per row
    np.testing.assert_allclose(dx.sum(axis=-1), 0.0, atol=1e-12)


def test_rmsnorm_vjp():
    rng = np.random.default_rng(3)
    x, gm = rng.standard_normal((2, 5, 3, 8)), rng.standard_normal(8)
    dy = rng.standard_normal((2, 5, 3, 8))
    dx, dg = G.rmsnorm_vjp(x, gm, dy, 1e-6)
    _dir_check(lambda t: O.rmsnorm(t, gm, 1e-6), x, dx, dy, rng)
    _dir_check(lambda t: O.rmsnorm(x, t, 1e-6), gm, dg, dy, rng)


def test_rope_vjp():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 5, 3, 8))
    ang = rng.standard_normal((2, 5, 4)) * 3
    dy = rng.standard_normal(x.shape)
    _dir_check(lambda t: O.apply_rope(t, ang), x, G.rope_vjp(dy, ang), dy, rng)


def test_attention_vjp():
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((2, 6, 3, 8)) for _ in range(3))
    do = rng.standard_normal((2, 6, 24))
    dq, dk, dv = G.attention_vjp(q, k, v, do)
    _dir_check(lambda t: O.attention(t, k, v), q, dq, do, rng)
    _dir_check(lambda t: O.attention(q, t, v), k, dk, do, rng)
    _dir_check(lambda t: O.attention(q, k, t), v, dv, do, rng)
    # softmax is invariant to adding a constant to every score of a row, and
    # the rows of P sum to one: sum over keys of dk is orthogonal to nothing
    # in particular, but dv summed over keys equals do summed per head
    np.testing.assert_allclose(dv.sum(axis=1).reshape(2, 24), do.sum(axis=1), atol=1e-12)


def test_adaln_vjp():
    rng = np.random.default_rng(6)
    vec, w, b = rng.standard_normal((2, 8)), rng.standard_normal((24, 8)), rng.standard_normal(24)
    dm = rng.standard_normal((2, 24))
    dvec, dw, db = G.adaln_vjp(vec, w, dm)
    f = lambda vv, ww, bb: np.concatenate(O.adaln(vv, ww, bb, 3), axis=-1)
    _dir_check(lambda t: f(t, w, b), vec, dvec, dm, rng)
    _dir_check(lambda t: f(vec, t, b), w, dw, dm, rng)
    _dir_check(lambda t: f(vec, w, t), b, db, dm, rng)


# ------------------------------ whole blocks ------------------------------ #
B, LI, LT, D, H, DH, F = 2, 3, 2, 16, 2, 8, 32
AXES = (2, 2, 4)


def _angles(rng, L):
    ids = np.stack([np.zeros((B, L)), rng.integers(0, 4, (B, L)), rng.integers(0, 4, (B, L))], axis=-1)
    return O.rope_angles(ids, AXES, 10000.0)


def _single_w(rng):
    s = 0.3
    return {"mod.w": rng.standard_normal((3 * D, D)) * s, "mod.b": rng.standard_normal(3 * D) * s,
            "lin1.w": rng.standard_normal((3 * D + F, D)) * s, "lin1.b": rng.standard_normal(3 * D + F) * s,
            "q_norm": 1 + 0.3 * rng.standard_normal(DH), "k_norm": 1 + 0.3 * rng.standard_normal(DH),
            "lin2.w": rng.standard_normal((D, D + F)) * s, "lin2.b": rng.standard_normal(D) * s}


def _double_w(rng):
    s, w = 0.3, {}
    for p in ("img_", "txt_"):
        for n, shp in (("mod", (6 * D, D)), ("qkv", (3 * D, D)), ("proj", (D, D)), ("fc1", (F, D)), ("fc2", (D, F))):
            w[p + n + ".w"] = rng.standard_normal(shp) * s
            w[p + n + ".b"] = rng.standard_normal(shp[0]) * s
        w[p + "q_norm"] = 1 + 0.3 * rng.standard_normal(DH)
        w[p + "k_norm"] = 1 + 0.3 * rng.standard_normal(DH)
    return w


def test_single_block_vjp():
    rng = np.random.default_rng(7)
    L = LI + LT
    x, vec, ang, w = rng.standard_normal((B, L, D)), rng.standard_normal((B, D)), _angles(rng, L), _single_w(rng)
    dout = rng.standard_normal((B, L, D))
    dx, dvec, g = G.single_block_vjp(x, vec, ang, w, H, 1e-6, dout)
    fwd = lambda xx=x, vv=vec, ww=w: O.single_block(xx, vv, ang, ww, H, 1e-6)
    _dir_check(lambda t: fwd(xx=t), x, dx, dout, rng)
    _dir_check(lambda t: fwd(vv=t), vec, dvec, dout, rng)
    assert set(g) == set(w)
    for n in w:
        _dir_check(lambda t: fwd(ww=dict(w, **{n: t})), w[n], g[n], dout, rng)


def test_double_block_vjp():
    rng = np.random.default_rng(8)
    xi, xt = rng.standard_normal((B, LI, D)), rng.standard_normal((B, LT, D))
    vec, ang, w = rng.standard_normal((B, D)), _angles(rng, LI + LT), _double_w(rng)
    di, dt = rng.standard_normal((B, LI, D)), rng.standard_normal((B, LT, D))
    dxi, dxt, dvec, g = G.double_block_vjp(xi, xt, vec, ang, w, H, 1e-6, di, dt)

    def fwd(a=xi, b=xt, vv=vec, ww=w):
        oi, ot = O.double_block(a, b, vv, ang, ww, H, 1e-6)
        return np.concatenate([oi, ot], axis=1)

    up = np.concatenate([di, dt], axis=1)
    _dir_check(lambda t: fwd(a=t), xi, dxi, up, rng)
    _dir_check(lambda t: fwd(b=t), xt, dxt, up, rng)
    _dir_check(lambda t: fwd(vv=t), vec, dvec, up, rng)
    assert set(g) == set(w)
    for n in w:
        _dir_check(lambda t: fwd(ww=dict(w, **{n: t})), w[n], g[n], up, rng)


def test_block_vjp_adaln_zero():
    # with the modulation weights and biases zero every gate is zero: the block
    # is the identity, so dx = dout, every gradient below the gates vanishes,
    # and the gate gradients are the column sums of y * dout
    rng = np.random.default_rng(9)
    L = LI + LT
    x, vec, ang, w = rng.standard_normal((B, L, D)), rng.standard_normal((B, D)), _angles(rng, L), _single_w(rng)
    w["mod.w"][:] = 0.0
    w["mod.b"][:] = 0.0
    dout = rng.standard_normal((B, L, D))
    dx, dvec, g = G.single_block_vjp(x, vec, ang, w, H, 1e-6, dout)
    np.testing.assert_array_equal(dx, dout)
    for n in ("lin1.w", "lin1.b", "lin2.w", "lin2.b", "q_norm", "k_norm"):
        assert np.all(g[n] == 0.0), n
    assert np.abs(g["mod.b"][2 * D:]).max() > 0 and np.all(g["mod.b"][:2 * D] == 0.0)


# --------------------------- head, embeddings, step --------------------------- #
C_LAT, HH, WW, CTX, YD, MC = 4, 2, 3, 12, 10, 16


def _emb_w(rng, with_y=True, with_txt=True):
    s, w = 0.3, {}
    shapes = {"img_in": (D, C_LAT), "time_in1": (D, MC), "time_in2": (D, D), "final_mod": (2 * D, D),
              "final_out": (C_LAT, D)}
    if with_y:
        shapes.update({"vector_in1": (D, YD), "vector_in2": (D, D)})
    if with_txt:
        shapes["txt_in"] = (D, CTX)
    for n, shp in shapes.items():
        w[n + ".w"] = rng.standard_normal(shp) * s
        w[n + ".b"] = rng.standard_normal(shp[0]) * s
    return w


def test_final_layer_vjp():
    rng = np.random.default_rng(10)
    w = _emb_w(rng)
    x, vec = rng.standard_normal((B, HH * WW, D)), rng.standard_normal((B, D))
    dv = rng.standard_normal((B, C_LAT, HH, WW))
    dx, dvec, g = G.final_layer_vjp(x, vec, w, 1e-6, dv)
    fwd = lambda xx=x, vv=vec, ww=w: O.final_layer(xx, vv, ww, HH, WW, 1e-6)
    _dir_check(lambda t: fwd(xx=t), x, dx, dv, rng)
    _dir_check(lambda t: fwd(vv=t), vec, dvec, dv, rng)
    for n in ("final_mod.w", "final_mod.b", "final_out.w", "final_out.b"):
        _dir_check(lambda t: fwd(ww=dict(w, **{n: t})), w[n], g[n], dv, rng)


def test_conditioning_vjp():
    rng = np.random.default_rng(11)
    w = _emb_w(rng)
    t, y = rng.uniform(size=B), rng.standard_normal((B, YD))
    dvec = rng.standard_normal((B, D))
    g = G.conditioning_vjp(t, y, w, dvec, MC)
    assert set(g) == {"time_in1.w", "time_in1.b", "time_in2.w", "time_in2.b", "vector_in1.w", "vector_in1.b",
                      "vector_in2.w", "vector_in2.b"}
    for n in g:
        _dir_check(lambda u: O.conditioning_vector(t, y, dict(w, **{n: u}), MC), w[n], g[n], dvec, rng)


def test_conditioning_vjp_with_guidance():
    rng = np.random.default_rng(13)
    w = _emb_w(rng)
    w["guidance_in.w"], w["guidance_in.b"] = rng.standard_normal((D, 1)), rng.standard_normal(D)
    t, y, gs = rng.uniform(size=B), rng.standard_normal((B, YD)), rng.uniform(1.0, 5.0, size=B)
    dvec = rng.standard_normal((B, D))
    g = G.conditioning_vjp(t, y, w, dvec, MC, guidance=gs)
    assert {"guidance_in.w", "guidance_in.b"} <= set(g)
    for n in ("guidance_in.w", "guidance_in.b", "time_in2.w"):
        _dir_check(lambda u: O.conditioning_vector(t, y, dict(w, **{n: u}), MC, gs), w[n], g[n], dvec, rng)
    # the embedding is affine in its weights: dW = sum_b g_b dvec_b exactly
    assert np.allclose(g["guidance_in.w"][:, 0], gs @ dvec, rtol=1e-14, atol=0)


def test_flux_train_vjp():
    # the gradient of the whole step's loss with respect to every weight group,
    # along random directions, against central differences of the forward loss
    rng = np.random.default_rng(12)
    w_emb = _emb_w(rng)
    w2, w1 = _double_w(rng), _single_w(rng)
    z0, z1 = rng.standard_normal((B, C_LAT, HH, WW)), rng.standard_normal((B, C_LAT, HH, WW))
    t = rng.uniform(0.05, 0.95, size=B)
    txt, y = rng.standard_normal((B, LT, CTX)), rng.standard_normal((B, YD))
    ids = np.concatenate([np.stack([np.zeros((B, HH * WW)), np.repeat(np.arange(HH), WW)[None].repeat(B, 0),
                                    np.tile(np.arange(WW), HH)[None].repeat(B, 0)], -1), np.zeros((B, LT, 3))], 1)
    loss, g_emb, g2, g1 = G.flux_train_vjp(z0, z1, t, txt, y, ids, w_emb, [w2], [w1], H, AXES, 1e4, 1e-6, MC)

    def J(we=w_emb, a=w2, b=w1):
        v = O.flux_forward(O.rf_noise(z0, z1, t)[0], txt, y, t, ids, we, [a], [b], H, AXES, 1e4, 1e-6, MC)
        return np.array(O.rf_loss(v, z0, z1)[0])

    assert abs(loss - float(J())) <= 1e-12 * max(1.0, abs(loss))
    assert set(g_emb) == set(w_emb)
    for n in w_emb:
        _dir_check(lambda u: J(we=dict(w_emb, **{n: u})), w_emb[n], g_emb[n], 1.0, rng)
    for n in ("img_qkv.w", "txt_fc2.b", "img_q_norm", "txt_mod.w"):
        _dir_check(lambda u: J(a=dict(w2, **{n: u})), w2[n], g2[0][n], 1.0, rng)
    for n in ("lin1.w", "k_norm", "mod.b"):
        _dir_check(lambda u: J(b=dict(w1, **{n: u})), w1[n], g1[0][n], 1.0, rng)


def test_single_block_sequential_vjp():
    rng = np.random.default_rng(13)
    L = LI + LT
    w = {k[len("img_"):]: v for k, v in _double_w(rng).items() if k.startswith("img_")}
    x, vec, ang = rng.standard_normal((B, L, D)), rng.standard_normal((B, D)), _angles(rng, L)
    dout = rng.standard_normal((B, L, D))
    dx, dvec, g = G.single_block_sequential_vjp(x, vec, ang, w, H, 1e-6, dout)
    fwd = lambda xx=x, vv=vec, ww=w: O.single_block_sequential(xx, vv, ang, ww, H, 1e-6)
    _dir_check(lambda t: fwd(xx=t), x, dx, dout, rng)
    _dir_check(lambda t: fwd(vv=t), vec, dvec, dout, rng)
    assert set(g) == set(w)
    for n in w:
        _dir_check(lambda t: fwd(ww=dict(w, **{n: t})), w[n], g[n], dout, rng)
