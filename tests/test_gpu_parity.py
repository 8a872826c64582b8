"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.

Tolerances: fp32 workloads and bf16 workloads alike must meet max-abs <= 3e-2
and relative L2 <= 1e-2 on every compared output; rf noising is bit-exact
against the oracle's float32 evaluation order, the loss within 1e-6
relative.  Larger shapes compare sampled token rows (the oracle evaluates just
those rows, keys and values still cover every token).
"""
import os

import numpy as np
import pytest

import oracle as O
from flow_matching_diffusion_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2 = 3e-2, 1e-2


def _say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from flow_matching_diffusion_amd import flux
    flux.lib()          # fails loudly when the library is missing
    torch.cuda.set_device(0)


def F():
    from flow_matching_diffusion_amd import flux
    return flux


def M():
    from flow_matching_diffusion_amd import model
    return model


def dev(a, bf16=False):
    return M().device_array(a, bf16)


def errs(g, o):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    d = g - o
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(o), 1e-300))


def assert_close(g, o, what, max_abs=MAX_ABS, rel=REL_L2):
    a, r = errs(g, o)
    print(f"    {what}: max_abs={a:.3e} rel_l2={r:.3e}", flush=True)
    assert np.all(np.isfinite(np.asarray(g))), what
    assert a <= max_abs and r <= rel, (what, a, r)


# --------------------------------------------------------------------------- #
# rectified flow
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("shape", [(1, 64, 8, 8), (1, 64, 32, 32), (2, 64, 64, 64), (3, 1, 1, 333)])
def test_rf_noise_bitexact_and_loss(shape):
    _say(f"rf_noise_loss shape={shape}")
    rng = np.random.default_rng(11)
    z0 = rng.standard_normal(shape).astype(np.float32)
    z1 = rng.standard_normal(shape).astype(np.float32)
    B = shape[0]
    t = np.array([0.0, 1.0, 0.37][:B] if B > 1 else [0.61], dtype=np.float32)
    if B == 2:
        t = np.array([0.0, 1.0], np.float32)
    vp = rng.standard_normal(shape).astype(np.float32)
    n = int(np.prod(shape[1:]))
    f = F()
    dz0, dz1, dt, dvp = dev(z0), dev(z1), dev(t), dev(vp)
    zt = torch.empty_like(dz0)
    vt = torch.empty_like(dz0)
    loss = torch.empty(1, device="cuda")
    lps = torch.empty(B, device="cuda")
    wsb = f.flux_rf_workspace_bytes(B, n)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    f.rf_noise_loss(B, n, dz0, dz1, dt, z_t=zt, v_target=vt, v_pred=dvp, loss=loss, loss_per_sample=lps,
                    workspace=ws, workspace_bytes=wsb)
    torch.cuda.synchronize()
    ozt, ovt = O.rf_noise_f32_order(z0, z1, t)
    assert np.array_equal(zt.cpu().numpy(), ozt)
    assert np.array_equal(vt.cpu().numpy(), ovt)
    if B >= 2:
        assert np.array_equal(zt.cpu().numpy()[0], z0[0]) and np.array_equal(zt.cpu().numpy()[1], z1[1])
    ol, ops = O.rf_loss(vp, z0, z1)
    assert abs(loss.item() - ol) <= 1e-6 * ol
    np.testing.assert_allclose(lps.cpu().numpy(), ops, rtol=1e-6)
    # fixed-order reduction: bitwise repeatable
    loss2 = torch.empty(1, device="cuda")
    f.rf_noise_loss(B, n, dz0, dz1, dt, v_pred=dvp, loss=loss2, workspace=ws, workspace_bytes=wsb)
    torch.cuda.synchronize()
    assert loss2.item() == loss.item()


# --------------------------------------------------------------------------- #
# RoPE table
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("name,cg", [("tiny_fp32", False), ("flux12b_blocks", False), ("flux12b_blocks", True)])
def test_rope_table(name, cg):
    _say(f"rope table {name} channel_group={cg}")
    wl = synth.WORKLOADS[name]
    ids = synth.joint_ids(wl, channel_group=cg)
    B, L = ids.shape[:2]
    table = torch.empty((B, L, wl.head_dim // 2, 2), device="cuda")
    F().flux_rope_table(dev(ids), B, L, wl.axes_dim, wl.theta, table)
    torch.cuda.synchronize()
    ang = O.rope_angles(ids, wl.axes_dim, wl.theta)
    g = table.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(g[..., 0], np.cos(ang), atol=1e-7, rtol=0)
    np.testing.assert_allclose(g[..., 1], np.sin(ang), atol=1e-7, rtol=0)


@pytest.mark.parametrize("batch,dim", [(1, 256), (5, 256), (3, 18)])
def test_timestep_embed(batch, dim):
    # both sides evaluate the sinusoid in fp64 from the same float32 t; the
    # float store is the only rounding
    _say(f"timestep sinusoid batch={batch} dim={dim}")
    rng = np.random.default_rng(batch * 31 + dim)
    t = rng.uniform(0.0, 1.0, size=batch).astype(np.float32)
    t[0] = 1.0
    if batch > 1:
        t[1] = 0.0
    out = torch.full((batch, dim), float("nan"), device="cuda")
    F().flux_timestep_embed(dev(t), batch, dim, 1000.0, out)
    torch.cuda.synchronize()
    ref = O.timestep_embedding(t.astype(np.float64), dim, 1000.0)
    np.testing.assert_allclose(out.cpu().numpy().astype(np.float64), ref, atol=1e-7, rtol=0)


# --------------------------------------------------------------------------- #
# linear (GEMM)
# --------------------------------------------------------------------------- #
# the 4608 x 9216 and the two 4096-wide cases run on the persistent ring
# kernel (>= 128 tiles of 256 x 256): K = 3072, and its smallest K (512, four
# k units) and an odd number of k units (640) with a partly filled last tile row
@pytest.mark.parametrize("prec,m,n,k", [("bf16", 80, 768, 256), ("bf16", 333, 1284, 512), ("bf16", 1536, 3072, 3072),
                                        ("bf16", 4608, 9216, 3072), ("bf16", 2100, 4096, 640),
                                        ("bf16", 2304, 4096, 512), ("f32", 80, 768, 256), ("f32", 77, 36, 40)])
def test_linear(prec, m, n, k):
    _say(f"linear {prec} m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 7 + n)
    bf = prec == "bf16"
    x = rng.standard_normal((m, k)).astype(np.float32)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    b = (0.02 * rng.standard_normal(n)).astype(np.float32)
    if bf:
        x, w, b = synth.round_to_bf16(x), synth.round_to_bf16(w), synth.round_to_bf16(b)
    y = torch.empty((m, n), device="cuda")
    p = F().FLUX_PREC_BF16 if bf else F().FLUX_PREC_F32
    xd, wd, bd = dev(x, bf), dev(w, bf), dev(b, bf)
    torch.cuda.synchronize()
    F().flux_timing_read()   # clears the counts of earlier launches
    F().flux_timing_enable(True)
    F().flux_linear_fwd(p, m, n, k, xd, k, wd, bd, y, n)
    torch.cuda.synchronize()
    launches = {c: v[1] for c, v in F().flux_timing_read().items() if v[1]}
    F().flux_timing_enable(False)
    if bf and m * n >= 128 * 256 * 256 and k >= 512:
        assert "gemm_256_bf16" in launches, launches   # the persistent ring kernel ran
    rows = np.arange(m) if m <= 512 else np.unique(np.r_[rng.choice(m, 96, replace=False), 0, m - 1])
    ref = O.linear(x[rows], w, b)
    g = y.cpu().numpy()[rows]
    # fp32 accumulation of exactly representable products: only summation rounding
    assert_close(g, ref, "linear", max_abs=1e-4, rel=1e-5)


# --------------------------------------------------------------------------- #
# attention
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("prec,B,L,H,dh", [("bf16", 1, 80, 4, 64), ("bf16", 2, 200, 2, 128), ("bf16", 1, 1536, 24, 128),
                                           ("bf16", 1, 4608, 24, 128), ("bf16", 1, 40, 2, 64), ("bf16", 2, 40, 2, 128),
                                           ("bf16", 1, 257, 3, 128),
                                           ("f32", 1, 80, 4, 64), ("f32", 2, 130, 2, 128)])
def test_attention(prec, B, L, H, dh):
    _say(f"attention {prec} B={B} L={L} H={H} dh={dh}")
    rng = np.random.default_rng(L + H)
    bf = prec == "bf16"
    D = H * dh
    q, k, v = (rng.standard_normal((B, L, D)).astype(np.float32) for _ in range(3))
    q *= 0.25  # scores of O(1) spread after the 1/sqrt(dh) scale
    if bf:
        q, k, v = synth.round_to_bf16(q), synth.round_to_bf16(k), synth.round_to_bf16(v)
    f = F()
    p = f.FLUX_PREC_BF16 if bf else f.FLUX_PREC_F32
    o = torch.empty((B, L, D), device="cuda", dtype=torch.bfloat16 if bf else torch.float32)
    wsb = f.flux_attention_workspace_bytes(p, B, L, H, dh)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    f.flux_attention_fwd(p, B, L, H, dh, dev(q, bf), dev(k, bf), dev(v, bf), D, o, D, ws, wsb)
    torch.cuda.synchronize()
    rows = np.arange(L) if L <= 256 else np.unique(np.r_[rng.choice(L, 64, replace=False), 0, L - 1])
    hd = lambda a: a.reshape(B, a.shape[1], H, dh)
    ref = O.attention(hd(q[:, rows]), hd(k), hd(v))
    g = o.float().cpu().numpy()[:, rows]
    assert_close(g, ref, "attention")


def test_attention_repeatable():
    # every launch of the same problem gives the same bits: the K / V tiles are
    # handed between waves through LDS under barriers, with no reduction whose
    # order depends on timing
    B, L, H, dh = 1, 4608, 24, 128
    _say(f"attention bf16 B={B} L={L} H={H} dh={dh}: 20 launches bit-identical")
    rng = np.random.default_rng(11)
    D = H * dh
    q, k, v = (dev(synth.round_to_bf16(rng.standard_normal((B, L, D)).astype(np.float32)), True) for _ in range(3))
    f = F()
    p = f.FLUX_PREC_BF16
    wsb = f.flux_attention_workspace_bytes(p, B, L, H, dh)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(20):
        o = torch.empty((B, L, D), device="cuda", dtype=torch.bfloat16)
        f.flux_attention_fwd(p, B, L, H, dh, q, k, v, D, o, D, ws, wsb)
        outs.append(o)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


# --------------------------------------------------------------------------- #
# blocks
# --------------------------------------------------------------------------- #
def _block_fixture(wl):
    w2 = synth.double_block_weights(wl, 0)
    w1 = synth.single_block_weights(wl, 1)
    inp = synth.block_inputs(wl)
    ids = synth.joint_ids(wl)
    return w2, w1, inp, ids


def _run_pair(wl, w2, w1, inp, ids, which, weights_f16=False):
    """Run the double block (which='double') or the single block on the joint
    buffer [x_img | x_txt] and return the joint result."""
    stack = M().BlockStack(wl, [w2] if which == "double" else [], [w1] if which == "single" else [],
                           weights_f16=weights_f16)
    x = dev(np.concatenate([inp["x_img"], inp["x_txt"]], axis=1))
    vec = dev(inp["vec"])
    rope = stack.rope_table(dev(ids))
    if which == "double":
        stack.double_fwd(0, x, vec, rope)
    else:
        stack.single_fwd(0, x, vec, rope)
    torch.cuda.synchronize()
    return x.cpu().numpy()


def _check_double(wl, w2, inp, ids, g, rows=None):
    ang = O.rope_angles(ids, wl.axes_dim, wl.theta)
    if rows is None:
        ri, rt = np.arange(wl.l_img), np.arange(wl.l_txt)
    else:
        ri, rt = rows
    oi, ot = O.double_block(inp["x_img"], inp["x_txt"], inp["vec"], ang, w2, wl.heads, wl.eps,
                            rows={"img": ri, "txt": rt})
    assert_close(g[:, ri], oi, "double img")
    assert_close(g[:, wl.l_img + rt], ot, "double txt")


def _check_single(wl, w1, inp, ids, g, rows=None):
    ang = O.rope_angles(ids, wl.axes_dim, wl.theta)
    x = np.concatenate([inp["x_img"], inp["x_txt"]], axis=1)
    sel = np.arange(wl.seq) if rows is None else rows
    o = O.single_block(x, inp["vec"], ang, w1, wl.heads, wl.eps, rows=sel)
    assert_close(g[:, sel], o, "single")


SMALL = {
    "tiny_fp32": synth.WORKLOADS["tiny_fp32"],
    "tiny_bf16": synth.custom_workload("tiny_bf16", base="tiny_fp32", precision="bf16"),
    # ragged: 7x9 image + 11 text tokens (L = 74), batch 2, Dh 128
    "ragged_bf16": synth.custom_workload("ragged_bf16", base="tiny_fp32", precision="bf16", batch=2, img_h=7, img_w=9,
                                         l_txt=11, hidden=256, heads=2, head_dim=128, mlp_hidden=512,
                                         axes_dim=(16, 56, 56)),
    "ragged_fp32": synth.custom_workload("ragged_fp32", base="tiny_fp32", batch=2, img_h=5, img_w=13, l_txt=3),
}


SMALL_CASES = [(n, False) for n in SMALL] + [(n, True) for n in SMALL if SMALL[n].precision == "bf16"]


@pytest.mark.parametrize("name,wf16", SMALL_CASES)
def test_double_block_small(name, wf16):
    wl = SMALL[name]
    _say(f"double block {name} weights_f16={wf16}")
    w2, w1, inp, ids = _block_fixture(wl)
    g = _run_pair(wl, w2, w1, inp, ids, "double", wf16)
    _check_double(wl, w2, inp, ids, g)


@pytest.mark.parametrize("name,wf16", SMALL_CASES)
def test_single_block_small(name, wf16):
    wl = SMALL[name]
    _say(f"single block {name} weights_f16={wf16}")
    w2, w1, inp, ids = _block_fixture(wl)
    g = _run_pair(wl, w2, w1, inp, ids, "single", wf16)
    _check_single(wl, w1, inp, ids, g)


def _f16_toward_zero(a):
    """fp16 of float32 values rounded toward zero, saturating finite values
    at +-65504 (numpy rounds to nearest; step back one ulp where it rounded
    away from zero)."""
    with np.errstate(over="ignore"):
        r = a.astype(np.float16)
    big = np.isfinite(a) & (np.abs(a) > 65504.0)
    r[big] = np.copysign(np.float16(65504.0), a[big]).astype(np.float16)
    up = np.isfinite(r) & (np.abs(r.astype(np.float32)) > np.abs(a))
    r[up] = np.nextafter(r[up], np.float16(0.0))
    return r


def test_convert_bf16_to_f16_toward_zero():
    _say("bf16 -> fp16 weight conversion")
    rng = np.random.default_rng(5)
    a = (0.02 * rng.standard_normal(100003)).astype(np.float32)
    a[:40] = np.float32(2.0) ** -np.arange(10, 50, dtype=np.float32)      # down through fp16 subnormals
    a[40:60] = rng.standard_normal(20).astype(np.float32) * 1000.0         # large magnitudes
    a[60:64] = [7.0e4, -1.0e6, 65504.0, -3.0e38]                            # beyond fp16's range: saturate
    a[100002] = -(2.0 ** -20) * 1.5                                        # odd tail element, subnormal
    a = synth.round_to_bf16(a)
    src = dev(a, True)
    dst = torch.empty(a.shape, dtype=torch.float16, device="cuda")
    F().flux_convert_bf16_to_f16(src, dst, a.size)
    torch.cuda.synchronize()
    ref = _f16_toward_zero(a)
    assert np.array_equal(dst.cpu().numpy().view(np.uint16), ref.view(np.uint16))
    # exact wherever the magnitude is in fp16's normal range
    normal = (np.abs(a) >= 2.0 ** -14) & (np.abs(a) <= 65504.0)
    assert np.array_equal(ref[normal].astype(np.float32), a[normal])
    inr = np.abs(a) <= 65504.0
    assert np.abs(ref[inr].astype(np.float64) - a[inr]).max() <= 2.0 ** -24


def test_block_no_text_tokens():
    wl = synth.custom_workload("img_only_bf16", base="tiny_fp32", precision="bf16", l_txt=0)
    _say("double + single block with l_txt = 0")
    w2, w1, inp, ids = _block_fixture(wl)
    g = _run_pair(wl, w2, w1, inp, ids, "double")
    ang = O.rope_angles(ids, wl.axes_dim, wl.theta)
    oi, _ = O.double_block(inp["x_img"], inp["x_txt"], inp["vec"], ang, w2, wl.heads, wl.eps)
    assert_close(g, oi, "double img-only")
    g = _run_pair(wl, w2, w1, inp, ids, "single")
    _check_single(wl, w1, inp, ids, g)


@pytest.fixture(scope="module")
def big_case():
    wl = synth.WORKLOADS["flux12b_blocks"]
    _say("generating flux12b_blocks weights")
    return (wl,) + _block_fixture(wl)


def _sample_rows(wl, seed):
    rng = np.random.default_rng(seed)
    ri = np.unique(np.r_[rng.choice(wl.l_img, 24, replace=False), 0, wl.l_img - 1])
    rt = np.unique(np.r_[rng.choice(wl.l_txt, 8, replace=False), 0, wl.l_txt - 1])
    return ri, rt


@pytest.mark.slow
def test_double_block_flux12b_shapes_sampled(big_case):
    wl, w2, w1, inp, ids = big_case
    _say("double block flux12b_blocks (L=4608) sampled rows, fp16-held linear weights")
    g = _run_pair(wl, w2, w1, inp, ids, "double", True)
    _check_double(wl, w2, inp, ids, g, rows=_sample_rows(wl, 1))


@pytest.mark.slow
def test_single_block_flux12b_shapes_sampled(big_case):
    wl, w2, w1, inp, ids = big_case
    _say("single block flux12b_blocks (L=4608) sampled rows, fp16-held linear weights")
    g = _run_pair(wl, w2, w1, inp, ids, "single", True)
    ri, rt = _sample_rows(wl, 2)
    _check_single(wl, w1, inp, ids, g, rows=np.r_[ri, wl.l_img + rt])


def test_adaln_zero_identity_and_determinism():
    wl = SMALL["tiny_bf16"]
    _say("adaLN-zero identity / determinism (tiny_bf16)")
    w2, w1, inp, ids = _block_fixture(wl)
    z2 = dict(w2)
    for k in z2:
        if "_mod." in k:
            z2[k] = np.zeros_like(z2[k])
    z1 = dict(w1, **{"mod.w": np.zeros_like(w1["mod.w"]), "mod.b": np.zeros_like(w1["mod.b"])})
    x0 = np.concatenate([inp["x_img"], inp["x_txt"]], axis=1)
    assert np.array_equal(_run_pair(wl, z2, z1, inp, ids, "double"), x0)
    assert np.array_equal(_run_pair(wl, z2, z1, inp, ids, "single"), x0)
    a = _run_pair(wl, w2, w1, inp, ids, "double")
    b = _run_pair(wl, w2, w1, inp, ids, "double")
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------- #
# whole forward + loss
# --------------------------------------------------------------------------- #
def _forward_case(wl, weights_f16=False):
    emb = synth.embed_weights(wl)
    w2s = [synth.double_block_weights(wl, i) for i in range(wl.n_double)]
    w1s = [synth.single_block_weights(wl, 100 + i) for i in range(wl.n_single)]
    mi = synth.model_inputs(wl)
    m = M().FluxModel(wl, emb, w2s, w1s, weights_f16=weights_f16)
    bf = wl.precision != "f32"
    out = m.forward_loss(dev(mi["z0"]), dev(mi["z1"]), dev(mi["t"]), dev(mi["txt"], bf),
                         dev(mi["y"]) if "y" in mi else None, dev(mi["ids"]))
    torch.cuda.synchronize()
    zt, _ = O.rf_noise(mi["z0"], mi["z1"], mi["t"])
    v = O.flux_forward(zt, mi["txt"], mi.get("y"), mi["t"], mi["ids"], emb, w2s, w1s, wl.heads, wl.axes_dim,
                       wl.theta, wl.eps, wl.model_channels)
    loss, per = O.rf_loss(v, mi["z0"], mi["z1"])
    assert_close(out["v_pred"].cpu().numpy(), v, "v_pred")
    gl = out["loss"].item()
    print(f"    loss gpu={gl:.6f} oracle={loss:.6f}", flush=True)
    assert abs(gl - loss) <= 1e-2 * abs(loss)
    np.testing.assert_allclose(out["loss_per_sample"].cpu().numpy(), per, rtol=1e-2)


def test_forward_tiny_fp32():
    _say("whole forward + loss tiny_fp32")
    _forward_case(synth.WORKLOADS["tiny_fp32"])


def test_forward_tiny_bf16_with_pooled_vector():
    _say("whole forward + loss tiny (bf16, txt_in and vector_in)")
    wl = synth.custom_workload("tiny_bf16_full", base="tiny_fp32", precision="bf16", context_dim=128, vec_in_dim=64,
                               batch=2, t_dist="logit_normal")
    _forward_case(wl)


@pytest.mark.slow
def test_forward_flux535m():
    _say("whole forward + loss flux535m (L=1536), fp16-held linear weights")
    _forward_case(synth.WORKLOADS["flux535m"], weights_f16=True)


@pytest.fixture(scope="module")
def padded_case():
    # batch 2, 50x60 image + 77 text tokens: L = 3077 is padded to 3328 for
    # attention, the text stream starts at a row that is not a multiple of 32,
    # and the q|k|v projection still runs on the persistent GEMM, whose
    # epilogue writes the attention layouts (RMSNorm and RoPE fused)
    wl = synth.custom_workload("padded_12b_width", base="flux12b_blocks", batch=2, img_h=50, img_w=60, l_txt=77)
    _say("generating padded 12B-width weights")
    w2, w1, inp, ids = _block_fixture(wl)
    ids = synth.joint_ids(wl, channel_group=True)        # axis-0 ids nonzero: every RoPE axis turns
    return wl, w2, w1, inp, ids


@pytest.mark.slow
def test_fused_qkv_epilogue_double_block_padded(padded_case):
    wl, w2, w1, inp, ids = padded_case
    _say("double block, B=2, L=3000+77 (padded to 3328), fused q/k norm + RoPE epilogue, sampled rows")
    g = _run_pair(wl, w2, w1, inp, ids, "double", True)
    ri, rt = _sample_rows(wl, 3)
    _check_double(wl, w2, inp, ids, g, rows=(ri, rt))


@pytest.mark.slow
def test_fused_qkv_epilogue_single_block_padded(padded_case):
    wl, w2, w1, inp, ids = padded_case
    _say("single block, B=2, L=3077 (padded to 3328), fused q/k norm + RoPE epilogue, sampled rows")
    g = _run_pair(wl, w2, w1, inp, ids, "single", True)
    ri, rt = _sample_rows(wl, 4)
    _check_single(wl, w1, inp, ids, g, rows=np.r_[ri, wl.l_img + rt])


def test_fp16_activation_store_saturates():
    """fp16 activation stores saturate at +-65504 instead of overflowing to
    infinity: the output head's LayerNorm-modulate output (an fp16 operand of
    the output linear) with scale = 999424 reaches |h| ~ 1e6.  The reference
    clips h at 65504, rounds it to fp16 and applies the linear in float64."""
    _say("output head with |LayerNorm-modulate output| far beyond fp16's range (saturating fp16 store)")
    rng = np.random.default_rng(65504)
    B, C, H, W, D, eps = 1, 64, 4, 4, 256, 1e-6
    HW = H * W
    x = rng.standard_normal((B, HW, D)).astype(np.float32)
    vec = rng.standard_normal((B, D)).astype(np.float32)
    mod_w = np.zeros((2 * D, D), np.float32)
    mod_b = np.concatenate([np.zeros(D), np.full(D, 999424.0)]).astype(np.float32)   # shift 0, scale 999424 (bf16-exact)
    out_w = synth.round_to_bf16((0.02 * rng.standard_normal((C, D))).astype(np.float32))
    out_b = np.zeros(C, np.float32)
    f = F()
    v = torch.empty((B, C, H, W), device="cuda")
    wsb = f.flux_final_workspace_bytes(f.FLUX_PREC_BF16, B, H, W, D)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
    f.flux_final_fwd(f.FLUX_PREC_BF16, B, C, H, W, D, eps, dev(mod_w, True), dev(mod_b, True), dev(out_w, True),
                     dev(out_b, True), dev(x), HW * D, dev(vec), v, ws, wsb)
    torch.cuda.synchronize()
    got = v.cpu().numpy()
    xd = x.astype(np.float64)
    mu = xd.mean(-1, keepdims=True)
    var = ((xd - mu) ** 2).mean(-1, keepdims=True)
    h = (xd - mu) / np.sqrt(var + eps) * (1.0 + 999424.0)
    assert np.abs(h).max() > 1e5          # far beyond fp16's largest finite value
    h16 = np.clip(h, -65504.0, 65504.0).astype(np.float16).astype(np.float64)
    tok = h16 @ out_w.astype(np.float64).T
    ref = tok.reshape(B, H, W, C).transpose(0, 3, 1, 2)
    assert np.isfinite(got).all(), "an fp16 activation overflowed"
    assert_close(got, ref, "v_pred with saturated activations", max_abs=1e-3 * np.abs(ref).max(), rel=1e-3)


@pytest.mark.slow
def test_stream_k_tail_matches_whole_tiles_and_repeats(big_case):
    """Stream-K tail of the block linears (qkv 648 tiles, fc1 864, proj / fc2
    216 per launch at L=4608): two runs are bitwise equal; the outputs agree
    with the whole-tile path (stream-K off) to rounding; with a poll limit of
    one the finishing blocks compute late shares themselves and the result
    still agrees.  The oracle check of the same block is
    test_double_block_flux12b_shapes_sampled."""
    wl, w2, w1, inp, ids = big_case
    f = F()
    _say("stream-K tail: double + single block at L=4608, repeatability, whole-tile and fallback agreement")
    prev = f.flux_gemm_stream_k(True)
    try:
        for which in ("double", "single"):
            a = _run_pair(wl, w2, w1, inp, ids, which, True)
            b = _run_pair(wl, w2, w1, inp, ids, which, True)
            assert np.array_equal(a, b), f"{which}: stream-K run is not bitwise repeatable"
            f.flux_gemm_stream_k(False)
            c = _run_pair(wl, w2, w1, inp, ids, which, True)
            f.flux_gemm_stream_k(True, spin=1)
            d = _run_pair(wl, w2, w1, inp, ids, which, True)
            f.flux_gemm_stream_k(True, spin=0)
            x0 = np.concatenate([inp["x_img"], inp["x_txt"]], axis=1)
            for name, o in (("whole tiles", c), ("poll limit 1", d)):
                # compare the block's update (output - input): every element of it
                # went through the linears
                assert_close(a - x0, o - x0, f"{which}: stream-K vs {name}", max_abs=1e-2, rel=1e-3)
    finally:
        f.flux_gemm_stream_k(prev, spin=0)
