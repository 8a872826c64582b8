"""GPU parity of the training path (the block backward under the
rectified-flow objective) against oracle/backward_oracle.py:

  * flux_attention_fwd_train / flux_attention_bwd: the log-sum-exp and dq, dk,
    dv of softmax attention on ragged lengths;
  * flux_single_fwd_train + flux_single_bwd and flux_block_fwd_train +
    flux_block_bwd: the block output, the input and vec gradients and every
    parameter gradient, on ragged image / text lengths with B = 2;
  * repeatability: two backward passes give the same bits;
  * the Flux-12B block shapes (L = 4608, D = 3072, F = 12288): the training
    forward on sampled token rows (max |error| <= 3e-2, relative L2 <= 1e-2,
    the forward's bar) and the gradients (full biases, norm scales and vec;
    sampled rows of the input and weight gradients) against the values that
    tests/golden/make_flux12b_train_golden.py wrote from oracle/ alone.

Tolerances.  The training forward's linears take fp16 activations (relative
rounding <= 2^-11); the backward rounds every GEMM operand to bf16 (8
significant bits, relative error <= 2^-9), including the recomputed
probabilities, the score gradients and the output gradients that feed the
weight-gradient GEMMs; each gradient passes through a handful of such
roundings, whose errors are independent, so the relative L2 error is a
small multiple of 2^-9 ~ 2e-3.  The bar is relative L2 <= 1e-2 and max |error| <= 3e-2 of the
largest |reference| value of the same tensor.
"""
import numpy as np
import pytest

import oracle as O
from oracle import backward_oracle as G
from flow_matching_diffusion_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL_L2, MAX_REL = 1e-2, 3e-2


def _say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from flow_matching_diffusion_amd import flux
    flux.lib()
    torch.cuda.set_device(0)


def F():
    from flow_matching_diffusion_amd import flux
    return flux


def _dev(a, bf16=False):
    from flow_matching_diffusion_amd.model import device_array
    return device_array(a, bf16)


def _close(got, ref, what, rel=REL_L2, max_rel=MAX_REL):
    g = np.asarray(got, np.float64)
    d = g - ref
    scale = float(np.abs(ref).max())
    r = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    m = float(np.abs(d).max()) / max(scale, 1e-300)
    print(f"    {what}: rel_l2={r:.2e} max_err/max={m:.2e} (max |ref| {scale:.2e})", flush=True)
    assert np.isfinite(g).all(), what
    assert r <= rel and m <= max_rel, (what, r, m)


def _ws(nbytes):
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")


# ------------------------------- attention ------------------------------- #
@pytest.mark.parametrize("B,L,H", [(1, 80, 2), (2, 333, 2), (1, 1000, 3)])
def test_attention_bwd(B, L, H):
    _say(f"attention backward B={B} L={L} H={H} Dh=128")
    rng = np.random.default_rng(L * 3 + H)
    D = H * 128
    q = synth.round_to_bf16(0.25 * rng.standard_normal((B, L, D)).astype(np.float32))
    k = synth.round_to_bf16(rng.standard_normal((B, L, D)).astype(np.float32))
    v = synth.round_to_bf16(rng.standard_normal((B, L, D)).astype(np.float32))
    do = synth.round_to_bf16(rng.standard_normal((B, L, D)).astype(np.float32))
    f = F()
    qd, kd, vd, dod = _dev(q, True), _dev(k, True), _dev(v, True), _dev(do, True)
    Lp = (L + 255) // 256 * 256
    o = torch.empty((B, L, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, Lp), -1.0, dtype=torch.float32, device="cuda")
    wsb = f.flux_attention_train_workspace_bytes(B, L, H)
    ws = _ws(wsb)
    f.flux_attention_fwd_train(B, L, H, qd, kd, vd, D, o, D, lse, ws, wsb)
    dqkv = torch.empty((B, L, 3 * D), dtype=torch.bfloat16, device="cuda")
    f.flux_attention_bwd(B, L, H, qd, kd, vd, D, o, dod, D, lse, dqkv, ws, wsb)
    torch.cuda.synchronize()
    hd = lambda a: a.reshape(B, L, H, 128)
    # log-sum-exp of the scaled scores, log2 domain; +inf on the padded rows
    s = np.einsum("blhd,bmhd->bhlm", hd(q).astype(np.float64), hd(k).astype(np.float64)) / np.sqrt(128.0)
    mx = s.max(axis=-1, keepdims=True)
    ref_lse = (np.log(np.exp(s - mx).sum(axis=-1)) + mx[..., 0]) / np.log(2.0)
    got_lse = lse.cpu().numpy()
    np.testing.assert_allclose(got_lse[:, :, :L], ref_lse, atol=2e-3, rtol=0)
    assert np.all(np.isinf(got_lse[:, :, L:]) & (got_lse[:, :, L:] > 0))
    _close(o.float().cpu().numpy(), O.attention(hd(q), hd(k), hd(v)), "o")
    dq, dk, dv = G.attention_vjp(hd(q), hd(k), hd(v), do)
    g = dqkv.float().cpu().numpy()
    _close(g[..., :D], dq.reshape(B, L, D), "dq")
    _close(g[..., D:2 * D], dk.reshape(B, L, D), "dk")
    _close(g[..., 2 * D:], dv.reshape(B, L, D), "dv")


# -------------------------------- blocks --------------------------------- #
WL = {
    "ragged": synth.custom_workload("bwd_ragged", base="tiny_fp32", precision="bf16", batch=2, img_h=7, img_w=9,
                                    l_txt=11, hidden=256, heads=2, head_dim=128, mlp_hidden=512,
                                    axes_dim=(16, 56, 56)),
    "img_only": synth.custom_workload("bwd_img_only", base="tiny_fp32", precision="bf16", batch=1, img_h=8, img_w=10,
                                      l_txt=0, hidden=256, heads=2, head_dim=128, mlp_hidden=512,
                                      axes_dim=(16, 56, 56)),
    "wide": synth.custom_workload("bwd_wide", base="tiny_fp32", precision="bf16", batch=1, img_h=16, img_w=16,
                                  l_txt=40, hidden=512, heads=4, head_dim=128, mlp_hidden=1024,
                                  axes_dim=(16, 56, 56)),
}


def _setup(wl, seed):
    from flow_matching_diffusion_amd.model import upload_weights
    inp = synth.block_inputs(wl)
    ids = synth.joint_ids(wl)
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal((wl.batch, wl.seq, wl.hidden)).astype(np.float32)
    rope = torch.empty((wl.batch, wl.seq, 64, 2), dtype=torch.float32, device="cuda")
    F().flux_rope_table(_dev(ids), wl.batch, wl.seq, wl.axes_dim, wl.theta, rope)
    ang = O.rope_angles(ids, wl.axes_dim, wl.theta)
    return inp, dout, rope, ang, upload_weights


def _grad_buffers(w):
    return {k: torch.full(np.shape(v), float("nan"), dtype=torch.float32, device="cuda") for k, v in w.items()}


def _run_single(wl, w, inp, dout, rope, upload):
    f = F()
    dims = f.dims_for(wl)
    wd = upload(w, True)
    x = _dev(np.concatenate([inp["x_img"], inp["x_txt"]], axis=1))
    vec = _dev(inp["vec"])
    L, D = wl.seq, wl.hidden
    sb = f.flux_train_saved_bytes(dims, 1)
    saved = _ws(sb)
    f.flux_single_fwd_train(dims, f.single_weights(wd), x, L * D, vec, rope, saved, sb)
    dx = _dev(dout)
    dvec = torch.zeros_like(vec)
    grads = _grad_buffers(w)
    wsb = f.flux_bwd_workspace_bytes(dims, 1)
    ws = _ws(wsb)
    f.flux_single_bwd(dims, f.single_weights(wd), dx, L * D, vec, rope, saved, sb, f.single_grads(grads), dvec, ws, wsb)
    torch.cuda.synchronize()
    return x.cpu().numpy(), dx.cpu().numpy(), dvec.cpu().numpy(), {k: v.cpu().numpy() for k, v in grads.items()}


@pytest.mark.parametrize("name", ["ragged", "img_only", "wide"])
def test_single_block_backward(name):
    wl = WL[name]
    _say(f"single block forward-train + backward {name} (B={wl.batch}, L={wl.l_img}+{wl.l_txt}, D={wl.hidden})")
    w = synth.single_block_weights(wl, 1)
    inp, dout, rope, ang, upload = _setup(wl, 5)
    x0 = np.concatenate([inp["x_img"], inp["x_txt"]], axis=1)
    out, dx, dvec, g = _run_single(wl, w, inp, dout, rope, upload)
    _close(out, O.single_block(x0, inp["vec"], ang, w, wl.heads, wl.eps), "forward output")
    rdx, rdvec, rg = G.single_block_vjp(x0, inp["vec"], ang, w, wl.heads, wl.eps, dout)
    _close(dx, rdx, "dx")
    _close(dvec, rdvec, "dvec")
    for n in sorted(w):
        _close(g[n], rg[n], "d " + n)


def _run_double(wl, w, inp, dout, rope, upload):
    f = F()
    dims = f.dims_for(wl)
    wd = upload(w, True)
    L, D, Li = wl.seq, wl.hidden, wl.l_img
    x = _dev(np.concatenate([inp["x_img"], inp["x_txt"]], axis=1))   # joint buffer, streams as halves
    vec = _dev(inp["vec"])
    sb = f.flux_train_saved_bytes(dims, 0)
    saved = _ws(sb)
    iw, tw = f.stream_weights(wd, "img"), f.stream_weights(wd, "txt")
    txt_ptr = x.data_ptr() + Li * D * 4
    f.flux_block_fwd_train(dims, iw, tw, x, L * D, txt_ptr, L * D, vec, rope, saved, sb)
    d = _dev(dout)
    dvec = torch.zeros_like(vec)
    grads = _grad_buffers(w)
    wsb = f.flux_bwd_workspace_bytes(dims, 0)
    ws = _ws(wsb)
    f.flux_block_bwd(dims, iw, tw, d, L * D, d.data_ptr() + Li * D * 4, L * D, vec, rope, saved, sb,
                     f.stream_grads(grads, "img"), f.stream_grads(grads, "txt"), dvec, ws, wsb)
    torch.cuda.synchronize()
    return x.cpu().numpy(), d.cpu().numpy(), dvec.cpu().numpy(), {k: v.cpu().numpy() for k, v in grads.items()}


@pytest.mark.parametrize("name", ["ragged", "wide"])
def test_double_block_backward(name):
    wl = WL[name]
    _say(f"double block forward-train + backward {name} (B={wl.batch}, L={wl.l_img}+{wl.l_txt}, D={wl.hidden})")
    w = synth.double_block_weights(wl, 0)
    inp, dout, rope, ang, upload = _setup(wl, 6)
    Li = wl.l_img
    out, d, dvec, g = _run_double(wl, w, inp, dout, rope, upload)
    oi, ot = O.double_block(inp["x_img"], inp["x_txt"], inp["vec"], ang, w, wl.heads, wl.eps)
    _close(out, np.concatenate([oi, ot], axis=1), "forward output")
    rdi, rdt, rdvec, rg = G.double_block_vjp(inp["x_img"], inp["x_txt"], inp["vec"], ang, w, wl.heads, wl.eps,
                                             dout[:, :Li], dout[:, Li:])
    _close(d[:, :Li], rdi, "dx_img")
    _close(d[:, Li:], rdt, "dx_txt")
    _close(dvec, rdvec, "dvec")
    for n in sorted(w):
        _close(g[n], rg[n], "d " + n)


def test_backward_repeatable():
    wl = WL["ragged"]
    _say("double and single block backward: two runs bit-identical")
    inp, dout, rope, ang, upload = _setup(wl, 7)
    w2, w1 = synth.double_block_weights(wl, 0), synth.single_block_weights(wl, 1)
    a = _run_double(wl, w2, inp, dout, rope, upload)
    b = _run_double(wl, w2, inp, dout, rope, upload)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)
    for k in a[3]:
        assert np.array_equal(a[3][k], b[3][k]), k
    a = _run_single(wl, w1, inp, dout, rope, upload)
    b = _run_single(wl, w1, inp, dout, rope, upload)
    for k in a[3]:
        assert np.array_equal(a[3][k], b[3][k]), k
    assert np.array_equal(a[1], b[1])


def test_train_rejects_unsupported():
    f = F()
    wl = WL["ragged"]
    d = f.dims_for(wl)
    d.head_dim, d.heads = 64, 4
    assert f.flux_train_saved_bytes(d, 0) == 0
    d = f.dims_for(synth.custom_workload("bwd_f32", base="tiny_fp32", hidden=256, heads=2, head_dim=128,
                                         mlp_hidden=512, axes_dim=(16, 56, 56)))
    assert f.flux_bwd_workspace_bytes(d, 1) == 0


# ------------------------- full Flux-12B block shapes ------------------------- #
def _pair_at_full_size(zero_mod):
    from flow_matching_diffusion_amd.model import BlockPairTrainer
    wl = synth.WORKLOADS["flux12b_blocks"]
    B, L, D = wl.batch, wl.seq, wl.hidden
    tr = BlockPairTrainer(wl, synth.device_block_weights(wl, 0, "double", zero_mod=zero_mod),
                          synth.device_block_weights(wl, 1, "single", zero_mod=zero_mod))
    g = torch.Generator(device="cuda").manual_seed(99)
    x_in = torch.randn((B, L, D), generator=g, device="cuda")
    d_out = torch.randn((B, L, D), generator=g, device="cuda")
    vec = torch.randn((B, D), generator=g, device="cuda")
    rope = torch.empty((B, L, 64, 2), dtype=torch.float32, device="cuda")
    F().flux_rope_table(torch.from_numpy(synth.joint_ids(wl)).cuda(), B, L, wl.axes_dim, wl.theta, rope)

    def run():
        x, d, dvec = x_in.clone(), d_out.clone(), torch.zeros_like(vec)
        tr.forward(x, vec, rope)
        tr.backward(d, vec, rope, dvec)
        torch.cuda.synchronize()
        return x, d, dvec, {k: v.clone() for k, v in {**tr.g2, **{"s_" + k: v for k, v in tr.g1.items()}}.items()}

    return tr, x_in, d_out, run


def test_pair_backward_flux12b_adaln_zero_identity():
    # every shift, scale and gate is zero: both blocks are the identity, so the
    # input gradient equals the output gradient bit for bit, every gradient
    # below the gates is exactly zero, and so is the vec gradient (zero
    # modulation weights); the gate rows of the modulation bias gradient are
    # the column sums of y * dout and do not vanish
    _say("block pair training forward + backward, Flux-12B shapes (L=4608), adaLN-zero")
    tr, x_in, d_out, run = _pair_at_full_size(True)
    x, d, dvec, g = run()
    assert torch.equal(x, x_in)
    assert torch.equal(d, d_out)
    assert bool((dvec == 0).all())
    D = tr.wl.hidden
    for k, v in g.items():
        if k.endswith("mod.w") or k.endswith("mod.b"):
            continue
        assert bool((v == 0).all()), k
    for k in ("img_mod.b", "txt_mod.b"):
        gate_rows = torch.cat([g[k][2 * D:3 * D], g[k][5 * D:]])
        assert bool(torch.isfinite(g[k]).all()) and float(gate_rows.abs().max()) > 0, k
        assert bool((g[k][:2 * D] == 0).all()), k
    assert float(g["s_mod.b"][2 * D:].abs().max()) > 0 and bool((g["s_mod.b"][:2 * D] == 0).all())


def test_pair_backward_flux12b_repeatable_and_finite():
    _say("block pair training forward + backward, Flux-12B shapes (L=4608): two runs bit-identical, finite")
    tr, x_in, d_out, run = _pair_at_full_size(False)
    a = run()
    b = run()
    for u, v in zip(a[:3], b[:3]):
        assert torch.equal(u, v)
        assert bool(torch.isfinite(u).all())
    for k in a[3]:
        assert torch.equal(a[3][k], b[3][k]), k
        assert bool(torch.isfinite(a[3][k]).all()) and float(a[3][k].abs().max()) > 0, k


# ------------------------------ whole training step ------------------------------ #
STEP_WL = {
    # text and pooled-vector embedders present, ragged text, B = 2
    "embedders": synth.custom_workload("step_embedders", base="flux535m", batch=2, hidden=256, heads=2, head_dim=128,
                                       mlp_hidden=512, img_h=6, img_w=8, l_txt=11, context_dim=128, vec_in_dim=64),
    # text at hidden width, no pooled vector (the block-pair bench's model)
    "plain": synth.custom_workload("step_plain", base="flux535m", batch=1, hidden=256, heads=2, head_dim=128,
                                   mlp_hidden=512, img_h=8, img_w=8, l_txt=16, context_dim=None, vec_in_dim=None),
    # all embedders and the guidance embedding (Linear 1 -> D of per-sample guidance values)
    "guidance": synth.custom_workload("step_guidance", base="flux535m", batch=3, hidden=256, heads=2, head_dim=128,
                                      mlp_hidden=512, img_h=4, img_w=8, l_txt=7, context_dim=128, vec_in_dim=64),
}


@pytest.mark.parametrize("name", list(STEP_WL))
def test_flux_train_step(name):
    from flow_matching_diffusion_amd.model import FluxTrainer
    wl = STEP_WL[name]
    _say(f"whole training step {name}: noise, embeddings, double + single block, head, MSE, backward")
    with_g = name == "guidance"
    emb = synth.embed_weights(wl, guidance=with_g)
    w2, w1 = synth.double_block_weights(wl, 0), synth.single_block_weights(wl, 1)
    mi = synth.model_inputs(wl)
    gv = np.linspace(1.0, 5.0, wl.batch).astype(np.float32) if with_g else None
    tr = FluxTrainer(wl, emb, [w2], [w1])
    y = _dev(mi["y"]) if "y" in mi else None
    # the text is bf16 on the device (the element type of the bf16 path, with or
    # without txt_in); the oracle takes the same bf16 values
    txt = synth.round_to_bf16(mi["txt"])
    loss = tr.step(_dev(mi["z0"]), _dev(mi["z1"]), _dev(mi["t"]), _dev(txt, True), y,
                   _dev(mi["ids"]), guidance=_dev(gv) if with_g else None)
    torch.cuda.synchronize()
    ref_loss, g_emb, g2, g1 = G.flux_train_vjp(mi["z0"], mi["z1"], mi["t"], txt, mi.get("y"), mi["ids"], emb, [w2],
                                               [w1], wl.heads, wl.axes_dim, wl.theta, wl.eps, wl.model_channels,
                                               guidance=gv)
    got = float(loss.item())
    print(f"    loss: gpu {got:.6f} oracle {ref_loss:.6f}", flush=True)
    assert abs(got - ref_loss) <= 1e-2 * ref_loss
    assert set(tr.grads) == set(g_emb)
    for n in sorted(g_emb):
        _close(tr.grads[n].cpu().numpy(), g_emb[n], "d " + n)
    for n in sorted(w2):
        _close(tr.g_double[0][n].cpu().numpy(), g2[0][n], "d double " + n)
    for n in sorted(w1):
        _close(tr.g_single[0][n].cpu().numpy(), g1[0][n], "d single " + n)


@pytest.mark.parametrize("name", ["ragged", "wide"])
def test_single_seq_block_backward(name):
    wl = WL[name]
    _say(f"sequential single block forward-train + backward {name} (B={wl.batch}, L={wl.seq}, D={wl.hidden})")
    from flow_matching_diffusion_amd.model import upload_weights
    f = F()
    w = synth.single_seq_block_weights(wl, 2)
    inp, dout, rope, ang, _ = _setup(wl, 8)
    x0 = np.concatenate([inp["x_img"], inp["x_txt"]], axis=1)
    dims = f.dims_for(wl)
    wd = upload_weights(w, True)
    sw = f.stream_weights(wd, None)
    L, D = wl.seq, wl.hidden
    x, vec = _dev(x0), _dev(inp["vec"])
    sb = f.flux_train_saved_bytes(dims, 2)
    saved = _ws(sb)
    f.flux_single_seq_fwd_train(dims, sw, x, L * D, vec, rope, saved, sb)
    d, dvec = _dev(dout), torch.zeros_like(vec)
    grads = _grad_buffers(w)
    wsb = f.flux_bwd_workspace_bytes(dims, 2)
    ws = _ws(wsb)
    f.flux_single_seq_bwd(dims, sw, d, L * D, vec, rope, saved, sb, f.stream_grads(grads, None), dvec, ws, wsb)
    torch.cuda.synchronize()
    _close(x.cpu().numpy(), O.single_block_sequential(x0, inp["vec"], ang, w, wl.heads, wl.eps), "forward output")
    rdx, rdvec, rg = G.single_block_sequential_vjp(x0, inp["vec"], ang, w, wl.heads, wl.eps, dout)
    _close(d.cpu().numpy(), rdx, "dx")
    _close(dvec.cpu().numpy(), rdvec, "dvec")
    for n in sorted(w):
        _close(grads[n].cpu().numpy(), rg[n], "d " + n)


# ------------- full Flux-12B block shapes against the oracle (sampled) ------------- #
def _golden_train():
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "flux12b_train_expected.npz")
    return np.load(path)


def _d_out(wl):
    # the output gradient tests/golden/make_flux12b_train_golden.py used
    return synth.normal((wl.batch, wl.seq, wl.hidden), 1.0, wl.config_id, 0, "d_out", False)


def _check_train_golden(prefix, exp, tok, out, dx, dvec, g):
    ref = exp[prefix + "out"].astype(np.float64)
    got = out[0, tok].astype(np.float64)
    a = float(np.abs(got - ref).max())
    r = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"    {prefix} training forward, sampled rows: max_abs={a:.3e} rel_l2={r:.3e}", flush=True)
    assert a <= 3e-2 and r <= 1e-2, (prefix, a, r)
    _close(dx[0, tok], exp[prefix + "dx"], prefix + " dx (sampled rows)")
    _close(dvec, exp[prefix + "dvec"], prefix + " dvec")
    for key in exp.files:
        if not key.startswith(prefix + "grad:"):
            continue
        name = key[len(prefix + "grad:"):]
        rows_key = prefix + "rows:" + name
        gv = g[name][exp[rows_key]] if rows_key in exp.files else g[name]
        _close(gv, exp[key], f"{prefix} d {name}" + (" (sampled rows)" if rows_key in exp.files else ""))


def test_double_block_training_flux12b_against_oracle_golden():
    wl = synth.WORKLOADS["flux12b_blocks"]
    _say("double block training forward + backward at Flux-12B shapes (L=4608, D=3072) against the oracle")
    exp = _golden_train()
    tok = exp["token_rows"]
    inp, _, rope, _, upload = _setup(wl, 0)
    out, d, dvec, g = _run_double(wl, synth.double_block_weights(wl, 0), inp, _d_out(wl), rope, upload)
    _check_train_golden("double:", exp, tok, out, d, dvec, g)


def test_single_block_training_flux12b_against_oracle_golden():
    wl = synth.WORKLOADS["flux12b_blocks"]
    _say("single block training forward + backward at Flux-12B shapes (L=4608, D=3072) against the oracle")
    exp = _golden_train()
    tok = exp["token_rows"]
    inp, _, rope, _, upload = _setup(wl, 0)
    out, dx, dvec, g = _run_single(wl, synth.single_block_weights(wl, 1), inp, _d_out(wl), rope, upload)
    _check_train_golden("single:", exp, tok, out, dx, dvec, g)
