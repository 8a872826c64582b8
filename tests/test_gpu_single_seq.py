"""GPU parity of the sequential single block (flux_single_seq_fwd: "Flux
architecture deep dive", Model components / Flux single block, in the form
written out step by step) against oracle.single_block_sequential.

Tolerances as for the other blocks: bf16 and fp32 workloads max-abs <= 3e-2
and relative L2 <= 1e-2; E4M3 linears relative L2 <= 5e-2 under the
delayed-scaling protocol, the oracle taking the scales the GPU used.
"""
import numpy as np
import pytest

import oracle as O
from oracle import fp8_oracle as Q
from flow_matching_diffusion_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2, REL_L2_FP8 = 3e-2, 1e-2, 5e-2


def _say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from flow_matching_diffusion_amd import flux
    flux.lib()
    torch.cuda.set_device(0)


def _dev(a, bf16=False):
    from flow_matching_diffusion_amd.model import device_array
    return device_array(a, bf16)


def _errs(g, o):
    d = np.asarray(g, np.float64) - o
    return float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(o))


def _fixture(wl):
    return synth.single_seq_block_weights(wl, 2), synth.block_inputs(wl), synth.joint_ids(wl)


def _run(wl, w, inp, ids, weights_f16=False, n_fwd=1):
    """n_fwd forwards of the block from the same input (fp8: weight cast before
    and scale update after each but the last); returns the last output and the
    stack."""
    from flow_matching_diffusion_amd.model import BlockStack
    stack = BlockStack(wl, [], [w], weights_f16=weights_f16)
    assert stack.single_seq == [True]
    x0 = np.concatenate([inp["x_img"], inp["x_txt"]], axis=1)
    vec = _dev(inp["vec"])
    rope = stack.rope_table(_dev(ids))
    for f in range(n_fwd):
        x = _dev(x0)
        if stack.fp8:
            stack.fp8_cast_weights()
        stack.single_fwd(0, x, vec, rope)
        if stack.fp8 and f < n_fwd - 1:
            stack.fp8_update()
    torch.cuda.synchronize()
    return x.cpu().numpy(), stack


def _check(wl, w, inp, ids, g, rows=None, lin=None, rel=REL_L2, max_abs=MAX_ABS):
    ang = O.rope_angles(ids, wl.axes_dim, wl.theta)
    x = np.concatenate([inp["x_img"], inp["x_txt"]], axis=1)
    sel = np.arange(wl.seq) if rows is None else rows
    o = O.single_block_sequential(x, inp["vec"], ang, w, wl.heads, wl.eps, rows=sel, lin=lin)
    a, r = _errs(g[:, sel], o)
    print(f"    single (sequential): max_abs={a:.3e} rel_l2={r:.3e}", flush=True)
    assert np.isfinite(g).all()
    assert r <= rel and (max_abs is None or a <= max_abs), (a, r)


SMALL = {
    "tiny_fp32": synth.WORKLOADS["tiny_fp32"],
    "tiny_bf16": synth.custom_workload("tiny_bf16", base="tiny_fp32", precision="bf16"),
    "ragged_bf16": synth.custom_workload("ragged_bf16", base="tiny_fp32", precision="bf16", batch=2, img_h=7, img_w=9,
                                         l_txt=11, hidden=256, heads=2, head_dim=128, mlp_hidden=512,
                                         axes_dim=(16, 56, 56)),
    "ragged_fp32": synth.custom_workload("ragged_fp32", base="tiny_fp32", batch=2, img_h=5, img_w=13, l_txt=3),
    "img_only_bf16": synth.custom_workload("img_only_bf16", base="tiny_fp32", precision="bf16", l_txt=0),
}
CASES = [(n, False) for n in SMALL] + [(n, True) for n in SMALL if SMALL[n].precision == "bf16"]


@pytest.mark.parametrize("name,wf16", CASES)
def test_single_seq_small(name, wf16):
    wl = SMALL[name]
    _say(f"sequential single block {name} weights_f16={wf16}")
    w, inp, ids = _fixture(wl)
    g, _ = _run(wl, w, inp, ids, wf16)
    _check(wl, w, inp, ids, g)


def test_single_seq_adaln_zero_identity_and_determinism():
    wl = SMALL["ragged_bf16"]
    _say("sequential single block adaLN-zero identity / determinism")
    w, inp, ids = _fixture(wl)
    x0 = np.concatenate([inp["x_img"], inp["x_txt"]], axis=1)
    wz = dict(w, **{"mod.w": np.zeros_like(w["mod.w"]), "mod.b": np.zeros_like(w["mod.b"])})
    assert np.array_equal(_run(wl, wz, inp, ids)[0], x0)
    g1, _ = _run(wl, w, inp, ids)
    g2, _ = _run(wl, w, inp, ids)
    assert np.array_equal(g1, g2)


@pytest.mark.slow
def test_single_seq_flux12b_shapes_sampled():
    wl = synth.WORKLOADS["flux12b_blocks"]
    _say("sequential single block flux12b_blocks (L=4608) sampled rows, fp16-held linear weights")
    w, inp, ids = _fixture(wl)
    g, _ = _run(wl, w, inp, ids, True)
    rng = np.random.default_rng(7)
    rows = np.unique(np.r_[rng.choice(wl.seq, 32, replace=False), 0, wl.l_img - 1, wl.l_img, wl.seq - 1])
    _check(wl, w, inp, ids, g, rows=rows)


FP8_SMALL = synth.custom_workload("ragged_fp8", base="tiny_fp32", precision="fp8", batch=2, img_h=7, img_w=9,
                                  l_txt=11, hidden=256, heads=2, head_dim=128, mlp_hidden=512,
                                  axes_dim=(16, 56, 56))


def test_single_seq_fp8_delayed_scaling():
    wl = FP8_SMALL
    _say("fp8 sequential single block ragged (B=2, 63 + 11 tokens), delayed scaling")
    w, inp, ids = _fixture(wl)
    g, stack = _run(wl, w, inp, ids, n_fwd=3)
    recs = stack.fp8_records()
    assert len(recs) == 8
    sc = {n: (recs[2 * li]["scale"], recs[2 * li + 1]["scale"]) for li, n in enumerate(Q.TOKEN_LINEARS_DOUBLE)}
    for n, (_, s_w) in sc.items():       # weight scales are bitwise fp32(448 / max|W|)
        assert s_w == float(np.float32(448.0) / np.float32(np.abs(w[n + ".w"]).max())), n
    seen = {}
    _check(wl, w, inp, ids, g, lin=Q.fp8_linears(sc, seen), rel=REL_L2_FP8, max_abs=None)
    for n in sc:                          # activation scales track the oracle's own amax
        ref = 448.0 / seen[n]
        assert abs(sc[n][0] - ref) <= 1e-2 * ref, (n, sc[n][0], ref)
