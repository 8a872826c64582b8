"""Device checks (FLUX_DEBUG_CHECKS / flux_debug_checks): read-only passes
that OR a bit into the device's status word when a timestep is outside
[0, 1] ("Flux model API reference", Common issues: the timestep range) or a
residual, v_pred, loss, velocity or input gradient is not finite.

  * rf_noise_loss: t outside [0, 1] and NaN t set FLUX_DBG_T_RANGE; a
    non-finite v_pred sets FLUX_DBG_NONFINITE_LOSS; valid inputs set nothing;
    with the checks off nothing is set; results are bitwise the same with the
    checks on and off;
  * a whole forward (noise, embeddings, double and single block, head, loss)
    on clean inputs sets nothing; with one infinite latent value the
    residual, velocity and loss bits are set;
  * a whole training step with one infinite latent value also sets the
    input-gradient bit.
"""
import numpy as np
import pytest

from flow_matching_diffusion_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def f():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from flow_matching_diffusion_amd import flux
    flux.lib()
    torch.cuda.set_device(0)
    prev = flux.flux_debug_checks(True)
    flux.flux_debug_status(clear=True)
    yield flux
    flux.flux_debug_checks(prev)
    flux.flux_debug_status(clear=True)


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _dev(a, bf16=False):
    from flow_matching_diffusion_amd.model import device_array
    return device_array(a, bf16)


def _rf(f, z0, z1, t, vp):
    B, n = z0.shape[0], int(np.prod(z0.shape[1:]))
    zt = torch.empty_like(z0)
    loss = torch.empty(1, device="cuda")
    wsb = f.flux_rf_workspace_bytes(B, n)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    f.rf_noise_loss(B, n, z0, z1, t, z_t=zt, v_pred=vp, loss=loss, workspace=ws, workspace_bytes=wsb)
    torch.cuda.synchronize()
    return zt.cpu().numpy(), float(loss.item())


def test_rf_checks(f):
    _say("device checks: rf_noise_loss timestep range and non-finite v_pred")
    rng = np.random.default_rng(5)
    shape = (2, 16, 8, 8)
    z0, z1, vp = (_dev(rng.standard_normal(shape).astype(np.float32)) for _ in range(3))
    good = _dev(np.array([0.0, 1.0], np.float32))
    a = _rf(f, z0, z1, good, vp)
    assert f.flux_debug_status(clear=True) == 0
    _rf(f, z0, z1, _dev(np.array([0.3, 1.5], np.float32)), vp)
    assert f.flux_debug_status(clear=True) == f.FLUX_DBG_T_RANGE
    _rf(f, z0, z1, _dev(np.array([np.nan, 0.5], np.float32)), vp)
    assert f.flux_debug_status(clear=True) & f.FLUX_DBG_T_RANGE
    bad_vp = vp.clone()
    bad_vp.view(-1)[777] = float("inf")
    _rf(f, z0, z1, good, bad_vp)
    assert f.flux_debug_status(clear=True) == f.FLUX_DBG_NONFINITE_LOSS
    # checks off: nothing is recorded, and the results do not depend on the setting
    f.flux_debug_checks(False)
    try:
        b = _rf(f, z0, z1, good, vp)
        _rf(f, z0, z1, _dev(np.array([0.3, 1.5], np.float32)), bad_vp)
        assert f.flux_debug_status(clear=True) == 0
    finally:
        f.flux_debug_checks(True)
    assert np.array_equal(a[0], b[0]) and a[1] == b[1]


def _forward(wl, emb, w2, w1, mi, z0):
    from flow_matching_diffusion_amd.model import FluxModel
    m = FluxModel(wl, emb, [w2], [w1])
    out = m.forward_loss(z0, _dev(mi["z1"]), _dev(mi["t"]), _dev(mi["txt"], True), None, _dev(mi["ids"]))
    torch.cuda.synchronize()
    return out


def test_forward_checks(f):
    wl = synth.custom_workload("debug_bf16", base="tiny_fp32", precision="bf16")
    _say(f"device checks: whole forward + loss on {wl.name}, clean and with one infinite latent value")
    emb = synth.embed_weights(wl)
    w2, w1 = synth.double_block_weights(wl, 0), synth.single_block_weights(wl, 1)
    mi = synth.model_inputs(wl)
    f.flux_debug_status(clear=True)
    out = _forward(wl, emb, w2, w1, mi, _dev(mi["z0"]))
    assert np.isfinite(float(out["loss"].item()))
    assert f.flux_debug_status(clear=True) == 0
    z0 = mi["z0"].copy()
    z0.reshape(-1)[3] = np.inf
    _forward(wl, emb, w2, w1, mi, _dev(z0))
    st = f.flux_debug_status(clear=True)
    want = f.FLUX_DBG_NONFINITE_RESIDUAL | f.FLUX_DBG_NONFINITE_LOSS | f.FLUX_DBG_NONFINITE_OUTPUT
    assert st & want == want and not st & f.FLUX_DBG_T_RANGE, hex(st)


def test_train_step_gradient_check(f):
    from flow_matching_diffusion_amd.model import FluxTrainer
    wl = synth.custom_workload("debug_step", base="flux535m", batch=1, hidden=256, heads=2, head_dim=128,
                               mlp_hidden=512, img_h=8, img_w=8, l_txt=16, context_dim=None, vec_in_dim=None)
    _say(f"device checks: training step on {wl.name}, clean and with one infinite latent value")
    emb = synth.embed_weights(wl)
    w2, w1 = synth.double_block_weights(wl, 0), synth.single_block_weights(wl, 1)
    mi = synth.model_inputs(wl)
    tr = FluxTrainer(wl, emb, [w2], [w1])
    f.flux_debug_status(clear=True)
    tr.step(_dev(mi["z0"]), _dev(mi["z1"]), _dev(mi["t"]), _dev(mi["txt"], True), None, _dev(mi["ids"]))
    torch.cuda.synchronize()
    assert f.flux_debug_status(clear=True) == 0
    z0 = mi["z0"].copy()
    z0.reshape(-1)[5] = np.inf
    tr.step(_dev(z0), _dev(mi["z1"]), _dev(mi["t"]), _dev(mi["txt"], True), None, _dev(mi["ids"]))
    torch.cuda.synchronize()
    st = f.flux_debug_status(clear=True)
    assert st & f.FLUX_DBG_NONFINITE_GRAD and st & f.FLUX_DBG_NONFINITE_RESIDUAL, hex(st)
