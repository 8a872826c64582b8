"""The full Flux-12B-shaped forward on one GPU: 19 double + 38 single blocks,
batch 2, 512 text + 64x64 image tokens, hidden 3072, logit-normal t, rectified
flow noising and velocity MSE ("Flux architecture deep dive", Model variants:
12B = 19 joint + 38 single layers; Data flow / Complete forward pass).

  * end to end against the fp64 oracle: the block weights are drawn on the
    host from the same seeded streams the oracle used, and v_pred (every one
    of its 524,288 elements) and the loss are compared with the values that
    tests/golden/make_flux12b_full_golden.py wrote from oracle/ alone
    (bf16 bounds: max |error| <= 3e-2 and relative L2 <= 1e-2; loss within
    1e-2 relative);
  * adaLN-zero: with every modulation weight and bias zero, each block's
    shifts, scales and gates are 0 and the block is the identity, so v_pred
    is the oracle's input embedding + output head of the same inputs; the
    forward is deterministic (two runs, bit-identical v_pred and loss).
"""
import json
import os

import numpy as np
import pytest

import oracle as O
from flow_matching_diffusion_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2 = 3e-2, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from flow_matching_diffusion_amd import flux
    flux.lib()
    torch.cuda.set_device(0)


def _model(wl, emb, zero_mod):
    from flow_matching_diffusion_amd.model import FluxModel
    dws = [synth.device_block_weights(wl, i, "double", zero_mod=zero_mod) for i in range(wl.n_double)]
    sws = [synth.device_block_weights(wl, wl.n_double + i, "single", zero_mod=zero_mod) for i in range(wl.n_single)]
    m = FluxModel(wl, emb, dws, sws, weights_f16=True)
    del dws, sws
    return m


def _run(m, mi):
    from flow_matching_diffusion_amd.model import device_array
    dev = lambda a, bf=False: device_array(a, bf)
    out = m.forward_loss(dev(mi["z0"]), dev(mi["z1"]), dev(mi["t"]), dev(mi["txt"], True), dev(mi["y"]),
                         dev(mi["ids"]))
    torch.cuda.synchronize()
    return out["v_pred"].cpu().numpy(), float(out["loss"].item())


def test_flux12b_full_forward_adaln_zero_and_determinism():
    wl = synth.WORKLOADS["flux12b_full"]
    print(f"[case] {wl.name}: {wl.n_double} double + {wl.n_single} single blocks, B={wl.batch}, L={wl.seq}",
          flush=True)
    emb = synth.embed_weights(wl)
    mi = synth.model_inputs(wl)
    m = _model(wl, emb, zero_mod=True)
    v1, l1 = _run(m, mi)
    v2, l2 = _run(m, mi)
    assert np.array_equal(v1, v2) and l1 == l2, "forward is not bitwise repeatable"
    # blocks are the identity: v_pred = head(embed(z_t)); no block ever mixes text into image rows
    zt, _ = O.rf_noise(mi["z0"], mi["z1"], mi["t"])
    ref = O.flux_forward(zt, mi["txt"], mi["y"], mi["t"], mi["ids"], emb, [], [], wl.heads, wl.axes_dim,
                         wl.theta, wl.eps, wl.model_channels)
    d = v1.astype(np.float64) - ref
    a, r = float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref))
    print(f"    v_pred (adaLN-zero stack): max_abs={a:.3e} rel_l2={r:.3e}", flush=True)
    assert a <= MAX_ABS and r <= REL_L2, (a, r)
    loss, _ = O.rf_loss(ref, mi["z0"], mi["z1"])
    print(f"    loss gpu={l1:.6f} oracle={loss:.6f}", flush=True)
    assert abs(l1 - loss) <= 1e-2 * abs(loss)
    del m
    torch.cuda.empty_cache()


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_flux12b_full_forward_matches_oracle_end_to_end():
    from flow_matching_diffusion_amd.model import FluxModel, upload_weights
    wl = synth.WORKLOADS["flux12b_full"]
    exp = json.load(open(os.path.join(GOLDEN, "flux12b_full_expected.json")))
    v_ref = np.load(os.path.join(GOLDEN, "flux12b_full_v_pred.npy")).astype(np.float64)
    print(f"[case] {wl.name}: host-drawn weights, end to end against the oracle", flush=True)
    emb = synth.embed_weights(wl)
    mi = synth.model_inputs(wl)
    assert np.allclose(mi["t"], exp["t"], rtol=0, atol=0)
    dws, sws = [], []
    for kind, i, w in synth.iter_block_weights(wl):
        (dws if kind == "double" else sws).append(upload_weights(w, True))
    torch.cuda.synchronize()
    print(f"    uploaded {len(dws)} double + {len(sws)} single blocks", flush=True)
    m = FluxModel(wl, emb, dws, sws, weights_f16=True)
    del dws, sws
    v, loss = _run(m, mi)
    d = v.astype(np.float64) - v_ref
    a, r = float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(v_ref))
    print(f"    v_pred ({v.size} elements): max_abs={a:.3e} rel_l2={r:.3e}", flush=True)
    print(f"    loss gpu={loss:.6f} oracle={exp['loss']:.6f}", flush=True)
    assert np.isfinite(v).all()
    assert a <= MAX_ABS and r <= REL_L2, (a, r)
    assert abs(loss - exp["loss"]) <= 1e-2 * abs(exp["loss"])
    del m
    torch.cuda.empty_cache()
