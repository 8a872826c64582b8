"""The whole forward + loss captured in a HIP graph (torch.cuda.CUDAGraph on
the library's stream argument) replays bit-identically to the eager step:
every launch of the library is graph-capturable (no allocation, no memset,
no synchronisation inside an entry point).  Each replay is checked against
the eager result, with eager work and synchronisations between replays."""
import numpy as np
import pytest

from flow_matching_diffusion_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from flow_matching_diffusion_amd import flux
    flux.lib()
    torch.cuda.set_device(0)


@pytest.mark.parametrize("name", ["tiny_bf16", "flux535m"])
def test_forward_loss_graph_replays_match_eager(name):
    from flow_matching_diffusion_amd.model import FluxModel, device_array
    wl = synth.WORKLOADS.get(name) or synth.custom_workload(name, base="tiny_fp32", precision="bf16")
    print(f"[case] graph capture of forward + loss, {wl.name}", flush=True)
    emb = synth.embed_weights(wl)
    m = FluxModel(wl, emb, [synth.double_block_weights(wl, 0)], [synth.single_block_weights(wl, 1)],
                  weights_f16=True)
    mi = synth.model_inputs(wl)
    dev = lambda a, bf=False: device_array(a, bf)
    z0, z1, t, ids = dev(mi["z0"]), dev(mi["z1"]), dev(mi["t"]), dev(mi["ids"])
    txt = dev(mi["txt"], True)
    y = dev(mi["y"]) if "y" in mi else None
    out = {}
    m.forward_loss(z0, z1, t, txt, y, ids, out)
    torch.cuda.synchronize()
    ref_v, ref_l = out["v_pred"].clone(), out["loss"].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        m.forward_loss(z0, z1, t, txt, y, ids, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.forward_loss(z0, z1, t, txt, y, ids, out)
    torch.cuda.synchronize()
    for r in range(4):
        out["v_pred"].fill_(float("nan"))
        out["loss"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out["v_pred"], ref_v), f"replay {r}: v_pred differs"
        assert torch.equal(out["loss"], ref_l), f"replay {r}: loss differs"
        m.forward_loss(z0, z1, t, txt, y, ids, out)      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out["v_pred"], ref_v)
    assert np.isfinite(float(ref_l.item()))
