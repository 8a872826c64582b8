"""Write the expected output of the full Flux-12B-shaped forward (19 double +
38 single blocks, batch 2, 512 text + 64x64 image tokens, hidden 3072, 24 x
128 heads; "Flux architecture deep dive", Model variants and Data flow /
Complete forward pass) from the fp64 oracle alone.

    python tests/golden/make_flux12b_full_golden.py

Inputs and weights are the seeded synthetic streams of
flow_matching_diffusion_amd.synth (workload "flux12b_full": N(0,1) latents,
noise and text tokens, logit-normal t, N(0, 0.02) weights rounded to bf16,
RMSNorm scales 1 + 0.1 N(0,1)); block weights are drawn one block at a time
(block ids 0..18 double, 19..56 single) and dropped after use.  Nothing here
touches the GPU or the HIP library.  Writes flux12b_full_v_pred.npy (float32
[2, 64, 64, 64]) and flux12b_full_expected.json (the loss and per-sample
losses in fp64).  About half an hour of fp64 BLAS on 8 cores.
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from flow_matching_diffusion_amd import synth  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    wl = synth.WORKLOADS["flux12b_full"]
    emb = synth.embed_weights(wl)
    mi = synth.model_inputs(wl)
    t0 = time.time()

    def blocks(kind, ids):
        for i in ids:
            w = (synth.double_block_weights if kind == "double" else synth.single_block_weights)(wl, i)
            print(f"  {kind} block {i} ({time.time() - t0:.0f} s)", flush=True)
            yield w

    zt, _ = O.rf_noise(mi["z0"], mi["z1"], mi["t"])
    v = O.flux_forward(zt, mi["txt"], mi["y"], mi["t"], mi["ids"], emb,
                       blocks("double", range(wl.n_double)),
                       blocks("single", range(wl.n_double, wl.n_double + wl.n_single)),
                       wl.heads, wl.axes_dim, wl.theta, wl.eps, wl.model_channels)
    loss, per = O.rf_loss(v, mi["z0"], mi["z1"])
    np.save(os.path.join(HERE, "flux12b_full_v_pred.npy"), v.astype(np.float32))
    rec = {
        "what": "fp64 oracle of the full Flux-12B-shaped forward + velocity MSE on the seeded synthetic inputs",
        "source": "Flux architecture deep dive: Model variants (12B = 19 joint + 38 single layers), "
                  "Data flow / Complete forward pass, Flow matching objective",
        "workload": wl.name, "batch": wl.batch, "l_txt": wl.l_txt, "l_img": wl.l_img, "hidden": wl.hidden,
        "n_double": wl.n_double, "n_single": wl.n_single, "base_seed": synth.BASE_SEED,
        "block_ids": "double 0..18, single 19..56",
        "t": [float(x) for x in mi["t"]],
        "loss": float(loss), "loss_per_sample": [float(x) for x in per],
        "v_pred_rms": float(np.sqrt((v * v).mean())), "v_pred_max_abs": float(np.abs(v).max()),
        "script": "tests/golden/make_flux12b_full_golden.py", "oracle_seconds": round(time.time() - t0, 1),
    }
    with open(os.path.join(HERE, "flux12b_full_expected.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
