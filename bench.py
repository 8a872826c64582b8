#!/usr/bin/env python3
"""Throughput of the Flux MMDiT block forward under rectified-flow training on
one MI355X, through the libflux C ABI.

One step = the whole hot path over one synthetic batch at the Flux-12B block
shapes (batch 1, 512 text + 64x64 image tokens = 4608 joint tokens, hidden
3072, 24 x 128 heads, MLP 12288, bf16 operands with fp32 accumulation):
rf noising of the [1, 64, 64, 64] latents -> image embedding + conditioning
vector -> one double block -> one single block -> output head -> velocity
MSE.  Inputs and weights (N(0, 0.02)) are resident in HBM before timing.

Prints ONE JSON line with tokens/s, the per-kernel roofline of the dominant
kernel (durations from HIP events recorded on the launch stream inside the
timed region), the joint-attention TFLOP/s and a CPU baseline (the fp64
oracle timed on this host on a bounded sample, scaled by algorithmic FLOPs).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MMDiT block fwd tokens/s & joint-attn TFLOP/s (512 txt+4096 img, bf16)"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 4 SIMD x 1024 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5033.2       # MI355X dense fp8 (OCP e4m3) MFMA
PEAK_FP4_TFLOPS = 10066.3      # MI355X dense fp4 (OCP e2m1) MFMA, twice the fp8 rate (published as 10.1 PFLOP/s)


def algorithmic_work(wl, single_seq=False):
    """FLOPs the method must do per step ("Flux architecture deep dive", MMDiT
    layer and Flux single block): every linear 2*M*N*K, attention 4*B*H*L^2*Dh,
    over the workload's double and single blocks plus the image embedding,
    the text projection (when the workload has one) and the output linear.
    single_seq: the single blocks in the sequential form (qkv, proj, fc1, fc2
    over the joint sequence: the double block's linears)."""
    B, L, Li, Lt = wl.batch, wl.seq, wl.l_img, wl.l_txt
    D, F, H, dh, C = wl.hidden, wl.mlp_hidden, wl.heads, wl.head_dim, wl.latent_ch
    T = B * L
    gemm_double = 2 * T * D * (3 * D + D + F + F)         # qkv, proj, fc1, fc2 over both streams
    gemm_single = 2 * T * D * (3 * D + F) + 2 * T * (D + F) * D
    if single_seq:
        gemm_single = gemm_double
    attn = 4 * B * H * L * L * dh                         # QK^T and PV, no mask
    small_gemm = 2 * B * Li * C * D + 2 * B * Li * D * C  # image embedding, output linear
    if wl.context_dim:
        small_gemm += 2 * B * Lt * wl.context_dim * D     # text projection
    n_blocks = wl.n_double + wl.n_single
    gemm = wl.n_double * gemm_double + wl.n_single * gemm_single + small_gemm
    return {
        "gemm": gemm,
        "attention": n_blocks * attn,
        "total_flops": gemm + n_blocks * attn,
        "double_block_flops": gemm_double + attn,
    }


def recorded_traffic(kernel_class):
    """HBM bytes per launch of a kernel class from profiles/traffic.json (two
    rocprofv3 --pmc runs, FETCH_SIZE then WRITE_SIZE, scaled by a plain copy
    of known size), reported only while the kernel's source file is unchanged
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(kernel_class)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    try:
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    if digest != rec["source_sha256"]:
        return None
    return rec["hbm_bytes_per_launch"]


# kernel class of the timing hook -> (source file, kernel-name patterns of one launch of that class)
KERNEL_CLASSES = {
    "gemm_256_f16": ("flow_matching_diffusion_amd/csrc/gemm.hip", [r"gemm_dl_kernel<[23],"]),
    "gemm_256_bf16": ("flow_matching_diffusion_amd/csrc/gemm.hip", [r"gemm_dl_kernel<1,"]),
    "gemm_256_fp8": ("flow_matching_diffusion_amd/csrc/gemm.hip", [r"gemm_fp8r_kernel<\d+>"]),
    "gemm_256_mxfp8": ("flow_matching_diffusion_amd/csrc/gemm.hip", [r"gemm_fp8_kernel<\d+, 1>"]),
    "gemm_128x128": ("flow_matching_diffusion_amd/csrc/gemm.hip", [r"gemm_mfma_kernel<"]),
    "attention": ("flow_matching_diffusion_amd/csrc/attention.hip", [r"attn_(bf16|f32)_kernel"]),
    "ln_modulate": ("flow_matching_diffusion_amd/csrc/rowwise.hip", [r"ln_mod_kernel"]),
    "gemv": ("flow_matching_diffusion_amd/csrc/rowwise.hip", [r"gemv_kernel"]),
    "qk_prep": ("flow_matching_diffusion_amd/csrc/rowwise.hip", [r"prep_kernel<"]),
}
PROFILE_WORKLOAD = "flux12b_block_pair"
PROFILE_COMMANDS = [
    "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_trace -o bench -- "
    "python -u bench.py --steps 20 --warmup 5 --no-cpu-baseline",
    "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_fetch -o bench -- "
    "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline",
    "rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/pmc_write -o bench -- "
    "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline",
    "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_copy_fetch -o copy -- "
    "python -u bench.py --copy-calibration-mib 1024",
    "rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/pmc_copy_write -o copy -- "
    "python -u bench.py --copy-calibration-mib 1024",
    "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE -f csv -d gpurun_out/pmc_mfma -o bench -- "
    "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline",
    "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_BF16 "
    "-f csv -d gpurun_out/pmc_lds -o bench -- python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline",
    "python bench.py --summarize-counters gpurun_out --profiles-out gpurun_out/profiles",
]
SIMDS = 256 * 4   # MI355X: 256 CUs of 4 SIMDs
XCDS = 8          # GRBM_GUI_ACTIVE comes summed over the 8 XCDs


def _csv(directory, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "*" + suffix)))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    return list(csv.DictReader(open(files[0])))


def _counter_per_dispatch(rows, counter):
    """{kernel name: [counter value of each dispatch]} (KiB, summed over the
    per-XCD rows a dispatch may be split into)."""
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
        per[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def summarize_counters(directory, out_dir):
    """Turn the rocprofv3 CSVs of PROFILE_COMMANDS into profiles/traffic.json
    and two text summaries.  HBM bytes per launch of a class = mean FETCH_SIZE
    and WRITE_SIZE per dispatch of each of its kernels, each scaled by what the
    counter reads for a device copy of 1 GiB."""
    import hashlib
    import re
    copy_bytes = 1 << 30
    factors = {}
    for counter, sub in (("FETCH_SIZE", "pmc_copy_fetch"), ("WRITE_SIZE", "pmc_copy_write")):
        per = _counter_per_dispatch(_csv(os.path.join(directory, sub), "counter_collection.csv"), counter)
        vals = [v for k, vs in per.items() if "stream_copy_kernel" in k for v in vs]
        factors[counter] = copy_bytes / (1024.0 * sum(vals) / len(vals))
    fetch = _counter_per_dispatch(_csv(os.path.join(directory, "pmc_fetch"), "counter_collection.csv"), "FETCH_SIZE")
    write = _counter_per_dispatch(_csv(os.path.join(directory, "pmc_write"), "counter_collection.csv"), "WRITE_SIZE")
    stats = _csv(os.path.join(directory, "prof_trace"), "kernel_stats.csv")
    traffic, lines = {}, []
    for cls, (src, pats) in KERNEL_CLASSES.items():
        f_b = w_b = 0.0
        found = True
        for pat in pats:
            fk = [v for k, vs in fetch.items() if re.search(pat, k) for v in vs]
            wk = [v for k, vs in write.items() if re.search(pat, k) for v in vs]
            if not fk or not wk:
                found = False
                break
            f_b += 1024.0 * factors["FETCH_SIZE"] * sum(fk) / len(fk)
            w_b += 1024.0 * factors["WRITE_SIZE"] * sum(wk) / len(wk)
        if not found:
            continue
        digest = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
        traffic[cls] = {"source": src, "source_sha256": digest, "kernels": pats,
                        "fetch_bytes_per_launch": round(f_b), "write_bytes_per_launch": round(w_b),
                        "hbm_bytes_per_launch": round(f_b + w_b)}
        lines.append(f"| {cls} | {f_b / 2**20:.1f} | {w_b / 2**20:.1f} | {(f_b + w_b) / 2**20:.1f} |")
    out = {"workload": PROFILE_WORKLOAD, "commands": PROFILE_COMMANDS,
           "copy_calibration": {"bytes": copy_bytes, "fetch_factor": round(factors["FETCH_SIZE"], 4),
                                "write_factor": round(factors["WRITE_SIZE"], 4)}}
    out.update(traffic)
    # the timing hook's per-launch duration in the traced run, beside rocprofv3's
    hook = None
    for line in open(os.path.join(directory, "prof_trace.log")):
        if line.startswith('{"metric"'):
            hook = json.loads(line)
    agree = []
    if hook:
        for cls, (_, pats) in KERNEL_CLASSES.items():
            if cls not in hook["kernels"]:
                continue
            rows = [r for r in stats if any(re.search(pat, r["Name"]) for pat in pats)]
            # one launch of a class may be several kernels (prep: one; GEMM: one per epilogue kind):
            # duration per launch = total time / calls, per kernel name, summed over the names that
            # make up one launch when a class launches more than one kernel per call
            per_name = [int(r["TotalDurationNs"]) / int(r["Calls"]) for r in rows]
            if len(pats) > 1:
                avg = sum(per_name) / 1e3
            else:
                avg = sum(int(r["TotalDurationNs"]) for r in rows) / max(1, sum(int(r["Calls"]) for r in rows)) / 1e3
            agree.append(f"| {cls} | {1e3 * hook['kernels'][cls]['ms_per_launch']:.1f} | {avg:.1f} |")
        out["dominant_kernel"] = hook["roofline"]["kernel"]
    os.makedirs(out_dir, exist_ok=True)
    json.dump(out, open(os.path.join(out_dir, "traffic.json"), "w"), indent=1)
    cmds = "\n".join("    " + c for c in PROFILE_COMMANDS)
    with open(os.path.join(out_dir, f"hbm_traffic_{PROFILE_WORKLOAD}.md"), "w") as fh:
        fh.write(f"# HBM traffic per launch, {PROFILE_WORKLOAD}\n\nMade by:\n\n{cmds}\n\n"
                 f"Copy calibration (1 GiB device copy): FETCH_SIZE x {factors['FETCH_SIZE']:.3f}, "
                 f"WRITE_SIZE x {factors['WRITE_SIZE']:.3f}.\n\n"
                 "| class | fetch MiB/launch | write MiB/launch | total MiB/launch |\n|---|---|---|---|\n"
                 + "\n".join(lines) + "\n")
    with open(os.path.join(out_dir, f"kernel_stats_{PROFILE_WORKLOAD}.md"), "w") as fh:
        fh.write(f"# rocprofv3 --kernel-trace --stats, {PROFILE_WORKLOAD} (5 warmup, 20 timed eager steps, the graph capture and its replay check, 20 timed graph replays)\n\n"
                 f"Made by:\n\n    {PROFILE_COMMANDS[0]}\n\n"
                 "| kernel | calls | total ms | avg us | % |\n|---|---|---|---|---|\n")
        for r in stats:
            if float(r["Percentage"]) < 0.05:
                continue
            name = re.sub(r"\(.*$", "", r["Name"].replace("void ", ""))[:70]
            fh.write(f"| {name} | {r['Calls']} | {int(r['TotalDurationNs']) / 1e6:.2f} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |\n")
        if agree:
            fh.write("\nSame run, per launch of each class: the HIP-event hook of bench.py (timed steps only) "
                     "against rocprofv3's average over all dispatches (warmup included).\n\n"
                     "| class | hook us | rocprofv3 us |\n|---|---|---|\n" + "\n".join(agree) + "\n")
            fh.write("\nbench.py line of this run:\n\n    " + json.dumps({k: hook[k] for k in (
                "value", "unit", "ms_per_step", "roofline", "attention_tflops", "gemm_tflops")}) + "\n")
    summarize_mfma_lds(directory, out_dir)
    print(json.dumps(out, indent=1))
    return 0


def summarize_mfma_lds(directory, out_dir):
    """MFMA utilisation and LDS bank conflicts per kernel from the two extra
    --pmc passes of PROFILE_COMMANDS: busy = sum over SIMDs of
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); the
    engine clock of a dispatch = (GRBM_GUI_ACTIVE / 8) / its duration; counted
    MFMA FLOPs = 512 x SQ_INSTS_VALU_MFMA_MOPS_{F16,BF16}; conflict rate =
    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE."""
    import re
    try:
        mf = _csv(os.path.join(directory, "pmc_mfma"), "counter_collection.csv")
        ld = _csv(os.path.join(directory, "pmc_lds"), "counter_collection.csv")
    except SystemExit:
        return
    def per(rows, counter):
        return _counter_per_dispatch(rows, counter)
    dur = {}   # kernel -> [dispatch duration ns] in the MFMA pass
    for r in mf:
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            dur.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    busy, gui, sqb = (per(mf, c) for c in ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES"))
    conf, act, m16, mb16 = (per(ld, c) for c in ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
                                                  "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_BF16"))
    # _counter_per_dispatch scales nothing: raw counter values (KiB only for FETCH/WRITE_SIZE)
    lines = []
    for name in sorted(set(busy) | set(conf)):
        short = re.sub(r"\(.*$", "", name.replace("void ", ""))[:60]
        b, g = busy.get(name, []), gui.get(name, [])
        util = (sum(b) / (sum(g) / XCDS * SIMDS)) if b and g and sum(g) > 0 else None
        d = dur.get(name, [])
        # GHz; only for dispatches long enough (>= 50 us) that counting overhead does not matter
        clock = (sum(g) / XCDS / sum(d)) if g and d and min(d) >= 50000 else None
        c, a = conf.get(name, []), act.get(name, [])
        crate = (sum(c) / sum(a)) if c and a and sum(a) > 0 else None
        mops = sum(m16.get(name, [])) + sum(mb16.get(name, []))
        n = max(len(b), len(c), 1)
        nd = max(len(m16.get(name, [])), len(mb16.get(name, [])), 1)
        flops = 512.0 * mops / nd
        if util is None and crate is None:
            continue
        if (util or 0) < 1e-4 and (crate or 0) < 1e-4 and flops == 0:
            continue
        lines.append(f"| {short} | {n} | {'' if util is None else f'{100 * util:.1f}'} | "
                     f"{'' if clock is None else f'{clock:.2f}'} | "
                     f"{'' if crate is None else f'{100 * crate:.2f}'} | {flops / 1e9:.1f} |")
    cmds = "\n".join("    " + c for c in PROFILE_COMMANDS if "pmc SQ_" in c)
    with open(os.path.join(out_dir, f"mfma_lds_counters_{PROFILE_WORKLOAD}.md"), "w") as fh:
        fh.write(f"# MFMA utilisation and LDS bank conflicts per kernel, {PROFILE_WORKLOAD}\n\nMade by:\n\n{cmds}\n\n"
                 "MFMA busy = sum of SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 "
                 "SIMDs), the fraction of engine cycles the matrix units were busy; engine clock = "
                 "(GRBM_GUI_ACTIVE / 8) / dispatch duration (in the counters' own run); "
                 "LDS conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; counted GFLOP per dispatch = "
                 "512 x (SQ_INSTS_VALU_MFMA_MOPS_F16 + _BF16) / 1e9.\n\n"
                 "| kernel | dispatches | MFMA busy % | engine clock GHz | LDS bank-conflict % | "
                 "counted GFLOP / dispatch |\n|---|---|---|---|---|---|\n" + "\n".join(lines) + "\n")


HBM_CLASSES = ("ln_modulate", "gemv", "rf_noise_loss", "qk_prep")


def hbm_checks(FX, step, steps):
    """HBM-class kernels measured two ways, and the streaming ceiling.

    warm: the hooked eager steps as the step runs them (inputs may sit in L2
    or the 256 MB Infinity Cache, e.g. the residual a GEMM epilogue has just
    written); cold: the same steps with 512 MB overwritten before every timed
    launch (flux_timing_flush), so each kernel reads from HBM.  copy: the
    library's streaming copy of 1 GiB (read + write), the practical ceiling."""
    import torch
    out = {}
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for mode in ("warm", "cold"):
        FX.flux_timing_read()
        FX.flux_timing_flush(flush if mode == "cold" else None, flush.numel())
        FX.flux_timing_enable(True)
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        FX.flux_timing_enable(False)
        FX.flux_timing_flush(None)
        k = FX.flux_timing_read()
        out[mode] = {c: {"us_per_launch": round(1e3 * ms / n, 2), "gbs": round(w / (ms * 1e-3) / 1e9, 1)}
                     for c, (ms, n, w) in k.items() if n and c in HBM_CLASSES}
    del flush
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        FX.flux_stream_copy(src, dst, n)
    FX.flux_timing_read()
    FX.flux_timing_enable(True)
    for _ in range(10):
        FX.flux_stream_copy(src, dst, n)
    torch.cuda.synchronize()
    FX.flux_timing_enable(False)
    ms, cnt, w = FX.flux_timing_read()["hbm_copy"]
    out["copy_1gib_gbs"] = round(w / (ms * 1e-3) / 1e9, 1)
    out["note"] = ("gbs = algorithmic bytes / launch time; cold = 512 MB overwritten before each timed launch; "
                   "copy = flux_stream_copy of 1 GiB, read + write counted")
    del src, dst
    torch.cuda.empty_cache()
    return out


def hbm_sweep() -> int:
    """rf noising + loss (rf_noise_loss) and the streaming copy from 2^20 to
    2^28 elements (fp32), cold: each size's buffers are touched once, then a
    512 MB flush runs before each timed launch.  One JSON line per size."""
    import torch
    from flow_matching_diffusion_amd import flux as FX
    torch.cuda.set_device(0)
    FX.lib()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for lg in range(20, 29, 2):
        n = 1 << lg
        z0 = torch.randn(n, device="cuda")
        z1 = torch.randn(n, device="cuda")
        t = torch.full((1,), 0.3, device="cuda")
        zt, vt, vp = torch.empty_like(z0), torch.empty_like(z0), torch.randn(n, device="cuda")
        loss = torch.empty(1, device="cuda")
        wsb = FX.lib().flux_rf_workspace_bytes(1, n)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
        rec = {"elements": n}
        for mode in ("warm", "cold"):
            FX.rf_noise_loss(1, n, z0, z1, t, z_t=zt, v_target=vt)
            FX.rf_noise_loss(1, n, z0, z1, t, v_pred=vp, loss=loss, workspace=ws, workspace_bytes=wsb)
            torch.cuda.synchronize()
            FX.flux_timing_read()
            FX.flux_timing_flush(flush if mode == "cold" else None, flush.numel())
            FX.flux_timing_enable(True)
            for _ in range(5):
                FX.rf_noise_loss(1, n, z0, z1, t, z_t=zt, v_target=vt)          # 16 B per element
            torch.cuda.synchronize()
            FX.flux_timing_enable(False)
            ms, cnt, w = FX.flux_timing_read()["rf_noise_loss"]
            rec[mode + "_noise_gbs"] = round(w / (ms * 1e-3) / 1e9, 1)
            rec[mode + "_noise_us"] = round(1e3 * ms / cnt, 2)
            FX.flux_timing_enable(True)
            for _ in range(5):
                FX.rf_noise_loss(1, n, z0, z1, t, v_pred=vp, loss=loss, workspace=ws, workspace_bytes=wsb)
            torch.cuda.synchronize()
            FX.flux_timing_enable(False)
            ms, cnt, w = FX.flux_timing_read()["rf_noise_loss"]
            rec[mode + "_loss_gbs"] = round(w / (ms * 1e-3) / 1e9, 1)
            rec[mode + "_loss_us"] = round(1e3 * ms / cnt, 2)
            FX.flux_timing_enable(True)
            for _ in range(5):
                FX.flux_stream_copy(z0, zt, 4 * n)
            torch.cuda.synchronize()
            FX.flux_timing_enable(False)
            FX.flux_timing_flush(None)
            ms, cnt, w = FX.flux_timing_read()["hbm_copy"]
            rec[mode + "_copy_gbs"] = round(w / (ms * 1e-3) / 1e9, 1)
        print(json.dumps(rec), flush=True)
        del z0, z1, zt, vt, vp, ws
        torch.cuda.empty_cache()
    return 0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, emb, dws, sws, mi, work):
    """The fp64 oracle running the whole bench step once on this host: rf
    noising, image embedding, conditioning vector, the double and the single
    block over all 4608 tokens, the output head and the velocity MSE, on the
    same seeded inputs and weights as the GPU step.  BLAS threads are the
    host cores this process may use."""
    import numpy as np

    import oracle as O
    cores = len(os.sched_getaffinity(0))
    threads = cores
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores)
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [cores])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        limiter = None
    t0 = time.perf_counter()
    zt, _ = O.rf_noise(mi["z0"], mi["z1"], mi["t"])
    v = O.flux_forward(zt, mi["txt"], None, mi["t"], mi["ids"], emb, dws, sws, wl.heads, wl.axes_dim, wl.theta,
                       wl.eps, wl.model_channels)
    loss, _ = O.rf_loss(v, mi["z0"], mi["z1"])
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    assert np.isfinite(loss)
    return {"value": round(wl.tokens / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 numpy oracle, one whole step (rf noise, embed, 1 double + 1 single block over "
                       f"{wl.l_txt}+{wl.l_img} tokens, head, velocity MSE; {work['total_flops'] / 1e12:.2f} TFLOP) "
                       f"in {dt:.1f} s = {work['total_flops'] / dt / 1e9:.1f} GFLOP/s on {threads} BLAS threads "
                       f"({cores} usable cores, {_cpu_model()})"),
            "seconds": round(dt, 2), "loss": loss}


def _blas_name() -> str:
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info() if p.get("user_api") == "blas"]
        return ", ".join(libs) or "unknown"
    except Exception:  # pragma: no cover - threadpoolctl is optional
        return "unknown"


ORACLE_CONFIGS = ("C1", "C2", "C3", "C4", "C5")


def oracle_timing(which) -> int:
    """The fp64 numpy oracle timed on this host's usable cores, one JSON line
    per configuration (a reported baseline beside the GPU numbers, never the
    target):
      C1  tiny fp32 model, whole forward + loss (repeated for >= 2 s);
      C2  the Flux-535M-shaped model (1536 tokens), whole forward + loss;
      C3  the Flux-12B block-pair step (4608 tokens), whole;
      C4  the 19 + 38-block Flux-12B forward at batch 2, extrapolated: one
          double and one single block of one sample timed, times 19 / 38 and
          the batch, plus the embeddings and head timed at batch 2;
      C5  the block pair with E4M3 linears (the fp8 simulation: every token-path
          operand quantized and decoded, current scaling), one sample of the
          batch of 4 timed, times 4.
    No GPU is used."""
    import numpy as np

    import oracle as O
    from oracle import fp8_oracle as Q
    from flow_matching_diffusion_amd import synth

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        pass
    cpu, blas = _cpu_model(), _blas_name()

    def emit(cfg, wl, seconds, flops, tokens, sample):
        print(json.dumps({"config": cfg, "workload": wl.name, "kind": "oracle", "seconds": round(seconds, 3),
                          "tokens_per_s": round(tokens / seconds, 3), "fp64_gflops": round(flops / seconds / 1e9, 1),
                          "cores": cores, "cpu": cpu, "blas": blas, "sample": sample}), flush=True)

    def whole(cfg, wl):
        emb = synth.embed_weights(wl)
        dws = [synth.double_block_weights(wl, i) for i in range(wl.n_double)]
        sws = [synth.single_block_weights(wl, wl.n_double + i) for i in range(wl.n_single)]
        mi = synth.model_inputs(wl)
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < 2.0:
            zt, _ = O.rf_noise(mi["z0"], mi["z1"], mi["t"])
            v = O.flux_forward(zt, mi["txt"], mi.get("y"), mi["t"], mi["ids"], emb, dws, sws, wl.heads, wl.axes_dim,
                               wl.theta, wl.eps, wl.model_channels)
            loss, _ = O.rf_loss(v, mi["z0"], mi["z1"])
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        assert np.isfinite(loss)
        emit(cfg, wl, dt, algorithmic_work(wl)["total_flops"], wl.tokens,
             f"whole forward + loss, mean of {reps} run(s)")

    def pair_one_sample(wl, lin=None):
        one = synth.custom_workload(wl.name + "_one_sample", base=wl.name, batch=1)
        inp = synth.block_inputs(one)
        ang = O.rope_angles(synth.joint_ids(one), wl.axes_dim, wl.theta)
        w2, w1 = synth.double_block_weights(one, 0), synth.single_block_weights(one, 1)
        t0 = time.perf_counter()
        xi, xt = O.double_block(inp["x_img"], inp["x_txt"], inp["vec"], ang, w2, wl.heads, wl.eps, lin=lin)
        td = time.perf_counter() - t0
        print(f"[oracle] {wl.name}: double block of one sample {td:.1f} s", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        y = O.single_block(np.concatenate([xi, xt], axis=1), inp["vec"], ang, w1, wl.heads, wl.eps, lin=lin)
        ts = time.perf_counter() - t0
        print(f"[oracle] {wl.name}: single block of one sample {ts:.1f} s", file=sys.stderr, flush=True)
        assert np.isfinite(y).all()
        return td, ts

    for cfg in which:
        if cfg == "C1":
            whole(cfg, synth.WORKLOADS["tiny_fp32"])
        elif cfg == "C2":
            whole(cfg, synth.WORKLOADS["flux535m"])
        elif cfg == "C3":
            whole(cfg, synth.WORKLOADS["flux12b_blocks"])
        elif cfg == "C4":
            wl = synth.WORKLOADS["flux12b_full"]
            td, ts = pair_one_sample(wl)
            emb, mi = synth.embed_weights(wl), synth.model_inputs(wl)
            t0 = time.perf_counter()
            zt, _ = O.rf_noise(mi["z0"], mi["z1"], mi["t"])
            v = O.flux_forward(zt, mi["txt"], mi.get("y"), mi["t"], mi["ids"], emb, [], [], wl.heads, wl.axes_dim,
                               wl.theta, wl.eps, wl.model_channels)
            O.rf_loss(v, mi["z0"], mi["z1"])
            te = time.perf_counter() - t0
            total = wl.batch * (wl.n_double * td + wl.n_single * ts) + te
            emit(cfg, wl, total, algorithmic_work(wl)["total_flops"], wl.tokens,
                 f"extrapolated: one double ({td:.1f} s) and one single block ({ts:.1f} s) of one sample timed, "
                 f"x{wl.n_double} / x{wl.n_single} blocks x{wl.batch} samples, plus noising, embeddings, head "
                 f"and loss at batch {wl.batch} ({te:.1f} s)")
        elif cfg == "C5":
            wl = synth.WORKLOADS["flux12b_blocks_fp8"]

            def fp8_lin(name, x, w, b):
                return Q.fp8_linear(x, w, b, Q.current_scale(x), Q.current_scale(w))

            td, ts = pair_one_sample(wl, lin=fp8_lin)
            work = algorithmic_work(synth.custom_workload("c5_one", base=wl.name, batch=1))
            blocks = work["total_flops"] - 2 * 2 * wl.l_img * wl.latent_ch * wl.hidden   # no embedding / head
            emit(cfg, wl, wl.batch * (td + ts), wl.batch * blocks, wl.tokens,
                 f"block pair with E4M3 linears (fp8 simulation, current scaling), one sample timed "
                 f"({td + ts:.1f} s), x{wl.batch} samples")
        else:
            print(f"unknown configuration {cfg}", file=sys.stderr)
            return 2
    return 0


def mx_linears_bench(args, fp4=False) -> int:
    """The six token-path linears of the Flux-12B block pair at batch 4
    (qkv, proj, fc1, fc2 over the joint 4608-token rows of 4 samples; lin1,
    lin2 of the single block) as MXFP8 (E4M3 elements) or, with fp4, MXFP4
    (E2M1 elements) linears: per step, every input is quantized (bf16 source)
    and multiplied with its quantized weight.  Weights are quantized once,
    before timing (static)."""
    import numpy as np
    import torch

    from flow_matching_diffusion_amd import flux as FX

    torch.cuda.set_device(0)
    FX.lib()
    B, L, D, F = 4, 4608, 3072, 12288
    M = B * L
    shapes = [("qkv", D, 3 * D), ("proj", D, D), ("fc1", D, F), ("fc2", F, D), ("lin1", D, 3 * D + F),
              ("lin2", D + F, D)]
    if fp4:
        scale_bytes, quantize, linear = FX.flux_mxfp4_scale_bytes, FX.flux_mxfp4_quantize, FX.flux_mxfp4_linear_fwd
        gemm_cls, quant_cls, peak, tag = "gemm_256_mxfp4", "mxfp4_quantize", PEAK_FP4_TFLOPS, "mxfp4"
    else:
        scale_bytes, quantize, linear = FX.flux_mx_scale_bytes, FX.flux_mx_quantize, FX.flux_mxfp8_linear_fwd
        gemm_cls, quant_cls, peak, tag = "gemm_256_mxfp8", "mx_quantize", PEAK_FP8_TFLOPS, "mxfp8"
    cb = 2 if fp4 else 1   # values per code byte
    g = torch.Generator(device="cuda").manual_seed(1234)
    ops = []
    for name, K, N in shapes:
        x = (torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32)).to(torch.bfloat16)
        w = (torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32) * 0.02).to(torch.bfloat16)
        xq = torch.empty((M, K // cb), dtype=torch.uint8, device="cuda")
        xs = torch.empty((scale_bytes(M, K),), dtype=torch.uint8, device="cuda")
        wq = torch.empty((N, K // cb), dtype=torch.uint8, device="cuda")
        ws = torch.empty((scale_bytes(N, K),), dtype=torch.uint8, device="cuda")
        quantize(FX.FLUX_PREC_BF16, w, N, K, wq, ws)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        ops.append((name, K, N, x, xq, xs, wq, ws, y))
        del w
    torch.cuda.synchronize()

    def step():
        for name, K, N, x, xq, xs, wq, ws, y in ops:
            quantize(FX.FLUX_PREC_BF16, x, M, K, xq, xs)
            linear(M, N, K, xq, xs, wq, ws, None, y, N)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    FX.flux_timing_read()
    FX.flux_timing_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    FX.flux_timing_enable(False)
    kernels = FX.flux_timing_read()
    ms_step = e0.elapsed_time(e1) / args.steps
    flops = sum(2.0 * M * N * K for _, K, N, *_ in ops)
    gms, gn, gw = kernels[gemm_cls]
    qms, qn, qw = kernels[quant_cls]
    assert abs(gw / args.steps - flops) <= 1e-6 * flops
    tflops = gw / (gms * 1e-3) / 1e12
    assert bool(torch.isfinite(ops[-1][-1]).all())
    elem = "E2M1" if fp4 else "E4M3"
    rec = {
        "metric": f"{tag.upper()} block-linear TFLOP/s (the six token-path linears of the Flux-12B block pair, "
                  "batch 4, inputs quantized every step)",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": f"{tag}_{elem.lower()} (E8M0 scale per 32 values along K)",
        "data": "synthetic",
        "config": {"workload": f"flux12b_block_pair_{tag}_linears", "rows": M, "hidden": D, "mlp_hidden": F,
                   "linears": [n for n, *_ in shapes]},
        "roofline": {"kernel": gemm_cls, "bound": "mfma", "achieved": round(tflops, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": None, "flops_per_launch": gw / gn, "ms_per_launch": round(gms / gn, 5)},
        "kernels": {gemm_cls: {"ms_per_launch": round(gms / gn, 5), "tflops": round(tflops, 2)},
                    quant_cls: {"ms_per_launch": round(qms / qn, 5),
                                "gbs": round(qw / (qms * 1e-3) / 1e9, 1)}},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def train_bench(args) -> int:
    """One rectified-flow training step of the Flux-12B-shaped block-pair model
    at batch 1 (4096 image + 512 text tokens): noising, image embedding and
    conditioning vector, the training forward of one double and one single
    block, the output head and the velocity MSE, then the backward of all of
    it in reverse (loss gradient, head, single block, double block,
    embeddings) -- every weight gradient.  Block weights are drawn on the
    device; the other weights and the inputs come from the host streams."""
    import torch

    from flow_matching_diffusion_amd import flux as FX
    from flow_matching_diffusion_amd import synth
    from flow_matching_diffusion_amd.model import FluxTrainer, device_array

    torch.cuda.set_device(0)
    FX.lib()
    wl = synth.WORKLOADS["flux12b_blocks"]
    B, L, D, Li, C = wl.batch, wl.seq, wl.hidden, wl.l_img, wl.latent_ch
    print(f"[bench] drawing weights for {wl.name}", file=sys.stderr, flush=True)
    tr = FluxTrainer(wl, synth.embed_weights(wl), [synth.device_block_weights(wl, 0, "double")],
                     [synth.device_block_weights(wl, 1, "single")])
    mi = synth.model_inputs(wl)
    dev = lambda a, bf=False: device_array(a, bf)
    z0, z1, t, ids = dev(mi["z0"]), dev(mi["z1"]), dev(mi["t"]), dev(mi["ids"])
    txt = dev(mi["txt"], True)

    def step():
        return tr.step(z0, z1, t, txt, None, ids)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps (per-kernel hook)", file=sys.stderr, flush=True)
    FX.flux_timing_read()
    FX.flux_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    FX.flux_timing_enable(False)
    kernels = FX.flux_timing_read()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        loss = step()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    assert bool(torch.isfinite(loss).all()) and bool(torch.isfinite(tr.g_double[0]["img_qkv.w"]).all())
    table = {}
    for name, (ms, n, work) in kernels.items():
        if n == 0:
            continue
        ent = {"ms_per_launch": round(ms / n, 5), "launches_per_step": n / args.steps,
               "ms_per_step": round(ms / args.steps, 5)}
        if name.startswith("gemm") or name.startswith("attention"):
            ent["tflops"] = round(work / (ms * 1e-3) / 1e12, 2)
            ent["flops_per_launch"] = work / n
        else:
            ent["gbs"] = round(work / (ms * 1e-3) / 1e9, 1)
        table[name] = ent
    # algorithmic FLOPs: block GEMMs forward plus their data and weight gradients; the image input
    # linear forward plus its weight gradient; the head linear forward, data and weight gradients;
    # attention forward (two L x L x Dh products per head) and backward (five)
    blk = 2.0 * B * L * D * D * (3 + 1 + 4 + 4 + 7 + 5)
    small = 2.0 * B * Li * C * D
    att = 4.0 * B * wl.heads * L * L * wl.head_dim
    flops = 3.0 * blk + 2.0 * small + 3.0 * small + 2 * att + 2 * 2.5 * att
    recorded = sum(w for nm, (ms, n, w) in kernels.items() if nm.startswith("gemm") or nm.startswith("attention"))
    assert abs(recorded / args.steps - flops) <= 1e-6 * flops, (recorded / args.steps, flops)
    dom = max((k for k in table if "tflops" in table[k]), key=lambda k: table[k]["ms_per_step"])
    peak = PEAK_BF16_TFLOPS
    rec = {
        "metric": "MMDiT block pair rectified-flow training step tokens/s (forward + backward, 512 txt + 4096 img, "
                  "bf16)",
        "value": round(B * L / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (device-drawn block weights)",
        "config": {"workload": "flux12b_block_pair_train_step", "batch": B, "l_txt": wl.l_txt, "l_img": Li,
                   "hidden": D, "heads": wl.heads, "head_dim": wl.head_dim, "mlp_hidden": wl.mlp_hidden,
                   "double_blocks": 1, "single_blocks": 1,
                   "step": "rf noise + embed + vec + double + single block training forwards + head + velocity "
                           "MSE, then the backward of all of it (every weight gradient)"},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": table[dom]["tflops"], "peak": peak,
                     "unit": "TFLOP/s", "frac": round(table[dom]["tflops"] / peak, 4), "traffic": None,
                     "flops_per_launch": table[dom]["flops_per_launch"], "ms_per_launch": table[dom]["ms_per_launch"]},
        "step_tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "loss": float(loss.item()),
        "kernels": table,
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def attention_fp8_bench(args) -> int:
    """Joint attention of the Flux-12B block shapes (B=1, 4608 tokens, 24
    heads of 128) with E4M3 operands: per step, Q, K and V (bf16 token rows)
    are laid out head-major, quantized with their current scales and attended
    on the fp8 MFMA (flux_attention_fp8_fwd)."""
    import torch

    from flow_matching_diffusion_amd import flux as FX

    torch.cuda.set_device(0)
    FX.lib()
    B, L, H = 1, 4608, 24
    D = H * 128
    g = torch.Generator(device="cuda").manual_seed(77)
    q, k, v = ((torch.randn((B, L, D), generator=g, device="cuda") * s).to(torch.bfloat16) for s in (0.25, 1.0, 1.0))
    o = torch.empty((B, L, D), dtype=torch.bfloat16, device="cuda")
    rec = torch.zeros(3 * FX.FP8_TENSOR_BYTES, dtype=torch.uint8, device="cuda")
    wsb = FX.flux_attention_fp8_workspace_bytes(B, L, H)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    def step():
        FX.flux_attention_fp8_fwd(B, L, H, q, k, v, D, o, D, rec, ws, wsb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    FX.flux_timing_read()
    FX.flux_timing_enable(True)              # per-kernel durations (HIP events around each launch)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    FX.flux_timing_enable(False)
    kernels = FX.flux_timing_read()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()                              # the step time, without the hook
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    flops = 4.0 * B * H * L * L * 128
    ams, an, aw = kernels["attention"]
    assert abs(aw / args.steps - flops) <= 1e-6 * flops
    tf = aw / (ams * 1e-3) / 1e12
    assert bool(torch.isfinite(o.float()).all())
    table = {n: {"ms_per_launch": round(ms / c, 5), "launches_per_step": c / args.steps} for n, (ms, c, w) in
             kernels.items() if c}
    rec_out = {
        "metric": "joint attention TFLOP/s with E4M3 operands (Flux-12B block shape, 4096 img + 512 txt tokens, "
                  "24 heads)",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3 Q, K, V and P (per-tensor current scales), fp32 accumulation",
        "data": "synthetic", "config": {"workload": "flux12b_joint_attention_fp8", "batch": B, "seq": L, "heads": H,
                                        "head_dim": 128},
        "roofline": {"kernel": "attention", "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": aw / an, "ms_per_launch": round(ams / an, 5)},
        "kernels": table,
        "cpu_baseline": None,
    }
    print(json.dumps(rec_out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager steps only (the default also captures the step in a HIP graph and "
                         "reports the replay time as ms_per_step)")
    ap.add_argument("--workload", default="flux12b_blocks",
                    choices=["flux12b_blocks", "flux12b_full", "flux12b_blocks_fp8", "flux12b_blocks_seq",
                             "flux12b_sample_cfg", "flux12b_mxfp8_linears", "flux12b_blocks_train",
                             "flux12b_attention_fp8", "flux12b_mxfp4_linears"],
                    help="flux12b_blocks (default): the block-pair step the headline metric is quoted on; "
                         "flux12b_full: the whole 19 + 38 block forward + loss at batch 2 (block weights "
                         "drawn on the device; no CPU baseline); flux12b_blocks_fp8: the block pair at batch 4 "
                         "with E4M3 linears under delayed scaling (static weights cast during warm-up); "
                         "flux12b_blocks_seq: the block pair with the single block in its sequential form "
                         "(flux_single_seq_fwd); flux12b_sample_cfg: Euler sampling steps of one image with "
                         "classifier-free guidance (conditional + null-prompt rows in one batch-2 forward, "
                         "guidance embedding on) on the block-pair model; flux12b_mxfp8_linears: the six "
                         "token-path linears of the block pair at batch 4 as MXFP8 linears; "
                         "flux12b_blocks_train: a whole rectified-flow training step (forward and backward) of the "
                         "block-pair model at batch 1; flux12b_attention_fp8: the joint attention of the block "
                         "shape with E4M3 operands; flux12b_mxfp4_linears: the six linears as MXFP4 linears")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a device copy of this many MiB, 5 times (the known-size kernel that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--hbm-sweep", action="store_true",
                    help="only run the HBM sweep: rf noising / loss and the streaming copy from 2^20 to 2^28 "
                         "fp32 elements, warm and with the caches flushed before each timed launch")
    ap.add_argument("--oracle-timing", metavar="CONFIGS", default=None,
                    help="no GPU: time the fp64 oracle on this host for a comma-separated subset of "
                         + ",".join(ORACLE_CONFIGS) + " (one JSON line each; C4 and C5 extrapolated from one "
                         "sample, as each line says)")
    ap.add_argument("--summarize-counters", metavar="DIR", default=None,
                    help="no GPU: write profiles/traffic.json and the profile summaries from the rocprofv3 "
                         "CSV folders under DIR (see PROFILE_COMMANDS)")
    ap.add_argument("--profiles-out", default=os.path.join(ROOT, "profiles"),
                    help="where --summarize-counters writes")
    args = ap.parse_args()
    if args.oracle_timing:
        return oracle_timing([c.strip() for c in args.oracle_timing.split(",") if c.strip()])
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.profiles_out)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on exactly one GPU (asked for {max(args.gpus, world)}); "
              "multi-GPU sharding is described in the design notes, not implemented", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.hbm_sweep:
        return hbm_sweep()
    if args.workload == "flux12b_mxfp8_linears":
        return mx_linears_bench(args)
    if args.workload == "flux12b_mxfp4_linears":
        return mx_linears_bench(args, fp4=True)
    if args.workload == "flux12b_blocks_train":
        return train_bench(args)
    if args.workload == "flux12b_attention_fp8":
        return attention_fp8_bench(args)
    if args.copy_calibration_mib:
        from flow_matching_diffusion_amd import flux as FX
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            FX.flux_stream_copy(src, dst, n)   # stream_copy_kernel: n bytes read, n written
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}))
        return 0

    from flow_matching_diffusion_amd import flux as FX
    from flow_matching_diffusion_amd import synth
    from flow_matching_diffusion_amd.model import FluxModel, device_array

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    FX.lib()
    full = args.workload == "flux12b_full"
    seq = args.workload == "flux12b_blocks_seq"
    sample = args.workload == "flux12b_sample_cfg"
    if sample:
        wl = synth.custom_workload("flux12b_sample_cfg", base="flux12b_blocks", batch=2)
    else:
        wl = synth.WORKLOADS["flux12b_blocks" if seq else args.workload]
    print(f"[bench] generating weights for {wl.name}", file=sys.stderr, flush=True)
    emb = synth.embed_weights(wl, guidance=sample)
    mi = synth.model_inputs(wl)
    if full:
        w2 = None
        dws = [synth.device_block_weights(wl, i, "double") for i in range(wl.n_double)]
        sws = [synth.device_block_weights(wl, wl.n_double + i, "single") for i in range(wl.n_single)]
    else:
        w2 = synth.double_block_weights(wl, 0)
        w1 = synth.single_seq_block_weights(wl, 1) if seq else synth.single_block_weights(wl, 1)
        dws = [w2]
        sws = [w1]
    # block linears held in fp16, converted once here (static weights; not timed)
    m = FluxModel(wl, emb, dws, sws, weights_f16=True)
    del dws, sws
    dev = lambda a, bf=False: device_array(a, bf)
    z0, z1, t, ids = dev(mi["z0"]), dev(mi["z1"]), dev(mi["t"]), dev(mi["ids"])
    txt = dev(mi["txt"], True)
    y = dev(mi["y"]) if "y" in mi else None
    out: dict = {}

    def step():
        m.forward_loss(z0, z1, t, txt, y, ids, out)

    if sample:
        si = synth.sampler_inputs(wl, 1)
        s_z1, s_txt, s_ids, s_g = dev(si["z1"]), dev(si["txt"], True), dev(si["ids"]), dev(si["guidance"])
        n_grid = args.warmup + args.steps
        step_i = [0]

        def step():   # noqa: F811 - one sampler step: batch-2 forward + guided Euler update
            m.sample(s_z1, n_grid, s_txt, None, s_ids, cfg_w=3.5, guidance=s_g, out=out,
                     steps=range(step_i[0], step_i[0] + 1))
            step_i[0] += 1

    fp8 = wl.precision == "fp8"
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(max(args.warmup, 2) if fp8 else args.warmup):
        step()
    torch.cuda.synchronize()
    fp8_cast_ms = None
    if fp8:
        # static weights: cast once more with the settled scales (timed on its own), then the
        # timed steps run blocks + scale update without the weight cast
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        m.fp8_cast_weights()
        e1.record()
        torch.cuda.synchronize()
        fp8_cast_ms = e0.elapsed_time(e1)
        m.cast_each_forward = False
    # per-kernel durations: eager steps with the HIP-event hook around every launch
    FX.flux_timing_read()                       # discard anything recorded so far
    FX.flux_timing_enable(True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} steps (per-kernel hook)", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    FX.flux_timing_enable(False)
    kernels = FX.flux_timing_read()
    ms_step_eager = ev0.elapsed_time(ev1) / args.steps
    hbm = hbm_checks(FX, step, args.steps) if not sample else None
    ms_step = ms_step_eager
    graph_ok = None
    # the step time: the same step captured once in a HIP graph and replayed
    # (no hook events, no launch gaps).  Every replay is checked against an
    # eager step on the same inputs before timing (a deterministic forward:
    # bit-identical outputs); the sampler's steps differ in their scalar
    # arguments and stay eager.
    if not args.no_graph and not sample:
        print("[bench] capturing the step in a HIP graph", file=sys.stderr, flush=True)
        step()
        torch.cuda.synchronize()
        ref_v = out["v_pred"].clone()
        ref_l = out["loss"].clone()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()                                  # eager on the capture stream once (allocations settle)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        graph_ok = True
        for r in range(3):
            out["v_pred"].zero_()
            graph.replay()
            torch.cuda.synchronize()
            same = bool(torch.equal(out["v_pred"], ref_v)) and bool(torch.equal(out["loss"], ref_l))
            if not same and not fp8:
                graph_ok = False
            step()                                  # eager work between replays
            torch.cuda.synchronize()
        if not fp8:
            assert graph_ok, "graph replay differs from the eager step"
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        print(f"[bench] timing {args.steps} graph replays", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms_step = g0.elapsed_time(g1) / args.steps
    if sample:
        loss = None
        assert bool(torch.isfinite(out["z"]).all()), "non-finite sample"
    else:
        loss = float(out["loss"].item())
        assert np.isfinite(loss), "non-finite loss"

    work = algorithmic_work(wl, single_seq=seq)
    kt = {}
    for k, (ms, n, w) in kernels.items():
        if not n:
            continue
        compute = k.startswith("gemm") or k == "attention"
        kt[k] = {"ms_per_launch": ms / n, "launches_per_step": n / args.steps, "ms_per_step": ms / args.steps,
                 ("tflops" if compute else "gbs"): (w / (ms * 1e-3) / (1e12 if compute else 1e9)) if ms > 0 else 0.0,
                 ("flops_per_launch" if compute else "bytes_per_launch"): w / n}
    # the launch-reported work must add up to the method's algorithmic FLOPs
    gemm_w = sum(v[2] for k, v in kernels.items() if k.startswith("gemm")) / args.steps
    attn_w = kernels.get("attention", (0, 0, 0.0))[2] / args.steps
    assert abs(gemm_w - work["gemm"]) <= 1e-6 * work["gemm"], (gemm_w, work["gemm"])
    assert abs(attn_w - work["attention"]) <= 1e-6 * work["attention"], (attn_w, work["attention"])
    dom = max(kt, key=lambda k: kt[k]["ms_per_step"])
    d = kt[dom]
    if "tflops" in d:
        # a contraction is measured against the MFMA peak of its own operand type
        peak = PEAK_FP8_TFLOPS if dom.endswith("fp8") else PEAK_BF16_TFLOPS
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(d["tflops"], 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(d["tflops"] / peak, 4), "traffic": recorded_traffic(dom),
                "flops_per_launch": d["flops_per_launch"], "ms_per_launch": round(d["ms_per_launch"], 5)}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(d["gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(d["gbs"] / PEAK_HBM_GBS, 4), "traffic": recorded_traffic(dom),
                "bytes_per_launch": d["bytes_per_launch"], "ms_per_launch": round(d["ms_per_launch"], 5)}
    attn = kt.get("attention")
    attn_tflops = attn["tflops"] if attn else None
    gemm_ms = sum(v["ms_per_step"] for k, v in kt.items() if k.startswith("gemm"))
    gemm_tflops = work["gemm"] / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None

    rec = {
        "metric": METRIC,
        "value": round(wl.tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 weights and attention q/k/v; fp16 GEMM activation operands x fp16 copies of the weights, "
                 "fp32 accumulation; fp32 residual stream",
        "data": "synthetic",
        "config": {"workload": "flux12b_full_forward_rf_step" if full else "flux12b_block_pair_rf_step",
                   "batch": wl.batch, "l_txt": wl.l_txt,
                   "l_img": wl.l_img, "hidden": wl.hidden, "heads": wl.heads, "head_dim": wl.head_dim,
                   "mlp_hidden": wl.mlp_hidden, "double_blocks": wl.n_double, "single_blocks": wl.n_single,
                   "step": ("rf noise + image/text embed + vec + %d double blocks + %d single blocks + head + "
                            "velocity MSE" % (wl.n_double, wl.n_single))},
        "roofline": roof,
        "attention_tflops": round(attn_tflops, 2) if attn_tflops else None,
        "attention_frac_of_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4) if attn_tflops else None,
        "gemm_tflops": round(gemm_tflops, 2) if gemm_tflops else None,
        "step_tflops": round(work["total_flops"] / (ms_step * 1e-3) / 1e12, 2),
        "kernels": {k: {kk: (round(vv, 5) if vv < 1e6 else vv) for kk, vv in v.items()} for k, v in kt.items()},
        "ms_per_step_eager_with_hook": round(ms_step_eager, 4),
        "hbm": hbm,
        "graph": None if graph_ok is None else ("replays bit-identical to eager" if graph_ok else "replayed"),
        "wall_s": round(wall, 3),
        "loss": loss,
    }
    if full:
        rec["metric"] = "Flux-12B-shaped forward + loss tokens/s (19 double + 38 single blocks, bf16)"
    if fp8:
        rec["metric"] = "MMDiT block fwd tokens/s, E4M3 linears with delayed scaling (512 txt+4096 img, batch 4)"
        rec["dtype"] = "fp8_e4m3 linears, bf16 attention"
        rec["config"]["workload"] = "flux12b_block_pair_fp8_rf_step"
        rec["fp8_weight_cast_ms"] = round(fp8_cast_ms, 4)
        fk = kt.get("gemm_256_fp8")
        if fk:
            rec["fp8_gemm_frac_of_fp8_peak"] = round(fk["tflops"] / PEAK_FP8_TFLOPS, 4)
    if sample:
        rec["metric"] = ("CFG Euler sampling tokens/s (1 image: conditional + null-prompt rows in one batch-2 "
                         "forward, 512 txt+4096 img, 1 double + 1 single block)")
        rec["config"]["workload"] = "flux12b_block_pair_cfg_euler_sampling_step"
        rec["config"]["step"] = ("embed (+ guidance embedding) + 1 double + 1 single block + head at batch 2, "
                                 "then the fused CFG combination + Euler update")
        rec["config"]["images"] = 1
        rec["sampler_step_ms"] = round(ms_step, 4)
    if seq:
        rec["metric"] = "MMDiT block fwd tokens/s, double + sequential single block (512 txt+4096 img)"
        rec["config"]["workload"] = "flux12b_block_pair_sequential_single_rf_step"
    if not args.no_cpu_baseline and not full and not fp8 and not seq and not sample:
        print("[bench] cpu baseline (oracle, whole step)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl, emb, [w2], [w1], mi, work)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
