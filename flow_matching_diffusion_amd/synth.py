"""Seeded synthetic inputs for the Flux MMDiT forward and the rectified-flow objective.

This module only draws random numbers and lays them out: it holds none of the
method's arithmetic.  Both the HIP path and the fp64 oracle consume the arrays
it returns, so the two sides see bit-identical inputs.

Every tensor has its own stream,
``numpy.random.Generator(PCG64(SeedSequence([1234, config_id, block_id, tensor_id])))``,
so any block's weights can be regenerated on its own.  Values meant for bf16
operands are rounded to bf16 (round-to-nearest-even) here, on the host, and are
returned as float32 arrays whose values are exactly representable in bf16.

Shapes follow the workloads of the Flux pages:
  * "Flux model API reference", FluxConfig key parameters: hidden 3072, 24
    heads, in_channels 64, context_dim 4096, vec_in_dim 768, model_channels 256,
    theta 10000, axes_dim (16, 56, 56), qkv bias, eps 1e-6.
  * "Flux architecture deep dive", Model variants: 535M = 1 joint + 1 single
    layer, 12B = 19 joint + 38 single layers.
Weights are N(0, 0.02); the QK-RMSNorm scales are 1 + 0.1 N(0, 1) so that a
dropped scale is visible; activations, latents and noise are N(0, 1).
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, Optional, Tuple

import numpy as np

BASE_SEED = 1234
WEIGHT_STD = 0.02
GAMMA_STD = 0.1


# --------------------------------------------------------------------------- #
# bf16 helpers (storage format only)
# --------------------------------------------------------------------------- #
def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even).

    Returns float32 whose low 16 bits are zero.  Inputs are finite draws.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = (u + bias) & np.uint32(0xFFFF0000)
    return out.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of bf16-representable float32 values."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("array is not bf16-representable; round it first")
    return (u >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------- #
# workload shapes
# --------------------------------------------------------------------------- #
@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic Flux workload (no weights, no values)."""

    name: str
    config_id: int
    batch: int
    hidden: int
    heads: int
    head_dim: int
    mlp_hidden: int
    img_h: int
    img_w: int
    l_txt: int
    axes_dim: Tuple[int, int, int]
    theta: float
    eps: float
    latent_ch: int
    n_double: int
    n_single: int
    precision: str                 # "f32" | "bf16" | "fp8"
    context_dim: Optional[int]     # T5 width; None -> text enters at hidden width
    vec_in_dim: Optional[int]      # CLIP pooled width; None -> no pooled vector
    model_channels: int = 256      # sinusoidal timestep width
    t_dist: str = "uniform"        # "uniform" | "logit_normal"
    vec_given: bool = False        # True -> vec ~ N(0,1) is an input (block-only workloads)

    @property
    def l_img(self) -> int:
        return self.img_h * self.img_w

    @property
    def seq(self) -> int:
        return self.l_img + self.l_txt

    @property
    def tokens(self) -> int:
        return self.batch * self.seq


WORKLOADS: Dict[str, Workload] = {
    # one double + one single block at hidden 256, 4x64 heads, 16 text + 8x8 image tokens, fp32
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 256, 4, 64, 1024, 8, 8, 16, (8, 28, 28), 10000.0, 1e-6,
                          64, 1, 1, "f32", None, None),
    # Flux-535M-shaped stack: 512 T5 tokens (4096-d) + 32x32 image tokens, bf16
    "flux535m": Workload("flux535m", 2, 1, 3072, 24, 128, 12288, 32, 32, 512, (16, 56, 56), 10000.0, 1e-6,
                         64, 1, 1, "bf16", 4096, 768),
    # Flux-12B block shapes: 512 text + 64x64 image tokens (4608 joint), vec given, bf16
    "flux12b_blocks": Workload("flux12b_blocks", 3, 1, 3072, 24, 128, 12288, 64, 64, 512, (16, 56, 56),
                               10000.0, 1e-6, 64, 1, 1, "bf16", None, None, vec_given=True),
    # full Flux-12B-shaped forward: 19 double + 38 single blocks, batch 2, logit-normal t
    "flux12b_full": Workload("flux12b_full", 4, 2, 3072, 24, 128, 12288, 64, 64, 512, (16, 56, 56),
                             10000.0, 1e-6, 64, 19, 38, "bf16", 4096, 768, t_dist="logit_normal"),
    # fp8 variant of the 12B block shapes, batch 4
    "flux12b_blocks_fp8": Workload("flux12b_blocks_fp8", 5, 4, 3072, 24, 128, 12288, 64, 64, 512,
                                   (16, 56, 56), 10000.0, 1e-6, 64, 1, 1, "fp8", None, None, vec_given=True),
}


def custom_workload(name: str, **kw) -> Workload:
    """A workload derived from a named one with some fields replaced (tests use
    this for ragged and tiny shapes)."""
    base = WORKLOADS[kw.pop("base", "tiny_fp32")]
    return dataclasses.replace(base, name=name, **kw)


# --------------------------------------------------------------------------- #
# random streams
# --------------------------------------------------------------------------- #
def tensor_id(name: str) -> int:
    return zlib.crc32(name.encode()) & 0x7FFFFFFF


def stream(config_id: int, block_id: int, name: str) -> np.random.Generator:
    ss = np.random.SeedSequence([BASE_SEED, config_id, block_id, tensor_id(name)])
    return np.random.Generator(np.random.PCG64(ss))


def normal(shape, std: float, config_id: int, block_id: int, name: str, bf16: bool) -> np.ndarray:
    g = stream(config_id, block_id, name)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return round_to_bf16(a) if bf16 else a


def uniform01(shape, config_id: int, block_id: int, name: str) -> np.ndarray:
    g = stream(config_id, block_id, name)
    return g.random(size=shape, dtype=np.float32)


# --------------------------------------------------------------------------- #
# weights (torch Linear layout: W [out, in], bias [out])
# --------------------------------------------------------------------------- #
def _lin(wl: Workload, blk: int, name: str, n_out: int, n_in: int, bf16: bool) -> Dict[str, np.ndarray]:
    return {
        name + ".w": normal((n_out, n_in), WEIGHT_STD, wl.config_id, blk, name + ".w", bf16),
        name + ".b": normal((n_out,), WEIGHT_STD, wl.config_id, blk, name + ".b", bf16),
    }


def _gamma(wl: Workload, blk: int, name: str) -> np.ndarray:
    g = normal((wl.head_dim,), 1.0, wl.config_id, blk, name, False)
    return (np.float32(1.0) + np.float32(GAMMA_STD) * g).astype(np.float32)


def operands_bf16(wl: Workload) -> bool:
    return wl.precision != "f32"


def double_block_weights(wl: Workload, blk: int) -> Dict[str, np.ndarray]:
    """Per stream s in (img, txt): mod [6D, D] (chunks shift1, scale1, gate1,
    shift2, scale2, gate2), qkv [3D, D] (rows q|k|v, head-major inside each),
    q_norm/k_norm [Dh], proj [D, D], fc1 [F, D], fc2 [D, F]."""
    D, F, bf = wl.hidden, wl.mlp_hidden, operands_bf16(wl)
    w: Dict[str, np.ndarray] = {}
    for s in ("img", "txt"):
        w.update(_lin(wl, blk, s + "_mod", 6 * D, D, bf))
        w.update(_lin(wl, blk, s + "_qkv", 3 * D, D, bf))
        w[s + "_q_norm"] = _gamma(wl, blk, s + "_q_norm")
        w[s + "_k_norm"] = _gamma(wl, blk, s + "_k_norm")
        w.update(_lin(wl, blk, s + "_proj", D, D, bf))
        w.update(_lin(wl, blk, s + "_fc1", F, D, bf))
        w.update(_lin(wl, blk, s + "_fc2", D, F, bf))
    return w


def single_block_weights(wl: Workload, blk: int) -> Dict[str, np.ndarray]:
    """mod [3D, D] (shift, scale, gate), lin1 [3D+F, D] (rows q|k|v|mlp_in),
    q_norm/k_norm [Dh], lin2 [D, D+F] (input columns attn|gelu(mlp))."""
    D, F, bf = wl.hidden, wl.mlp_hidden, operands_bf16(wl)
    w: Dict[str, np.ndarray] = {}
    w.update(_lin(wl, blk, "mod", 3 * D, D, bf))
    w.update(_lin(wl, blk, "lin1", 3 * D + F, D, bf))
    w["q_norm"] = _gamma(wl, blk, "q_norm")
    w["k_norm"] = _gamma(wl, blk, "k_norm")
    w.update(_lin(wl, blk, "lin2", D, D + F, bf))
    return w


def single_seq_block_weights(wl: Workload, blk: int) -> Dict[str, np.ndarray]:
    """Sequential single block: mod [6D, D] (shift1, scale1, gate1, shift2,
    scale2, gate2), qkv [3D, D], q_norm/k_norm [Dh], proj [D, D], fc1 [F, D],
    fc2 [D, F] (one stream of a double block's shapes)."""
    D, F, bf = wl.hidden, wl.mlp_hidden, operands_bf16(wl)
    w: Dict[str, np.ndarray] = {}
    w.update(_lin(wl, blk, "seq_mod", 6 * D, D, bf))
    w.update(_lin(wl, blk, "seq_qkv", 3 * D, D, bf))
    w["seq_q_norm"] = _gamma(wl, blk, "seq_q_norm")
    w["seq_k_norm"] = _gamma(wl, blk, "seq_k_norm")
    w.update(_lin(wl, blk, "seq_proj", D, D, bf))
    w.update(_lin(wl, blk, "seq_fc1", F, D, bf))
    w.update(_lin(wl, blk, "seq_fc2", D, F, bf))
    return {k[len("seq_"):]: v for k, v in w.items()}


def embed_weights(wl: Workload, guidance: bool = False) -> Dict[str, np.ndarray]:
    """img_in [D, C]; txt_in [D, context] (if any); time_in 256->D->D;
    vector_in vec_in->D->D (if any); guidance_in [D, 1] (guidance=True);
    final mod [2D, D] (shift, scale); out [C, D]."""
    D, bf, blk = wl.hidden, operands_bf16(wl), 1000
    w: Dict[str, np.ndarray] = {}
    w.update(_lin(wl, blk, "img_in", D, wl.latent_ch, bf))
    if wl.context_dim is not None:
        w.update(_lin(wl, blk, "txt_in", D, wl.context_dim, bf))
    w.update(_lin(wl, blk, "time_in1", D, wl.model_channels, bf))
    w.update(_lin(wl, blk, "time_in2", D, D, bf))
    if wl.vec_in_dim is not None:
        w.update(_lin(wl, blk, "vector_in1", D, wl.vec_in_dim, bf))
        w.update(_lin(wl, blk, "vector_in2", D, D, bf))
    if guidance:
        w.update(_lin(wl, blk, "guidance_in", D, 1, bf))
    w.update(_lin(wl, blk, "final_mod", 2 * D, D, bf))
    w.update(_lin(wl, blk, "final_out", wl.latent_ch, D, bf))
    return w


def sampler_inputs(wl: Workload, n_images: int) -> Dict[str, np.ndarray]:
    """Inputs of classifier-free-guided sampling of n_images images with a
    model of batch 2 * n_images: noise z1 [n, C, H, W] N(0,1); the
    conditional text / pooled vector rows, then the null-prompt rows (the
    embeddings an empty prompt would give, drawn as their own N(0,1) tensors;
    no text encoder is part of the path); guidance values [2n] for the
    guidance embedding; joint position ids [2n, L, 3]."""
    C, bf = wl.latent_ch, operands_bf16(wl)
    width = wl.context_dim if wl.context_dim is not None else wl.hidden
    n = n_images
    d = {"z1": normal((n, C, wl.img_h, wl.img_w), 1.0, wl.config_id, 0, "sample_z1", False)}
    txt_c = normal((n, wl.l_txt, width), 1.0, wl.config_id, 0, "sample_txt", bf)
    txt_u = normal((n, wl.l_txt, width), 1.0, wl.config_id, 0, "sample_txt_null", bf)
    d["txt"] = np.concatenate([txt_c, txt_u], axis=0)
    if wl.vec_in_dim is not None:
        y_c = normal((n, wl.vec_in_dim), 1.0, wl.config_id, 0, "sample_y", False)
        y_u = normal((n, wl.vec_in_dim), 1.0, wl.config_id, 0, "sample_y_null", False)
        d["y"] = np.concatenate([y_c, y_u], axis=0)
    d["guidance"] = np.full(2 * n, 3.5, dtype=np.float32)
    ids = joint_ids(wl)
    d["ids"] = np.repeat(ids[:1], 2 * n, axis=0)
    return d


# --------------------------------------------------------------------------- #
# activations and conditioning
# --------------------------------------------------------------------------- #
def image_ids(batch: int, h: int, w: int, channel_group: bool = False) -> np.ndarray:
    """Position ids [B, h*w, 3] float32, row-major token order h*W + w.

    Axis 0 is 0 by default; with channel_group=True it is (h*W + w) // 16,
    the alternative the architecture page prints for the 3D RoPE ids."""
    ids = np.zeros((batch, h * w, 3), dtype=np.float32)
    r, c = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    ids[:, :, 1] = r.reshape(-1)
    ids[:, :, 2] = c.reshape(-1)
    if channel_group:
        ids[:, :, 0] = (np.arange(h * w) // 16).astype(np.float32)
    return ids


def text_ids(batch: int, l_txt: int) -> np.ndarray:
    return np.zeros((batch, l_txt, 3), dtype=np.float32)


def joint_ids(wl: Workload, channel_group: bool = False) -> np.ndarray:
    """[B, L_img + L_txt, 3]: image rows first, then text rows."""
    return np.concatenate([image_ids(wl.batch, wl.img_h, wl.img_w, channel_group),
                           text_ids(wl.batch, wl.l_txt)], axis=1)


def block_inputs(wl: Workload, blk: int = 0) -> Dict[str, np.ndarray]:
    """Residual-stream inputs of a block pair: x_img [B, L_img, D], x_txt
    [B, L_txt, D] fp32 N(0,1) and vec [B, D] fp32 N(0,1)."""
    D = wl.hidden
    return {
        "x_img": normal((wl.batch, wl.l_img, D), 1.0, wl.config_id, blk, "x_img", False),
        "x_txt": normal((wl.batch, wl.l_txt, D), 1.0, wl.config_id, blk, "x_txt", False),
        "vec": normal((wl.batch, D), 1.0, wl.config_id, blk, "vec", False),
    }


def timesteps(wl: Workload, name: str = "t") -> np.ndarray:
    """t in (0, 1): U(0,1), or the logit-normal draw t = 1/(1+exp(-u)),
    u ~ N(0,1), that the API page's LogitNormalSampler(mean 0, std 1) names."""
    if wl.t_dist == "uniform":
        return uniform01((wl.batch,), wl.config_id, 0, name)
    u = normal((wl.batch,), 1.0, wl.config_id, 0, name + ".u", False).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-u))).astype(np.float32)


def model_inputs(wl: Workload) -> Dict[str, np.ndarray]:
    """Inputs of a whole forward + loss: clean latents z0 and noise z1
    [B, C, H, W] fp32 N(0,1), t [B], text tokens [B, S, context or D]
    (bf16-rounded when the operands are bf16), pooled y [B, vec_in] and the
    joint position ids."""
    C, bf = wl.latent_ch, operands_bf16(wl)
    shp = (wl.batch, C, wl.img_h, wl.img_w)
    d: Dict[str, np.ndarray] = {
        "z0": normal(shp, 1.0, wl.config_id, 0, "z0", False),
        "z1": normal(shp, 1.0, wl.config_id, 0, "z1", False),
        "t": timesteps(wl),
        "ids": joint_ids(wl),
    }
    width = wl.context_dim if wl.context_dim is not None else wl.hidden
    d["txt"] = normal((wl.batch, wl.l_txt, width), 1.0, wl.config_id, 0, "txt", bf)
    if wl.vec_in_dim is not None:
        d["y"] = normal((wl.batch, wl.vec_in_dim), 1.0, wl.config_id, 0, "y", False)
    return d


def iter_block_weights(wl: Workload, workers: int = 8, window: int = 8):
    """Yield ("double", i, weights) for i < n_double, then ("single", i,
    weights) for i < n_single, in order, with block ids i (double) and
    n_double + i (single), the same host streams as double_block_weights /
    single_block_weights.  Up to `window` blocks are drawn ahead on `workers`
    threads (numpy's generators release the GIL while they fill arrays), so a
    caller can upload one block while the next ones are drawn; memory stays
    bounded by the window."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = [("double", i) for i in range(wl.n_double)] + [("single", i) for i in range(wl.n_single)]

    def draw(job):
        kind, i = job
        if kind == "double":
            return double_block_weights(wl, i)
        return single_block_weights(wl, wl.n_double + i)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        pending = [ex.submit(draw, j) for j in jobs[:window]]
        for n, job in enumerate(jobs):
            w = pending[n].result()
            pending[n] = None
            if n + window < len(jobs):
                pending.append(ex.submit(draw, jobs[n + window]))
            yield job[0], job[1], w


# --------------------------------------------------------------------------- #
# device-drawn block weights for the full 12B-shaped stack
# --------------------------------------------------------------------------- #
def device_stream_seed(config_id: int, block_id: int, name: str) -> int:
    """Seed of torch's device generator for one tensor (same key as the host
    streams)."""
    return int(np.random.SeedSequence([BASE_SEED, config_id, block_id, tensor_id(name)]).generate_state(1)[0])


def _device_normal(shape, std: float, wl: Workload, blk: int, name: str, dtype, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(device_stream_seed(wl.config_id, blk, name))
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(dtype)


def device_block_weights(wl: Workload, blk: int, kind: str, device="cuda", zero_mod: bool = False):
    """Weights of double ("double") or single ("single") block blk drawn on the
    device with torch's generator (Philox), for stacks too large to draw on the
    host (the 12B-shaped forward holds 11.8 B parameters).  Same shapes, names
    and distributions as double_block_weights / single_block_weights: linears
    and biases N(0, 0.02) in the operand type, RMSNorm scales 1 + 0.1 N(0, 1)
    in fp32.  zero_mod=True zeroes the modulation weights and biases (every
    shift, scale and gate is 0, so the block is the identity on its inputs).
    These arrays never reach the oracle."""
    import torch
    D, F = wl.hidden, wl.mlp_hidden
    dt = torch.bfloat16 if operands_bf16(wl) else torch.float32
    w = {}

    def lin(name, n_out, n_in, zero=False):
        if zero:
            w[name + ".w"] = torch.zeros((n_out, n_in), dtype=dt, device=device)
            w[name + ".b"] = torch.zeros((n_out,), dtype=dt, device=device)
        else:
            w[name + ".w"] = _device_normal((n_out, n_in), WEIGHT_STD, wl, blk, name + ".w", dt, device)
            w[name + ".b"] = _device_normal((n_out,), WEIGHT_STD, wl, blk, name + ".b", dt, device)

    def gamma(name):
        w[name] = 1.0 + GAMMA_STD * _device_normal((wl.head_dim,), 1.0, wl, blk, name, torch.float32, device)

    if kind == "double":
        for s in ("img", "txt"):
            lin(s + "_mod", 6 * D, D, zero_mod)
            lin(s + "_qkv", 3 * D, D)
            gamma(s + "_q_norm")
            gamma(s + "_k_norm")
            lin(s + "_proj", D, D)
            lin(s + "_fc1", F, D)
            lin(s + "_fc2", D, F)
    else:
        lin("mod", 3 * D, D, zero_mod)
        lin("lin1", 3 * D + F, D)
        gamma("q_norm")
        gamma("k_norm")
        lin("lin2", D, D + F)
    return w
