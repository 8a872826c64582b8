"""Device-side composition of the Flux forward over the libflux C ABI.

This module only uploads arrays, allocates device buffers with torch and calls
the library in order ("Flux architecture deep dive", Data flow / Complete
forward pass and Training data flow): rf noising -> input embeddings and
conditioning vector -> double blocks -> single blocks over the joint sequence
-> output head -> velocity MSE.  No arithmetic of the method happens here.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np
import torch

from . import flux as F
from . import synth


def _check_text(txt, dtype) -> None:
    """The text tokens' element type follows the precision (flux_embed_fwd);
    the library reads them as that type, so a mismatch is refused here."""
    if txt.dtype != dtype:
        raise ValueError(f"text tokens must be {dtype}, got {txt.dtype}")


def device_array(a: np.ndarray, bf16: bool, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(device)
    return t.to(torch.bfloat16) if bf16 else t


def upload_weights(w: Dict[str, np.ndarray], bf16: bool, device="cuda") -> Dict[str, torch.Tensor]:
    """Linear weights/biases in the operand type; RMSNorm scales stay float.
    Tensors already on the device (drawn there) are taken as they are."""
    out = {}
    for k, v in w.items():
        if isinstance(v, torch.Tensor):
            out[k] = v
            continue
        is_norm = k.endswith("_norm") or k in ("q_norm", "k_norm")
        out[k] = device_array(v, bf16 and not is_norm, device)
    return out


def precision_of(wl: synth.Workload) -> int:
    """Precision of the embedding / head calls (fp8 workloads keep those in bf16)."""
    return F.FLUX_PREC_F32 if wl.precision == "f32" else F.FLUX_PREC_BF16


class Workspace:
    """One device scratch buffer, grown on demand (256-byte aligned)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


# the block linears whose weights may be held in fp16 (not the modulation GEMVs)
LINEARS = ("img_qkv.w", "img_proj.w", "img_fc1.w", "img_fc2.w", "txt_qkv.w", "txt_proj.w", "txt_fc1.w", "txt_fc2.w",
           "lin1.w", "lin2.w", "qkv.w", "proj.w", "fc1.w", "fc2.w")


def to_f16_weights(w: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    """One-time device conversion of the block linears' bf16 weights to fp16
    (flux_convert_bf16_to_f16); everything else is kept as is."""
    out = dict(w)
    for k in LINEARS:
        if k in w:
            dst = torch.empty(w[k].shape, dtype=torch.float16, device=w[k].device)
            F.flux_convert_bf16_to_f16(w[k], dst, w[k].numel())
            out[k] = dst
    return out


# token-path linears of a double-block stream and of a single block, in the
# order of their fp8 state slots (input X then weight W of each)
FP8_DOUBLE = ("qkv", "proj", "fc1", "fc2")
FP8_SINGLE = ("lin1", "lin2")


class BlockStack:
    """Double and single blocks of one workload, weights resident on the GPU.

    weights_f16: hold the block linears' weights in fp16, converted once here,
    instead of converting bf16 tiles inside every GEMM (bf16 workloads only).

    fp8 workloads keep bf16 master weights and E4M3 copies of the token-path
    linears, plus one zero-initialised delayed-scaling state buffer: 8 records
    per double-block stream (image then text), 4 per single block.  A forward
    under the recipe is fp8_cast_weights() -> blocks -> fp8_update()."""

    def __init__(self, wl: synth.Workload, double_ws: List[Dict[str, np.ndarray]],
                 single_ws: List[Dict[str, np.ndarray]], device="cuda", weights_f16: bool = False):
        self.wl = wl
        self.bf16 = wl.precision != "f32"
        self.fp8 = wl.precision == "fp8"
        weights_f16 = weights_f16 and wl.precision == "bf16"
        self.dims = F.dims_for(wl, weights_f16=weights_f16)
        self.double = [upload_weights(w, self.bf16, device) for w in double_ws]
        self.single = [upload_weights(w, self.bf16, device) for w in single_ws]
        if weights_f16:
            self.double = [to_f16_weights(w) for w in self.double]
            self.single = [to_f16_weights(w) for w in self.single]
            torch.cuda.synchronize()   # the bf16 sources of the conversions may be freed by the caller
        # a single block whose weights hold "qkv.w" is the sequential form
        # (flux_single_seq_fwd: one stream of a double block over the joint
        # sequence); otherwise the fused parallel form (flux_single_fwd)
        self.single_seq = ["qkv.w" in w for w in single_ws]
        self.fp8_state = None
        if self.fp8:
            n_single = [len(F.FP8_STREAM_SLOTS) if q else len(F.FP8_SINGLE_SLOTS) for q in self.single_seq]
            n = len(self.double) * 2 * len(F.FP8_STREAM_SLOTS) + sum(n_single)
            self.fp8_tensors = n
            self.fp8_state = torch.zeros(F.flux_fp8_state_bytes(n), dtype=torch.uint8, device=device)
            self._fp8_casts = []           # (master bf16, e4m3 copy, W record address)
            self._dq = [self._fp8_copies(w, ("img", "txt"), FP8_DOUBLE, 2 * 8 * i, 8)
                        for i, w in enumerate(self.double)]
            first = [len(self.double) * 16 + sum(n_single[:i]) for i in range(len(self.single))]
            self._sq = [self._fp8_copies(w, (None,), FP8_DOUBLE if q else FP8_SINGLE, f, 8 if q else 4)
                        for w, q, f in zip(self.single, self.single_seq, first)]
            self._dstructs = [(F.stream_weights(q, "img", self.fp8_record(2 * 8 * i)),
                               F.stream_weights(q, "txt", self.fp8_record(2 * 8 * i + 8)))
                              for i, q in enumerate(self._dq)]
            self._sstructs = [F.stream_weights(w, None, self.fp8_record(f)) if q else
                              F.single_weights(w, self.fp8_record(f))
                              for w, q, f in zip(self._sq, self.single_seq, first)]
        else:
            self._dstructs = [(F.stream_weights(w, "img"), F.stream_weights(w, "txt")) for w in self.double]
            self._sstructs = [F.stream_weights(w, None) if q else F.single_weights(w)
                              for w, q in zip(self.single, self.single_seq)]
        self.ws = Workspace(device)
        self.ws_bytes = max(F.flux_workspace_bytes(self.dims, op) for op in (0, 1, 2))
        self.device = device

    # ------------------------------------------------------------------ fp8
    def fp8_record(self, index: int) -> int:
        """Device address of state record `index`."""
        return self.fp8_state.data_ptr() + index * F.FP8_TENSOR_BYTES

    def _fp8_copies(self, w, prefixes, names, first, per_prefix):
        """Dict like w with the token-path linear weights replaced by E4M3
        copies (filled by fp8_cast_weights)."""
        out = dict(w)
        for pi, pre in enumerate(prefixes):
            for li, n in enumerate(names):
                key = f"{pre}_{n}.w" if pre else f"{n}.w"
                if key not in w:
                    continue
                q = torch.empty(w[key].shape, dtype=torch.uint8, device=w[key].device)
                out[key] = q
                self._fp8_casts.append((w[key], q, self.fp8_record(first + pi * per_prefix + 2 * li + 1)))
        return out

    def fp8_cast_weights(self) -> None:
        """Quantize every token-path weight with its record's current scale
        (and record its amax): the weight cast of a forward."""
        for src, dst, rec in self._fp8_casts:
            F.flux_fp8_quantize(F.FLUX_PREC_BF16, src, src.numel(), rec, dst)

    def fp8_update(self, algo: int = 0, margin: int = 0) -> None:
        """Delayed-scaling update of every record after a forward."""
        F.flux_fp8_update(self.fp8_state, self.fp8_tensors, algo, margin)

    def fp8_records(self) -> List[dict]:
        raw = self.fp8_state.cpu().numpy().tobytes()
        return [F.fp8_record_fields(raw[i * F.FP8_TENSOR_BYTES:(i + 1) * F.FP8_TENSOR_BYTES])
                for i in range(self.fp8_tensors)]

    def rope_table(self, ids: torch.Tensor) -> torch.Tensor:
        wl = self.wl
        B, L = ids.shape[0], ids.shape[1]
        table = torch.empty((B, L, wl.head_dim // 2, 2), dtype=torch.float32, device=self.device)
        F.flux_rope_table(ids, B, L, wl.axes_dim, wl.theta, table)
        return table

    def double_fwd(self, i: int, x: torch.Tensor, vec: torch.Tensor, rope: torch.Tensor) -> None:
        """x: joint [B, L, D] float residual (image rows then text rows), in place."""
        wl = self.wl
        L = wl.seq
        iw, tw = self._dstructs[i]
        ws = self.ws.get(self.ws_bytes)
        txt = x[:, wl.l_img:] if wl.l_txt > 0 else None
        F.flux_block_fwd(self.dims, iw, tw, x, L * wl.hidden, txt, L * wl.hidden, vec, rope, ws, ws.numel())

    def single_fwd(self, i: int, x: torch.Tensor, vec: torch.Tensor, rope: torch.Tensor) -> None:
        wl = self.wl
        ws = self.ws.get(self.ws_bytes)
        fwd = F.flux_single_seq_fwd if self.single_seq[i] else F.flux_single_fwd
        fwd(self.dims, self._sstructs[i], x, wl.seq * wl.hidden, vec, rope, ws, ws.numel())

    # fp8: re-cast the weights with their current scales on every forward (a
    # training step changes them); a caller with static weights may switch
    # this off once the weight scales have settled (after the first update the
    # scale of a static weight is 448 / amax and stays there)
    cast_each_forward = True

    def blocks_fwd(self, x: torch.Tensor, vec: torch.Tensor, rope: torch.Tensor) -> None:
        """All blocks in order; fp8 workloads cast the weights first and
        update the scales after."""
        if self.fp8 and self.cast_each_forward:
            self.fp8_cast_weights()
        for i in range(len(self.double)):
            self.double_fwd(i, x, vec, rope)
        for i in range(len(self.single)):
            self.single_fwd(i, x, vec, rope)
        if self.fp8:
            self.fp8_update()


class FluxModel(BlockStack):
    """Whole forward + rectified-flow loss of a workload."""

    def __init__(self, wl: synth.Workload, emb_w: Dict[str, np.ndarray], double_ws, single_ws, device="cuda",
                 weights_f16: bool = False):
        super().__init__(wl, double_ws, single_ws, device, weights_f16)
        self.emb = upload_weights(emb_w, self.bf16, device)
        self._estruct = F.embed_weights(self.emb)
        p = precision_of(wl)
        self.ws_bytes = max(self.ws_bytes,
                            F.flux_embed_workspace_bytes(p, wl.batch, wl.latent_ch, wl.img_h, wl.img_w, wl.hidden),
                            F.flux_final_workspace_bytes(p, wl.batch, wl.img_h, wl.img_w, wl.hidden),
                            F.flux_rf_workspace_bytes(wl.batch, wl.latent_ch * wl.l_img))

    def _buffers(self, ids, o: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
        wl, dev = self.wl, self.device
        B, C, D = wl.batch, wl.latent_ch, wl.hidden
        if not o:
            f32 = dict(dtype=torch.float32, device=dev)
            o["z_t"] = torch.empty((B, C, wl.img_h, wl.img_w), **f32)
            o["v_target"] = torch.empty_like(o["z_t"])
            o["x"] = torch.empty((B, wl.seq, D), **f32)
            o["vec"] = torch.empty((B, D), **f32)
            o["v_pred"] = torch.empty_like(o["z_t"])
            o["loss"] = torch.empty((1,), **f32)
            o["loss_per_sample"] = torch.empty((B,), **f32)
            o["rope"] = self.rope_table(ids)
        return o

    def _forward(self, o, z_t, t, txt, y, guidance=None) -> None:
        """Embeddings, blocks, output head: v_pred of z_t at times t into o."""
        wl = self.wl
        B, C, D = wl.batch, wl.latent_ch, wl.hidden
        p = precision_of(wl)
        ws = self.ws.get(self.ws_bytes)
        x = o["x"]
        # text enters through txt_in, or at the hidden width (the library then copies it into the joint buffer)
        _check_text(txt, torch.bfloat16 if p == F.FLUX_PREC_BF16 else torch.float32)
        F.flux_embed_fwd(p, B, C, wl.img_h, wl.img_w, wl.l_txt, wl.context_dim or 0, D, wl.model_channels,
                         wl.vec_in_dim or 0, self._estruct, z_t, txt, t, y, x, wl.seq * D, x[:, wl.l_img:],
                         wl.seq * D, o["vec"], ws, ws.numel(), guidance=guidance)
        self.blocks_fwd(x, o["vec"], o["rope"])
        F.flux_final_fwd(p, B, C, wl.img_h, wl.img_w, D, wl.eps, self.emb["final_mod.w"], self.emb["final_mod.b"],
                         self.emb["final_out.w"], self.emb["final_out.b"], x, wl.seq * D, o["vec"], o["v_pred"], ws,
                         ws.numel())

    def forward_loss(self, z0, z1, t, txt, y, ids, out: Optional[Dict[str, torch.Tensor]] = None):
        """Noise, forward, loss.  Returns a dict of device tensors: z_t, v_target,
        x (joint residual after the blocks), vec, v_pred, loss, loss_per_sample."""
        wl = self.wl
        B, n = wl.batch, wl.latent_ch * wl.l_img
        o = self._buffers(ids, out if out is not None else {})
        ws = self.ws.get(self.ws_bytes)
        F.rf_noise_loss(B, n, z0, z1, t, z_t=o["z_t"], v_target=o["v_target"])
        self._forward(o, o["z_t"], t, txt, y)
        F.rf_noise_loss(B, n, z0, z1, t, v_pred=o["v_pred"], loss=o["loss"], loss_per_sample=o["loss_per_sample"],
                        workspace=ws, workspace_bytes=ws.numel())
        return o

    def forward(self, z_t, t, txt, y, ids, guidance=None, out: Optional[Dict[str, torch.Tensor]] = None):
        """Velocity of z_t at times t (the model call of a sampler)."""
        o = self._buffers(ids, out if out is not None else {})
        self._forward(o, z_t, t, txt, y, guidance)
        return o

    def sample(self, z1, n_steps: int, txt, y, ids, cfg_w: Optional[float] = None, guidance=None,
               out: Optional[Dict[str, torch.Tensor]] = None, steps=None):
        """Euler sampling from noise z1 [B', C, H, W] at t = 1 down to t = 0 on
        the uniform grid of n_steps steps ("Flux architecture deep dive",
        Sampling (inference)).  With cfg_w the model batch is 2B' (this
        model's workload batch): txt / y hold the conditional rows then the
        unconditional (null prompt) rows, and each step combines the two
        velocities by classifier-free guidance in the step kernel.  Without
        cfg_w the model batch is B'.  guidance: optional [batch] device values
        for the guidance embedding.  steps: optional range of step indices to
        run (default all), for timing a subset.  Returns the state dict; "z"
        holds the sample."""
        wl = self.wl
        cfg = cfg_w is not None
        Bm = wl.batch
        Bs = Bm // 2 if cfg else Bm
        assert not cfg or Bm % 2 == 0, "classifier-free guidance needs an even model batch"
        n = wl.latent_ch * wl.l_img
        o = self._buffers(ids, out if out is not None else {})
        if "z" not in o:
            o["z"] = torch.empty((Bs,) + tuple(z1.shape[1:]), dtype=torch.float32, device=self.device)
            o["t"] = torch.empty((Bm,), dtype=torch.float32, device=self.device)
        ts = [1.0 - i / n_steps for i in range(n_steps + 1)]
        run = range(n_steps) if steps is None else steps
        for i in run:
            if i == 0:
                # the model input at t = 1 is the noise itself, in every batch half
                o["z"].copy_(z1)
                o["z_t"][:Bs].copy_(z1)
                if cfg:
                    o["z_t"][Bs:].copy_(z1)
                o["t"].fill_(ts[0])
            self._forward(o, o["z_t"], o["t"], txt, y, guidance)
            F.flux_euler_step(Bs, n, o["v_pred"], o["z"], ts[i], ts[i + 1], cfg=cfg,
                              guidance=cfg_w if cfg else 1.0, z_model=o["z_t"], copies=2 if cfg else 1,
                              t_model=o["t"], t_model_n=Bm)
        return o


class BlockPairTrainer:
    """Training forward and backward of one double block followed by one
    single block over the joint [B, L_img + L_txt, D] residual (bf16, head_dim
    128): the training forwards keep their activations in `saved` buffers,
    the backwards turn the output gradient into the input gradient in place
    and write every parameter gradient (fp32, keyed like the weights) and the
    vec gradient (accumulated into dvec)."""

    def __init__(self, wl: synth.Workload, w2: Dict[str, object], w1: Dict[str, object], device="cuda"):
        self.wl = wl
        self.dims = F.dims_for(wl)
        self.w2 = upload_weights(w2, True, device)
        self.w1 = upload_weights(w1, True, device)
        self.iw, self.tw = F.stream_weights(self.w2, "img"), F.stream_weights(self.w2, "txt")
        self.sw = F.single_weights(self.w1)
        nb = [F.flux_train_saved_bytes(self.dims, op) for op in (0, 1)]
        if min(nb) == 0:
            raise F.FluxError(F.FLUX_ERR_UNSUPPORTED, "BlockPairTrainer", F.lib().flux_last_error().decode())
        self.saved = [torch.empty(n, dtype=torch.uint8, device=device) for n in nb]
        self.ws_bytes = max(F.flux_bwd_workspace_bytes(self.dims, op) for op in (0, 1))
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.g2 = {k: torch.empty(tuple(v.shape), dtype=torch.float32, device=device) for k, v in self.w2.items()}
        self.g1 = {k: torch.empty(tuple(v.shape), dtype=torch.float32, device=device) for k, v in self.w1.items()}
        self.gi, self.gt = F.stream_grads(self.g2, "img"), F.stream_grads(self.g2, "txt")
        self.gs = F.single_grads(self.g1)

    def forward(self, x: torch.Tensor, vec: torch.Tensor, rope: torch.Tensor) -> None:
        wl = self.wl
        L, D = wl.seq, wl.hidden
        txt = x.data_ptr() + wl.l_img * D * 4
        F.flux_block_fwd_train(self.dims, self.iw, self.tw, x, L * D, txt, L * D, vec, rope, self.saved[0],
                               self.saved[0].numel())
        F.flux_single_fwd_train(self.dims, self.sw, x, L * D, vec, rope, self.saved[1], self.saved[1].numel())

    def backward(self, d: torch.Tensor, vec: torch.Tensor, rope: torch.Tensor, dvec: torch.Tensor) -> None:
        wl = self.wl
        L, D = wl.seq, wl.hidden
        F.flux_single_bwd(self.dims, self.sw, d, L * D, vec, rope, self.saved[1], self.saved[1].numel(), self.gs,
                          dvec, self.ws, self.ws_bytes)
        F.flux_block_bwd(self.dims, self.iw, self.tw, d, L * D, d.data_ptr() + wl.l_img * D * 4, L * D, vec, rope,
                         self.saved[0], self.saved[0].numel(), self.gi, self.gt, dvec, self.ws, self.ws_bytes)


class FluxTrainer:
    """One rectified-flow training step of a whole (bf16, head_dim 128) model:
    noising, input embeddings, double blocks, single blocks (fused form) and
    the output head with their training forwards, the velocity MSE, then the
    backward in reverse order -- the loss gradient, the head, every block and
    the embeddings -- leaving the fp32 gradient of every weight in `grads`
    (embeddings and head), `g_double[i]` and `g_single[i]`.  When the
    embedding weights hold the guidance embedding, step() takes the guidance
    values and its gradients join `grads`."""

    def __init__(self, wl: synth.Workload, emb_w: Dict[str, object], double_ws, single_ws, device="cuda"):
        self.wl, self.device = wl, device
        B, C, D = wl.batch, wl.latent_ch, wl.hidden
        self.dims = F.dims_for(wl)
        self.emb = upload_weights(emb_w, True, device)
        self.estruct = F.embed_weights(self.emb)
        self.dw = [upload_weights(w, True, device) for w in double_ws]
        self.sw = [upload_weights(w, True, device) for w in single_ws]
        self.dstructs = [(F.stream_weights(w, "img"), F.stream_weights(w, "txt")) for w in self.dw]
        self.sstructs = [F.single_weights(w) for w in self.sw]
        f32 = dict(dtype=torch.float32, device=device)
        grad = lambda w: {k: torch.empty(tuple(v.shape), **f32) for k, v in w.items()}
        self.grads = grad(self.emb)
        self.g_double = [grad(w) for w in self.dw]
        self.g_single = [grad(w) for w in self.sw]
        self.gstructs = ([(F.stream_grads(g, "img"), F.stream_grads(g, "txt")) for g in self.g_double],
                         [F.single_grads(g) for g in self.g_single])
        self.egrads = F.embed_grads(self.grads)
        saved = lambda op: torch.empty(F.flux_train_saved_bytes(self.dims, op), dtype=torch.uint8, device=device)
        self.saved_d = [saved(0) for _ in self.dw]
        self.saved_s = [saved(1) for _ in self.sw]
        ctx = wl.context_dim or 0
        self.ws_bytes = max(F.flux_bwd_workspace_bytes(self.dims, 0), F.flux_bwd_workspace_bytes(self.dims, 1),
                            F.flux_embed_workspace_bytes(F.FLUX_PREC_BF16, B, C, wl.img_h, wl.img_w, D),
                            F.flux_final_workspace_bytes(F.FLUX_PREC_BF16, B, wl.img_h, wl.img_w, D),
                            F.flux_rf_workspace_bytes(B, C * wl.l_img),
                            F.flux_final_bwd_workspace_bytes(B, C, wl.img_h, wl.img_w, D),
                            F.flux_embed_bwd_workspace_bytes(B, C, wl.img_h, wl.img_w, wl.l_txt, ctx, D))
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        shp = (B, C, wl.img_h, wl.img_w)
        self.o = {"z_t": torch.empty(shp, **f32), "v_target": torch.empty(shp, **f32),
                  "v_pred": torch.empty(shp, **f32), "dv": torch.empty(shp, **f32),
                  "x": torch.empty((B, wl.seq, D), **f32), "d": torch.empty((B, wl.seq, D), **f32),
                  "vec": torch.empty((B, D), **f32), "dvec": torch.empty((B, D), **f32),
                  "loss": torch.empty((1,), **f32), "loss_per_sample": torch.empty((B,), **f32)}
        self.rope = None

    def step(self, z0, z1, t, txt, y, ids, guidance=None) -> torch.Tensor:
        """Returns the loss (a device tensor); gradients land in the grad dicts.
        guidance: [batch] float device values, required exactly when the model
        has the guidance embedding."""
        if (guidance is None) == ("guidance_in.w" in self.emb):
            raise ValueError("guidance values are needed exactly when the model has a guidance embedding")
        wl, o, ws = self.wl, self.o, self.ws
        B, C, D, L, Li = wl.batch, wl.latent_ch, wl.hidden, wl.seq, wl.l_img
        n = C * Li
        bf = F.FLUX_PREC_BF16
        if self.rope is None:
            self.rope = torch.empty((B, L, wl.head_dim // 2, 2), dtype=torch.float32, device=self.device)
            F.flux_rope_table(ids, B, L, wl.axes_dim, wl.theta, self.rope)
        x, d, vec, dvec = o["x"], o["d"], o["vec"], o["dvec"]
        txt_ptr = x.data_ptr() + Li * D * 4
        d_txt_ptr = d.data_ptr() + Li * D * 4
        _check_text(txt, torch.bfloat16)
        F.rf_noise_loss(B, n, z0, z1, t, z_t=o["z_t"], v_target=o["v_target"])
        F.flux_embed_fwd(bf, B, C, wl.img_h, wl.img_w, wl.l_txt, wl.context_dim or 0, D, wl.model_channels,
                         wl.vec_in_dim or 0, self.estruct, o["z_t"], txt, t, y, x, L * D, txt_ptr, L * D, vec, ws,
                         self.ws_bytes, guidance=guidance)
        for (iw, tw), sv in zip(self.dstructs, self.saved_d):
            F.flux_block_fwd_train(self.dims, iw, tw, x, L * D, txt_ptr, L * D, vec, self.rope, sv, sv.numel())
        for sw, sv in zip(self.sstructs, self.saved_s):
            F.flux_single_fwd_train(self.dims, sw, x, L * D, vec, self.rope, sv, sv.numel())
        e = self.emb
        F.flux_final_fwd(bf, B, C, wl.img_h, wl.img_w, D, wl.eps, e["final_mod.w"], e["final_mod.b"], e["final_out.w"],
                         e["final_out.b"], x, L * D, vec, o["v_pred"], ws, self.ws_bytes)
        F.rf_noise_loss(B, n, z0, z1, t, v_pred=o["v_pred"], loss=o["loss"], loss_per_sample=o["loss_per_sample"],
                        workspace=ws, workspace_bytes=self.ws_bytes)
        # backward
        F.flux_rf_loss_grad(B, n, o["v_pred"], z0, z1, o["dv"])
        d.zero_()
        dvec.zero_()
        g = self.grads
        F.flux_final_bwd(B, C, wl.img_h, wl.img_w, D, wl.eps, e["final_mod.w"], e["final_mod.b"], e["final_out.w"], x,
                         L * D, vec, o["dv"], d, dvec, g["final_mod.w"], g["final_mod.b"], g["final_out.w"],
                         g["final_out.b"], ws, self.ws_bytes)
        dstr, sstr = self.gstructs
        for sw, sv, gs in reversed(list(zip(self.sstructs, self.saved_s, sstr))):
            F.flux_single_bwd(self.dims, sw, d, L * D, vec, self.rope, sv, sv.numel(), gs, dvec, ws, self.ws_bytes)
        for (iw, tw), sv, (gi, gt) in reversed(list(zip(self.dstructs, self.saved_d, dstr))):
            F.flux_block_bwd(self.dims, iw, tw, d, L * D, d_txt_ptr, L * D, vec, self.rope, sv, sv.numel(), gi, gt,
                             dvec, ws, self.ws_bytes)
        has_txt_in = "txt_in.w" in self.emb
        F.flux_embed_bwd(B, C, wl.img_h, wl.img_w, wl.l_txt, wl.context_dim or 0, D, wl.model_channels,
                         wl.vec_in_dim or 0, self.estruct, o["z_t"], txt if has_txt_in else None, t, y, d, L * D,
                         d_txt_ptr if has_txt_in else None, L * D, dvec, self.egrads, ws, self.ws_bytes,
                         guidance=guidance)
        return o["loss"]
