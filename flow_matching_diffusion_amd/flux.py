"""ctypes binding of libflux (include/flux.h).  Argument marshalling only:
every step of the computation runs in the HIP library.  Loading fails loudly
when the library has not been built; there is no fallback implementation.

Tensors are passed as torch tensors on the GPU (their data_ptr() is handed to
the library) or as raw integer device addresses; the stream defaults to
torch's current stream.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflux.so")

FLUX_OK = 0
FLUX_ERR_INVALID_ARGUMENT = 1
FLUX_ERR_UNSUPPORTED = 2
FLUX_ERR_WORKSPACE_TOO_SMALL = 3
FLUX_ERR_HIP = 4
FLUX_PREC_F32 = 0
FLUX_PREC_BF16 = 1
FLUX_PREC_FP8_E4M3 = 2

# flux_fp8_tensor: 8 words of state then the 1024-entry amax history
FLUX_FP8_HISTORY = 1024
FLUX_FP8_SCALE_SET = 1
FLUX_FP8_NONFINITE = 2
FP8_TENSOR_BYTES = 32 + 4 * FLUX_FP8_HISTORY
FP8_STREAM_SLOTS = ("qkv_x", "qkv_w", "proj_x", "proj_w", "fc1_x", "fc1_w", "fc2_x", "fc2_w")
FP8_SINGLE_SLOTS = ("lin1_x", "lin1_w", "lin2_x", "lin2_w")

# every symbol include/flux.h declares
EXPORTED = (
    "flux_block_fwd", "flux_single_fwd", "flux_single_seq_fwd", "rf_noise_loss", "flux_rope_table", "flux_embed_fwd",
    "flux_final_fwd", "flux_linear_fwd", "flux_attention_fwd", "flux_workspace_bytes",
    "flux_rf_workspace_bytes", "flux_embed_workspace_bytes", "flux_final_workspace_bytes",
    "flux_attention_workspace_bytes", "flux_status_string", "flux_last_error", "flux_timing_enable",
    "flux_timing_classes", "flux_timing_class_name", "flux_timing_read", "flux_convert_bf16_to_f16",
    "flux_fp8_state_bytes", "flux_fp8_quantize", "flux_fp8_update", "flux_fp8_linear_fwd", "flux_euler_step",
    "flux_mx_scale_bytes", "flux_mx_quantize", "flux_mxfp8_linear_fwd", "flux_fp8_quantize_current",
    "flux_train_saved_bytes", "flux_bwd_workspace_bytes", "flux_block_fwd_train", "flux_block_bwd",
    "flux_single_fwd_train", "flux_single_bwd", "flux_attention_train_workspace_bytes", "flux_attention_fwd_train",
    "flux_attention_bwd", "flux_rf_loss_grad", "flux_final_bwd_workspace_bytes", "flux_final_bwd",
    "flux_embed_bwd_workspace_bytes", "flux_embed_bwd", "flux_single_seq_fwd_train", "flux_single_seq_bwd",
    "flux_attention_fp8_workspace_bytes", "flux_attention_fp8_fwd", "flux_mxfp4_scale_bytes", "flux_mxfp4_quantize",
    "flux_mxfp4_linear_fwd", "flux_fp8_block_quantize", "flux_timestep_embed", "rf_noise_loss_noalloc",
    "flux_rf_noalloc_max_partials", "flux_timing_flush", "flux_stream_copy", "flux_debug_checks",
    "flux_debug_status", "flux_gemm_stream_k",
)


class FluxError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({_status_name(status)}): {detail}")
        self.status = status


def _status_name(s: int) -> str:
    return {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error"}.get(s, "?")


# --------------------------------------------------------------------------- #
# C structs (mirror include/flux.h)
# --------------------------------------------------------------------------- #
class flux_dims(C.Structure):
    _fields_ = [("batch", C.c_int32), ("l_img", C.c_int32), ("l_txt", C.c_int32), ("hidden", C.c_int32),
                ("heads", C.c_int32), ("head_dim", C.c_int32), ("mlp_hidden", C.c_int32),
                ("axes_dim", C.c_int32 * 3), ("theta", C.c_float), ("eps", C.c_float), ("precision", C.c_int32),
                ("weights_f16", C.c_int32)]


class flux_stream_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("mod_w", "mod_b", "qkv_w", "qkv_b", "q_norm", "k_norm", "proj_w",
                                          "proj_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b", "fp8")]


class flux_single_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("mod_w", "mod_b", "lin1_w", "lin1_b", "q_norm", "k_norm", "lin2_w",
                                          "lin2_b", "fp8")]


class flux_stream_grads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("mod_w", "mod_b", "qkv_w", "qkv_b", "q_norm", "k_norm", "proj_w",
                                          "proj_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")]


class flux_single_grads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("mod_w", "mod_b", "lin1_w", "lin1_b", "q_norm", "k_norm", "lin2_w",
                                          "lin2_b")]


class flux_embed_grads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("img_in_w", "img_in_b", "txt_in_w", "txt_in_b", "time_in1_w",
                                          "time_in1_b", "time_in2_w", "time_in2_b", "vector_in1_w",
                                          "vector_in1_b", "vector_in2_w", "vector_in2_b", "guidance_in_w",
                                          "guidance_in_b")]


class rf_args(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_per_sample", C.c_int64), ("z0", C.c_void_p), ("z1", C.c_void_p),
                ("t", C.c_void_p), ("z_t", C.c_void_p), ("v_target", C.c_void_p), ("v_pred", C.c_void_p),
                ("loss", C.c_void_p), ("loss_per_sample", C.c_void_p), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_size_t)]


class flux_embed_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("img_in_w", "img_in_b", "txt_in_w", "txt_in_b", "time_in1_w",
                                          "time_in1_b", "time_in2_w", "time_in2_b", "vector_in1_w",
                                          "vector_in1_b", "vector_in2_w", "vector_in2_b", "guidance_in_w",
                                          "guidance_in_b")]


class flux_euler_args(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_per_sample", C.c_int64), ("v", C.c_void_p), ("cfg", C.c_int32),
                ("guidance", C.c_float), ("t_cur", C.c_float), ("t_next", C.c_float), ("z", C.c_void_p),
                ("z_model", C.c_void_p), ("copies", C.c_int32), ("t_model", C.c_void_p), ("t_model_n", C.c_int32)]


# --------------------------------------------------------------------------- #
# library loading
# --------------------------------------------------------------------------- #
_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m flow_matching_diffusion_amd.build` "
                           "(there is no CPU fallback)")
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
    P = C.POINTER
    sig = {
        "flux_block_fwd": [P(flux_dims), P(flux_stream_weights), P(flux_stream_weights), vp, i64, vp, i64, vp, vp,
                           vp, sz, vp],
        "flux_single_fwd": [P(flux_dims), P(flux_single_weights), vp, i64, vp, vp, vp, sz, vp],
        "flux_single_seq_fwd": [P(flux_dims), P(flux_stream_weights), vp, i64, vp, vp, vp, sz, vp],
        "rf_noise_loss": [P(rf_args), vp],
        "rf_noise_loss_noalloc": [P(rf_args), vp],
        "flux_timing_flush": [vp, i64],
        "flux_stream_copy": [vp, vp, i64, vp],
        "flux_debug_checks": [i32],
        "flux_gemm_stream_k": [i32, i32],
        "flux_debug_status": [P(C.c_uint32), i32],
        "flux_rope_table": [vp, i32, i32, P(C.c_int32), f32, vp, vp],
        "flux_embed_fwd": [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, P(flux_embed_weights), vp, vp, vp, vp,
                           vp, vp, i64, vp, i64, vp, vp, sz, vp],
        "flux_euler_step": [P(flux_euler_args), vp],
        "flux_mx_quantize": [i32, vp, i32, i32, vp, vp, vp],
        "flux_mxfp8_linear_fwd": [i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, vp],
        "flux_mxfp4_quantize": [i32, vp, i32, i32, vp, vp, vp],
        "flux_fp8_block_quantize": [i32, vp, i32, i32, i32, vp, vp, vp],
        "flux_timestep_embed": [vp, i32, i32, f32, vp, vp],
        "flux_mxfp4_linear_fwd": [i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, vp],
        "flux_final_fwd": [i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, i64, vp, vp, vp, sz, vp],
        "flux_linear_fwd": [i32, i32, i32, i32, vp, i64, vp, vp, vp, i64, vp],
        "flux_attention_fwd": [i32, i32, i32, i32, i32, vp, vp, vp, i64, vp, i64, vp, sz, vp],
        "flux_convert_bf16_to_f16": [vp, vp, i64, vp],
        "flux_fp8_quantize": [i32, vp, i64, vp, vp, vp],
        "flux_fp8_quantize_current": [i32, vp, i64, vp, vp, vp],
        "flux_fp8_update": [vp, i32, i32, i32, vp],
        "flux_fp8_linear_fwd": [i32, i32, i32, vp, i64, vp, i64, vp, vp, vp, vp, i64, vp],
        "flux_block_fwd_train": [P(flux_dims), P(flux_stream_weights), P(flux_stream_weights), vp, i64, vp, i64, vp,
                                 vp, vp, sz, vp],
        "flux_block_bwd": [P(flux_dims), P(flux_stream_weights), P(flux_stream_weights), vp, i64, vp, i64, vp, vp, vp,
                           sz, P(flux_stream_grads), P(flux_stream_grads), vp, vp, sz, vp],
        "flux_single_fwd_train": [P(flux_dims), P(flux_single_weights), vp, i64, vp, vp, vp, sz, vp],
        "flux_single_bwd": [P(flux_dims), P(flux_single_weights), vp, i64, vp, vp, vp, sz, P(flux_single_grads), vp,
                            vp, sz, vp],
        "flux_attention_fwd_train": [i32, i32, i32, vp, vp, vp, i64, vp, i64, vp, vp, sz, vp],
        "flux_attention_bwd": [i32, i32, i32, vp, vp, vp, i64, vp, vp, i64, vp, vp, vp, sz, vp],
        "flux_rf_loss_grad": [i32, i64, vp, vp, vp, vp, vp],
        "flux_attention_fp8_fwd": [i32, i32, i32, vp, vp, vp, i64, vp, i64, vp, vp, sz, vp],
        "flux_single_seq_fwd_train": [P(flux_dims), P(flux_stream_weights), vp, i64, vp, vp, vp, sz, vp],
        "flux_single_seq_bwd": [P(flux_dims), P(flux_stream_weights), vp, i64, vp, vp, vp, sz, P(flux_stream_grads),
                                vp, vp, sz, vp],
        "flux_final_bwd": [i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                           vp],
        "flux_embed_bwd": [i32, i32, i32, i32, i32, i32, i32, i32, i32, P(flux_embed_weights), vp, vp, vp, vp, vp,
                           vp, i64, vp, i64, vp, P(flux_embed_grads), vp, sz, vp],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = C.c_int
    L.flux_workspace_bytes.argtypes = [P(flux_dims), i32]
    L.flux_rf_noalloc_max_partials.argtypes = []
    L.flux_rf_noalloc_max_partials.restype = i64
    L.flux_fp8_state_bytes.argtypes = [i32]
    L.flux_fp8_state_bytes.restype = sz
    L.flux_workspace_bytes.restype = sz
    L.flux_rf_workspace_bytes.argtypes = [i32, i64]
    L.flux_rf_workspace_bytes.restype = sz
    L.flux_mx_scale_bytes.argtypes = [i32, i32]
    L.flux_mx_scale_bytes.restype = sz
    L.flux_mxfp4_scale_bytes.argtypes = [i32, i32]
    L.flux_mxfp4_scale_bytes.restype = sz
    L.flux_embed_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    L.flux_embed_workspace_bytes.restype = sz
    L.flux_final_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.flux_final_workspace_bytes.restype = sz
    L.flux_attention_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.flux_attention_workspace_bytes.restype = sz
    L.flux_train_saved_bytes.argtypes = [P(flux_dims), i32]
    L.flux_train_saved_bytes.restype = sz
    L.flux_bwd_workspace_bytes.argtypes = [P(flux_dims), i32]
    L.flux_bwd_workspace_bytes.restype = sz
    L.flux_attention_train_workspace_bytes.argtypes = [i32, i32, i32]
    L.flux_attention_train_workspace_bytes.restype = sz
    L.flux_final_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.flux_final_bwd_workspace_bytes.restype = sz
    L.flux_embed_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.flux_embed_bwd_workspace_bytes.restype = sz
    L.flux_attention_fp8_workspace_bytes.argtypes = [i32, i32, i32]
    L.flux_attention_fp8_workspace_bytes.restype = sz
    L.flux_status_string.argtypes = [C.c_int]
    L.flux_status_string.restype = C.c_char_p
    L.flux_last_error.argtypes = []
    L.flux_last_error.restype = C.c_char_p
    L.flux_timing_enable.argtypes = [i32]
    L.flux_timing_enable.restype = C.c_int
    L.flux_timing_classes.argtypes = []
    L.flux_timing_classes.restype = i32
    L.flux_timing_class_name.argtypes = [i32]
    L.flux_timing_class_name.restype = C.c_char_p
    L.flux_timing_read.argtypes = [P(C.c_double), P(C.c_int64), P(C.c_double), i32]
    L.flux_timing_read.restype = C.c_int
    _lib = L
    return L


def _check(status: int, where: str) -> None:
    if status != FLUX_OK:
        raise FluxError(status, where, lib().flux_last_error().decode())


def ptr(x) -> Optional[int]:
    """Device address of a tensor (or pass-through int / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# --------------------------------------------------------------------------- #
# marshalling helpers
# --------------------------------------------------------------------------- #
def make_dims(batch, l_img, l_txt, hidden, heads, head_dim, mlp_hidden, axes_dim=(16, 56, 56), theta=10000.0,
              eps=1e-6, precision=FLUX_PREC_BF16, weights_f16=0) -> flux_dims:
    d = flux_dims()
    d.batch, d.l_img, d.l_txt, d.hidden, d.heads, d.head_dim, d.mlp_hidden = (
        batch, l_img, l_txt, hidden, heads, head_dim, mlp_hidden)
    d.axes_dim[:] = list(axes_dim)
    d.theta, d.eps, d.precision, d.weights_f16 = theta, eps, precision, int(weights_f16)
    return d


def precision_code(name: str) -> int:
    return {"f32": FLUX_PREC_F32, "bf16": FLUX_PREC_BF16, "fp8": FLUX_PREC_FP8_E4M3}[name]


def dims_for(wl, batch: Optional[int] = None, weights_f16: bool = False) -> flux_dims:
    """flux_dims of a synth.Workload."""
    return make_dims(batch or wl.batch, wl.l_img, wl.l_txt, wl.hidden, wl.heads, wl.head_dim, wl.mlp_hidden,
                     wl.axes_dim, wl.theta, wl.eps, precision_code(wl.precision), weights_f16)


def stream_weights(w: Dict[str, object], prefix: Optional[str], fp8=None) -> flux_stream_weights:
    """Keys "<prefix>_mod.w" ...; prefix None: unprefixed keys ("mod.w", the
    sequential single block).  fp8: device address of the stream's 8
    flux_fp8_tensor records (fp8 dims only)."""
    s = flux_stream_weights()
    pre = f"{prefix}_" if prefix else ""
    for f in ("mod", "qkv", "proj", "fc1", "fc2"):
        setattr(s, f + "_w", ptr(w[f"{pre}{f}.w"]))
        setattr(s, f + "_b", ptr(w[f"{pre}{f}.b"]))
    s.q_norm = ptr(w[f"{pre}q_norm"])
    s.k_norm = ptr(w[f"{pre}k_norm"])
    s.fp8 = ptr(fp8)
    return s


def single_weights(w: Dict[str, object], fp8=None) -> flux_single_weights:
    """fp8: device address of the block's 4 flux_fp8_tensor records (fp8 dims only)."""
    s = flux_single_weights()
    for f in ("mod", "lin1", "lin2"):
        setattr(s, f + "_w", ptr(w[f + ".w"]))
        setattr(s, f + "_b", ptr(w[f + ".b"]))
    s.q_norm = ptr(w["q_norm"])
    s.k_norm = ptr(w["k_norm"])
    s.fp8 = ptr(fp8)
    return s


def stream_grads(g: Dict[str, object], prefix: Optional[str]) -> flux_stream_grads:
    """fp32 gradient buffers keyed like the weights ("<prefix>_qkv.w", ...)."""
    s = flux_stream_grads()
    pre = f"{prefix}_" if prefix else ""
    for f in ("mod", "qkv", "proj", "fc1", "fc2"):
        setattr(s, f + "_w", ptr(g[f"{pre}{f}.w"]))
        setattr(s, f + "_b", ptr(g[f"{pre}{f}.b"]))
    s.q_norm = ptr(g[f"{pre}q_norm"])
    s.k_norm = ptr(g[f"{pre}k_norm"])
    return s


def single_grads(g: Dict[str, object]) -> flux_single_grads:
    s = flux_single_grads()
    for f in ("mod", "lin1", "lin2"):
        setattr(s, f + "_w", ptr(g[f + ".w"]))
        setattr(s, f + "_b", ptr(g[f + ".b"]))
    s.q_norm = ptr(g["q_norm"])
    s.k_norm = ptr(g["k_norm"])
    return s


def embed_grads(g: Dict[str, object]) -> flux_embed_grads:
    s = flux_embed_grads()
    for f in ("img_in", "txt_in", "time_in1", "time_in2", "vector_in1", "vector_in2", "guidance_in"):
        setattr(s, f + "_w", ptr(g.get(f + ".w")))
        setattr(s, f + "_b", ptr(g.get(f + ".b")))
    return s


def embed_weights(w: Dict[str, object]) -> flux_embed_weights:
    s = flux_embed_weights()
    for f in ("img_in", "txt_in", "time_in1", "time_in2", "vector_in1", "vector_in2", "guidance_in"):
        setattr(s, f + "_w", ptr(w.get(f + ".w")))
        setattr(s, f + "_b", ptr(w.get(f + ".b")))
    return s


# --------------------------------------------------------------------------- #
# entry points (names of include/flux.h)
# --------------------------------------------------------------------------- #
def flux_workspace_bytes(dims: flux_dims, op: int) -> int:
    return lib().flux_workspace_bytes(C.byref(dims), op)


def flux_block_fwd(dims: flux_dims, img_w: flux_stream_weights, txt_w: flux_stream_weights, img, img_bstride: int,
                   txt, txt_bstride: int, vec, rope, workspace, workspace_bytes: int, stream=None) -> None:
    _check(lib().flux_block_fwd(C.byref(dims), C.byref(img_w), C.byref(txt_w), ptr(img), img_bstride, ptr(txt),
                                txt_bstride, ptr(vec), ptr(rope), ptr(workspace), workspace_bytes,
                                _stream(stream)), "flux_block_fwd")


def flux_single_fwd(dims: flux_dims, w: flux_single_weights, x, x_bstride: int, vec, rope, workspace,
                    workspace_bytes: int, stream=None) -> None:
    _check(lib().flux_single_fwd(C.byref(dims), C.byref(w), ptr(x), x_bstride, ptr(vec), ptr(rope), ptr(workspace),
                                 workspace_bytes, _stream(stream)), "flux_single_fwd")


def flux_single_seq_fwd(dims: flux_dims, w: flux_stream_weights, x, x_bstride: int, vec, rope, workspace,
                        workspace_bytes: int, stream=None) -> None:
    _check(lib().flux_single_seq_fwd(C.byref(dims), C.byref(w), ptr(x), x_bstride, ptr(vec), ptr(rope),
                                     ptr(workspace), workspace_bytes, _stream(stream)), "flux_single_seq_fwd")


def flux_rf_workspace_bytes(batch: int, n_per_sample: int) -> int:
    return lib().flux_rf_workspace_bytes(batch, n_per_sample)


def rf_noise_loss(batch: int, n_per_sample: int, z0, z1, t, z_t=None, v_target=None, v_pred=None, loss=None,
                  loss_per_sample=None, workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    a = rf_args()
    a.batch, a.n_per_sample = batch, n_per_sample
    a.z0, a.z1, a.t, a.z_t, a.v_target, a.v_pred = map(ptr, (z0, z1, t, z_t, v_target, v_pred))
    a.loss, a.loss_per_sample, a.workspace = map(ptr, (loss, loss_per_sample, workspace))
    a.workspace_bytes = workspace_bytes
    _check(lib().rf_noise_loss(C.byref(a), _stream(stream)), "rf_noise_loss")


def rf_noise_loss_noalloc(batch: int, n_per_sample: int, z0, z1, t, z_t=None, v_target=None, v_pred=None,
                          loss=None, loss_per_sample=None, stream=None) -> None:
    a = rf_args()
    a.batch, a.n_per_sample = batch, n_per_sample
    a.z0, a.z1, a.t, a.z_t, a.v_target, a.v_pred = map(ptr, (z0, z1, t, z_t, v_target, v_pred))
    a.loss, a.loss_per_sample = map(ptr, (loss, loss_per_sample))
    _check(lib().rf_noise_loss_noalloc(C.byref(a), _stream(stream)), "rf_noise_loss_noalloc")


def flux_rf_noalloc_max_partials() -> int:
    return lib().flux_rf_noalloc_max_partials()


def flux_rope_table(ids, batch: int, seq: int, axes_dim, theta: float, table, stream=None) -> None:
    ax = (C.c_int32 * 3)(*axes_dim)
    _check(lib().flux_rope_table(ptr(ids), batch, seq, ax, theta, ptr(table), _stream(stream)), "flux_rope_table")


def flux_embed_workspace_bytes(precision, batch, channels, height, width, hidden) -> int:
    return lib().flux_embed_workspace_bytes(precision, batch, channels, height, width, hidden)


def flux_embed_fwd(precision, batch, channels, height, width, l_txt, ctx_dim, hidden, time_dim, y_dim,
                   w: flux_embed_weights, z_t, txt, t, y, x_img, img_bstride, x_txt, txt_bstride, vec, workspace,
                   workspace_bytes, stream=None, guidance=None) -> None:
    _check(lib().flux_embed_fwd(precision, batch, channels, height, width, l_txt, ctx_dim, hidden, time_dim, y_dim,
                                C.byref(w), ptr(z_t), ptr(txt), ptr(t), ptr(y), ptr(guidance), ptr(x_img),
                                img_bstride, ptr(x_txt), txt_bstride, ptr(vec), ptr(workspace), workspace_bytes,
                                _stream(stream)),
           "flux_embed_fwd")


def flux_mx_scale_bytes(rows: int, k: int) -> int:
    return lib().flux_mx_scale_bytes(rows, k)


def flux_mx_quantize(src_precision: int, src, rows: int, k: int, codes, scales, stream=None) -> None:
    _check(lib().flux_mx_quantize(src_precision, ptr(src), rows, k, ptr(codes), ptr(scales), _stream(stream)),
           "flux_mx_quantize")


def flux_mxfp8_linear_fwd(m: int, n: int, k: int, x, x_scales, w, w_scales, b, y, ldy: int, stream=None) -> None:
    _check(lib().flux_mxfp8_linear_fwd(m, n, k, ptr(x), ptr(x_scales), ptr(w), ptr(w_scales), ptr(b), ptr(y), ldy,
                                       _stream(stream)), "flux_mxfp8_linear_fwd")


def mx_scales_unswizzle(sc, rows: int, k: int):
    """[rows, k/32] scale bytes from the GEMM layout of flux_mx_quantize
    (numpy uint8 array in, numpy out; pad rows dropped)."""
    import numpy as np
    s = np.asarray(sc, dtype=np.uint8)
    rp = ((rows + 255) // 256) * 256
    # byte (((row/128)*(k/64) + kb/2)*2 + kb%2)*128 + (row%32)*4 + (row/32)%4
    t = s[: rp * (k // 32)].reshape(rp // 128, k // 64, 2, 32, 4)      # [rb, kt, h, l32, i]
    t = t.transpose(0, 4, 3, 1, 2).reshape(rp, k // 32)                 # rows rb*128 + i*32 + l32
    return t[:rows]


def flux_timestep_embed(t, batch: int, dim: int, time_factor: float, out, stream=None) -> None:
    _check(lib().flux_timestep_embed(ptr(t), batch, dim, time_factor, ptr(out), _stream(stream)),
           "flux_timestep_embed")


def flux_fp8_block_quantize(src_precision: int, src, rows: int, k: int, tile_rows: int, codes, scales,
                            stream=None) -> None:
    _check(lib().flux_fp8_block_quantize(src_precision, ptr(src), rows, k, tile_rows, ptr(codes), ptr(scales),
                                         _stream(stream)), "flux_fp8_block_quantize")


def flux_mxfp4_scale_bytes(rows: int, k: int) -> int:
    return lib().flux_mxfp4_scale_bytes(rows, k)


def flux_mxfp4_quantize(src_precision: int, src, rows: int, k: int, codes, scales, stream=None) -> None:
    _check(lib().flux_mxfp4_quantize(src_precision, ptr(src), rows, k, ptr(codes), ptr(scales), _stream(stream)),
           "flux_mxfp4_quantize")


def flux_mxfp4_linear_fwd(m: int, n: int, k: int, x, x_scales, w, w_scales, b, y, ldy: int, stream=None) -> None:
    _check(lib().flux_mxfp4_linear_fwd(m, n, k, ptr(x), ptr(x_scales), ptr(w), ptr(w_scales), ptr(b), ptr(y), ldy,
                                       _stream(stream)), "flux_mxfp4_linear_fwd")


def mxfp4_scales_unswizzle(sc, rows: int, k: int):
    """[rows, k/32] scale bytes from the GEMM layout of flux_mxfp4_quantize
    (numpy uint8 array in, numpy out; pad rows dropped)."""
    import numpy as np
    s = np.asarray(sc, dtype=np.uint8)
    rp = ((rows + 255) // 256) * 256
    # byte ((row/128)*(k/128) + kb/4)*512 + (kb%2)*256 + (row%32)*8 + ((kb%4)/2)*4 + (row/32)%4
    t = s[: rp * (k // 32)].reshape(rp // 128, k // 128, 2, 32, 2, 4)   # [rb, kt, kb%2, l32, (kb%4)/2, i]
    t = t.transpose(0, 5, 3, 1, 4, 2).reshape(rp, k // 32)              # rows rb*128 + i*32 + l32; kb = 4kt+2m+h
    return t[:rows]


def flux_euler_step(batch: int, n_per_sample: int, v, z, t_cur: float, t_next: float, cfg: bool = False,
                    guidance: float = 1.0, z_model=None, copies: int = 1, t_model=None, t_model_n: int = 0,
                    stream=None) -> None:
    a = flux_euler_args()
    a.batch, a.n_per_sample, a.v, a.cfg, a.guidance = batch, n_per_sample, ptr(v), int(bool(cfg)), guidance
    a.t_cur, a.t_next, a.z, a.z_model, a.copies = t_cur, t_next, ptr(z), ptr(z_model), copies
    a.t_model, a.t_model_n = ptr(t_model), t_model_n
    _check(lib().flux_euler_step(C.byref(a), _stream(stream)), "flux_euler_step")


def flux_final_workspace_bytes(precision, batch, height, width, hidden) -> int:
    return lib().flux_final_workspace_bytes(precision, batch, height, width, hidden)


def flux_final_fwd(precision, batch, channels, height, width, hidden, eps, mod_w, mod_b, out_w, out_b, x_img,
                   bstride, vec, v_pred, workspace, workspace_bytes, stream=None) -> None:
    _check(lib().flux_final_fwd(precision, batch, channels, height, width, hidden, eps, ptr(mod_w), ptr(mod_b),
                                ptr(out_w), ptr(out_b), ptr(x_img), bstride, ptr(vec), ptr(v_pred), ptr(workspace),
                                workspace_bytes, _stream(stream)), "flux_final_fwd")


def flux_linear_fwd(precision, m, n, k, x, lda, w, b, y, ldy, stream=None) -> None:
    _check(lib().flux_linear_fwd(precision, m, n, k, ptr(x), lda, ptr(w), ptr(b), ptr(y), ldy, _stream(stream)),
           "flux_linear_fwd")


def flux_attention_workspace_bytes(precision, batch, seq, heads, head_dim) -> int:
    return lib().flux_attention_workspace_bytes(precision, batch, seq, heads, head_dim)


def flux_attention_fwd(precision, batch, seq, heads, head_dim, q, k, v, ld_in, o, ld_out, workspace,
                       workspace_bytes, stream=None) -> None:
    _check(lib().flux_attention_fwd(precision, batch, seq, heads, head_dim, ptr(q), ptr(k), ptr(v), ld_in, ptr(o),
                                    ld_out, ptr(workspace), workspace_bytes, _stream(stream)), "flux_attention_fwd")


def flux_timing_enable(on: bool) -> None:
    _check(lib().flux_timing_enable(1 if on else 0), "flux_timing_enable")


def flux_timing_flush(buffer=None, nbytes: int = 0) -> None:
    """Overwrite `buffer` (device, nbytes) before every timed launch, so timed
    kernels start with cold caches; None turns it off."""
    _check(lib().flux_timing_flush(ptr(buffer), nbytes if buffer is not None else 0), "flux_timing_flush")


def flux_stream_copy(src, dst, nbytes: int, stream=None) -> None:
    _check(lib().flux_stream_copy(ptr(src), ptr(dst), nbytes, _stream(stream)), "flux_stream_copy")


def flux_gemm_stream_k(on: Optional[bool] = None, spin: int = 0) -> bool:
    """Stream-K tail of the block linears on / off (None: leave) and the owner's
    poll limit (0: default); returns the previous setting."""
    return bool(lib().flux_gemm_stream_k(-1 if on is None else (1 if on else 0), spin))


# device checks (status word bits)
FLUX_DBG_T_RANGE = 1
FLUX_DBG_NONFINITE_RESIDUAL = 2
FLUX_DBG_NONFINITE_LOSS = 4
FLUX_DBG_NONFINITE_OUTPUT = 8
FLUX_DBG_NONFINITE_GRAD = 16


def flux_debug_checks(on: Optional[bool] = None) -> bool:
    """Turn the device checks on / off (None: leave); returns the previous setting."""
    return bool(lib().flux_debug_checks(-1 if on is None else (1 if on else 0)))


def flux_debug_status(clear: bool = False) -> int:
    """The current device's status word (synchronizes the device)."""
    v = C.c_uint32(0)
    _check(lib().flux_debug_status(C.byref(v), 1 if clear else 0), "flux_debug_status")
    return int(v.value)


def flux_timing_read() -> Dict[str, tuple]:
    """{class name: (total ms, launches, algorithmic work)} of the launches
    since the last read (work in FLOPs for GEMM / attention, bytes otherwise)."""
    L = lib()
    n = L.flux_timing_classes()
    ms = (C.c_double * n)()
    cnt = (C.c_int64 * n)()
    work = (C.c_double * n)()
    _check(L.flux_timing_read(ms, cnt, work, n), "flux_timing_read")
    return {L.flux_timing_class_name(i).decode(): (ms[i], cnt[i], work[i]) for i in range(n)}


def flux_convert_bf16_to_f16(src, dst, n: int, stream=None) -> None:
    _check(lib().flux_convert_bf16_to_f16(ptr(src), ptr(dst), n, _stream(stream)), "flux_convert_bf16_to_f16")


# --------------------------------------------------------------------------- #
# fp8 (E4M3) delayed scaling
# --------------------------------------------------------------------------- #
def flux_fp8_state_bytes(n_tensors: int) -> int:
    return lib().flux_fp8_state_bytes(n_tensors)


def flux_fp8_quantize(src_precision: int, src, n: int, rec, dst, stream=None) -> None:
    _check(lib().flux_fp8_quantize(src_precision, ptr(src), n, ptr(rec), ptr(dst), _stream(stream)),
           "flux_fp8_quantize")


def flux_fp8_quantize_current(src_precision: int, src, n: int, rec, dst, stream=None) -> None:
    _check(lib().flux_fp8_quantize_current(src_precision, ptr(src), n, ptr(rec), ptr(dst), _stream(stream)),
           "flux_fp8_quantize_current")


def flux_fp8_update(recs, n_tensors: int, algo: int = 0, margin: int = 0, stream=None) -> None:
    _check(lib().flux_fp8_update(ptr(recs), n_tensors, algo, margin, _stream(stream)), "flux_fp8_update")


def flux_fp8_linear_fwd(m, n, k, x, ldx, w, ldw, rx, rw, b, y, ldy, stream=None) -> None:
    _check(lib().flux_fp8_linear_fwd(m, n, k, ptr(x), ldx, ptr(w), ldw, ptr(rx), ptr(rw), ptr(b), ptr(y), ldy,
                                     _stream(stream)), "flux_fp8_linear_fwd")


def fp8_record_fields(raw: bytes) -> dict:
    """Decode one flux_fp8_tensor record copied to the host (for tests and
    diagnostics): scale, scale_inv, amax, flags, hist_len, hist_pos, history."""
    import struct
    scale, scale_inv, amax_bits, flags, hist_len, hist_pos = struct.unpack_from("<ffIIII", raw, 0)
    hist = struct.unpack_from(f"<{FLUX_FP8_HISTORY}f", raw, 32)
    return {"scale": scale, "scale_inv": scale_inv, "amax": struct.unpack("<f", struct.pack("<I", amax_bits))[0],
            "flags": flags, "hist_len": hist_len, "hist_pos": hist_pos, "history": hist}


# --------------------------------------------------------------------------- #
# training (backward)
# --------------------------------------------------------------------------- #
def flux_train_saved_bytes(dims: flux_dims, op: int) -> int:
    return lib().flux_train_saved_bytes(C.byref(dims), op)


def flux_bwd_workspace_bytes(dims: flux_dims, op: int) -> int:
    return lib().flux_bwd_workspace_bytes(C.byref(dims), op)


def flux_block_fwd_train(dims: flux_dims, img_w: flux_stream_weights, txt_w: flux_stream_weights, img,
                         img_bstride: int, txt, txt_bstride: int, vec, rope, saved, saved_bytes: int,
                         stream=None) -> None:
    _check(lib().flux_block_fwd_train(C.byref(dims), C.byref(img_w), C.byref(txt_w), ptr(img), img_bstride, ptr(txt),
                                      txt_bstride, ptr(vec), ptr(rope), ptr(saved), saved_bytes, _stream(stream)),
           "flux_block_fwd_train")


def flux_block_bwd(dims: flux_dims, img_w: flux_stream_weights, txt_w: flux_stream_weights, d_img, img_bstride: int,
                   d_txt, txt_bstride: int, vec, rope, saved, saved_bytes: int, img_grads: flux_stream_grads,
                   txt_grads: flux_stream_grads, dvec, workspace, workspace_bytes: int, stream=None) -> None:
    _check(lib().flux_block_bwd(C.byref(dims), C.byref(img_w), C.byref(txt_w), ptr(d_img), img_bstride, ptr(d_txt),
                                txt_bstride, ptr(vec), ptr(rope), ptr(saved), saved_bytes, C.byref(img_grads),
                                C.byref(txt_grads), ptr(dvec), ptr(workspace), workspace_bytes, _stream(stream)),
           "flux_block_bwd")


def flux_single_fwd_train(dims: flux_dims, w: flux_single_weights, x, x_bstride: int, vec, rope, saved,
                          saved_bytes: int, stream=None) -> None:
    _check(lib().flux_single_fwd_train(C.byref(dims), C.byref(w), ptr(x), x_bstride, ptr(vec), ptr(rope), ptr(saved),
                                       saved_bytes, _stream(stream)), "flux_single_fwd_train")


def flux_single_bwd(dims: flux_dims, w: flux_single_weights, dx, x_bstride: int, vec, rope, saved, saved_bytes: int,
                    grads: flux_single_grads, dvec, workspace, workspace_bytes: int, stream=None) -> None:
    _check(lib().flux_single_bwd(C.byref(dims), C.byref(w), ptr(dx), x_bstride, ptr(vec), ptr(rope), ptr(saved),
                                 saved_bytes, C.byref(grads), ptr(dvec), ptr(workspace), workspace_bytes,
                                 _stream(stream)), "flux_single_bwd")


def flux_attention_train_workspace_bytes(batch: int, seq: int, heads: int) -> int:
    return lib().flux_attention_train_workspace_bytes(batch, seq, heads)


def flux_attention_fwd_train(batch: int, seq: int, heads: int, q, k, v, ld: int, o, ldo: int, lse, workspace,
                             workspace_bytes: int, stream=None) -> None:
    _check(lib().flux_attention_fwd_train(batch, seq, heads, ptr(q), ptr(k), ptr(v), ld, ptr(o), ldo, ptr(lse),
                                          ptr(workspace), workspace_bytes, _stream(stream)), "flux_attention_fwd_train")


def flux_attention_bwd(batch: int, seq: int, heads: int, q, k, v, ld: int, o, dout, ldo: int, lse, dqkv, workspace,
                       workspace_bytes: int, stream=None) -> None:
    _check(lib().flux_attention_bwd(batch, seq, heads, ptr(q), ptr(k), ptr(v), ld, ptr(o), ptr(dout), ldo, ptr(lse),
                                    ptr(dqkv), ptr(workspace), workspace_bytes, _stream(stream)), "flux_attention_bwd")


def flux_rf_loss_grad(batch: int, n_per_sample: int, v_pred, z0, z1, dv, stream=None) -> None:
    _check(lib().flux_rf_loss_grad(batch, n_per_sample, ptr(v_pred), ptr(z0), ptr(z1), ptr(dv), _stream(stream)),
           "flux_rf_loss_grad")


def flux_final_bwd_workspace_bytes(batch, channels, height, width, hidden) -> int:
    return lib().flux_final_bwd_workspace_bytes(batch, channels, height, width, hidden)


def flux_final_bwd(batch, channels, height, width, hidden, eps, mod_w, mod_b, out_w, x_img, bstride, vec, dv, dx_img,
                   dvec, g_mod_w, g_mod_b, g_out_w, g_out_b, workspace, workspace_bytes, stream=None) -> None:
    _check(lib().flux_final_bwd(batch, channels, height, width, hidden, eps, ptr(mod_w), ptr(mod_b), ptr(out_w),
                                ptr(x_img), bstride, ptr(vec), ptr(dv), ptr(dx_img), ptr(dvec), ptr(g_mod_w),
                                ptr(g_mod_b), ptr(g_out_w), ptr(g_out_b), ptr(workspace), workspace_bytes,
                                _stream(stream)), "flux_final_bwd")


def flux_embed_bwd_workspace_bytes(batch, channels, height, width, l_txt, ctx_dim, hidden) -> int:
    return lib().flux_embed_bwd_workspace_bytes(batch, channels, height, width, l_txt, ctx_dim, hidden)


def flux_embed_bwd(batch, channels, height, width, l_txt, ctx_dim, hidden, time_dim, y_dim, w: flux_embed_weights,
                   z_t, txt, t, y, d_img, img_bstride, d_txt, txt_bstride, dvec, grads: flux_embed_grads, workspace,
                   workspace_bytes, stream=None, guidance=None) -> None:
    _check(lib().flux_embed_bwd(batch, channels, height, width, l_txt, ctx_dim, hidden, time_dim, y_dim, C.byref(w),
                                ptr(z_t), ptr(txt), ptr(t), ptr(y), ptr(guidance), ptr(d_img), img_bstride, ptr(d_txt),
                                txt_bstride,
                                ptr(dvec), C.byref(grads), ptr(workspace), workspace_bytes, _stream(stream)),
           "flux_embed_bwd")


def flux_single_seq_fwd_train(dims: flux_dims, w: flux_stream_weights, x, x_bstride: int, vec, rope, saved,
                              saved_bytes: int, stream=None) -> None:
    _check(lib().flux_single_seq_fwd_train(C.byref(dims), C.byref(w), ptr(x), x_bstride, ptr(vec), ptr(rope),
                                           ptr(saved), saved_bytes, _stream(stream)), "flux_single_seq_fwd_train")


def flux_single_seq_bwd(dims: flux_dims, w: flux_stream_weights, dx, x_bstride: int, vec, rope, saved,
                        saved_bytes: int, grads: flux_stream_grads, dvec, workspace, workspace_bytes: int,
                        stream=None) -> None:
    _check(lib().flux_single_seq_bwd(C.byref(dims), C.byref(w), ptr(dx), x_bstride, ptr(vec), ptr(rope), ptr(saved),
                                     saved_bytes, C.byref(grads), ptr(dvec), ptr(workspace), workspace_bytes,
                                     _stream(stream)), "flux_single_seq_bwd")


def flux_attention_fp8_workspace_bytes(batch: int, seq: int, heads: int) -> int:
    return lib().flux_attention_fp8_workspace_bytes(batch, seq, heads)


def flux_attention_fp8_fwd(batch: int, seq: int, heads: int, q, k, v, ld_in: int, o, ld_out: int, recs, workspace,
                           workspace_bytes: int, stream=None) -> None:
    _check(lib().flux_attention_fp8_fwd(batch, seq, heads, ptr(q), ptr(k), ptr(v), ld_in, ptr(o), ld_out, ptr(recs),
                                        ptr(workspace), workspace_bytes, _stream(stream)), "flux_attention_fp8_fwd")
