"""fp64 reference of the MXFP8 (E4M3) linear: block-scaled FP8.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"FP8 training for Flux models" (Configuration / FP8 model configuration)
names "mxfp8" as an alternative to the delayed per-tensor recipe without
defining it.  The name refers to the OCP Microscaling (MX) format, v1.0: a
block of 32 consecutive values shares one power-of-two scale stored as an
E8M0 byte, and each value is stored as an FP8 element.  Readings taken here
(each repeated at its function):
  M1 blocks run along the reduction axis K of a linear (the last axis of the
     activation X [M, K] and of the weight W [N, K]), 32 values each; K is a
     multiple of 32.
  M2 the block's shared exponent is X = floor(log2(max |v|)) - 8, 8 being the
     exponent of E4M3's largest power of two (448 = 1.75 * 2^8), clamped to
     E8M0's range [-127, 127]; an all-zero block takes X = -127.  The scale
     byte is X + 127.  A block holding a non-finite value has the NaN scale
     byte 0xFF and its elements are encoded unscaled.
  M3 each element is e4m3_encode(v / 2^X): the division by a power of two is
     exact, then round to nearest even on the E4M3FN grid with saturation to
     +-448 (scaled magnitudes lie below 512, so values above 448 clip).
  M4 the linear is y = sum over K blocks of 2^(X_x + X_w) * sum over the block
     of dec(q_x) dec(q_w), plus the bias in high precision.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .flux_oracle import f64
from .fp8_oracle import e4m3_decode, e4m3_encode

__all__ = ["MX_BLOCK", "E4M3_EMAX", "mx_exponents", "mx_quantize", "mx_dequantize", "mx_linear"]

MX_BLOCK = 32
E4M3_EMAX = 8          # 448 = 1.75 * 2^8


def mx_exponents(x) -> np.ndarray:
    """Shared exponent X of every 32-value block along the last axis (M2), as
    int64; blocks holding a non-finite value get the marker 128."""
    x = f64(x)
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // MX_BLOCK, MX_BLOCK))
    a = np.abs(blocks).max(axis=-1)
    finite = np.isfinite(blocks).all(axis=-1)
    safe = np.where((a > 0) & finite, a, 1.0)
    # floor(log2(a)) exactly: frexp gives a = m 2^e with m in [0.5, 1)
    _, e = np.frexp(safe)
    X = (e.astype(np.int64) - 1) - E4M3_EMAX
    X = np.where(a > 0, X, -127)
    X = np.clip(X, -127, 127)
    return np.where(finite, X, 128)


def mx_quantize(x) -> Tuple[np.ndarray, np.ndarray]:
    """(codes [.., K] uint8, scale bytes [.., K/32] uint8) of x along its last
    axis (M1-M3)."""
    x = f64(x)
    assert x.shape[-1] % MX_BLOCK == 0, "K must be a multiple of 32"
    X = mx_exponents(x)
    nonfinite = X == 128
    Xe = np.where(nonfinite, 0, X)
    scale = np.repeat(np.exp2(Xe.astype(np.float64)), MX_BLOCK, axis=-1)
    codes = e4m3_encode(x / scale)
    sbytes = np.where(nonfinite, 0xFF, X + 127).astype(np.uint8)
    return codes, sbytes


def mx_dequantize(codes, sbytes) -> np.ndarray:
    """Values of MX codes: dec(code) * 2^(scale byte - 127); NaN under a NaN scale."""
    s = np.asarray(sbytes, dtype=np.int64)
    val = np.where(s == 0xFF, np.nan, np.exp2(s.astype(np.float64) - 127.0))
    return e4m3_decode(codes) * np.repeat(val, MX_BLOCK, axis=-1)


def mx_linear(x, w, b=None) -> np.ndarray:
    """x [M, K] and w [N, K] quantized to MXFP8 along K, y = deq(x) deq(w)^T
    (+ b) in fp64: every product of two E4M3 values times two powers of two is
    exact, so this is the block sum of M4 up to fp64 rounding."""
    xq, xs = mx_quantize(x)
    wq, ws = mx_quantize(w)
    y = mx_dequantize(xq, xs) @ mx_dequantize(wq, ws).T
    return y + f64(b) if b is not None else y
