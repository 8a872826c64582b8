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
  M5 MXFP4: the same blocks and E8M0 scales with E2M1 elements (2 exponent
     bits with bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
     negatives); X = floor(log2(max |v|)) - 2, 2 being the exponent of 6 =
     1.5 * 2^2; elements round to nearest even on the E2M1 grid and saturate
     to +-6.  Two codes share a byte, the even-indexed element in the low
     nibble.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .flux_oracle import f64
from .fp8_oracle import e4m3_decode, e4m3_encode

__all__ = ["MX_BLOCK", "E4M3_EMAX", "mx_exponents", "mx_quantize", "mx_dequantize", "mx_linear",
           "E2M1_EMAX", "e2m1_encode", "e2m1_decode", "mxfp4_quantize", "mxfp4_dequantize", "mxfp4_linear"]

MX_BLOCK = 32
E4M3_EMAX = 8          # 448 = 1.75 * 2^8


def mx_exponents(x, emax: int = E4M3_EMAX) -> np.ndarray:
    """Shared exponent X of every 32-value block along the last axis (M2; M5
    with emax = 2), as int64; blocks holding a non-finite value get the marker
    128."""
    x = f64(x)
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // MX_BLOCK, MX_BLOCK))
    a = np.abs(blocks).max(axis=-1)
    finite = np.isfinite(blocks).all(axis=-1)
    safe = np.where((a > 0) & finite, a, 1.0)
    # floor(log2(a)) exactly: frexp gives a = m 2^e with m in [0.5, 1)
    _, e = np.frexp(safe)
    X = (e.astype(np.int64) - 1) - emax
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


# ------------------------------------ MXFP4 (M5) ------------------------------------
E2M1_EMAX = 2                     # 6 = 1.5 * 2^2
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    """Value of 4-bit E2M1 codes (bit 3 the sign, then 2 exponent bits with
    bias 1 and 1 mantissa bit; exponent 0 is subnormal: 0 or 0.5)."""
    c = np.asarray(codes, dtype=np.int64) & 15
    mag = _E2M1[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_encode(x) -> np.ndarray:
    """Nearest E2M1 code of x, ties to the even code (mantissa bit 0),
    magnitudes above 6 saturate to 6; the sign of zero is kept."""
    x = f64(x)
    a = np.abs(x)
    # candidates below and above on the grid, then nearest with ties to even
    idx_hi = np.searchsorted(_E2M1, np.minimum(a, 6.0), side="left")
    idx_hi = np.clip(idx_hi, 0, 7)
    idx_lo = np.clip(idx_hi - 1, 0, 7)
    lo, hi = _E2M1[idx_lo], _E2M1[idx_hi]
    d_lo, d_hi = a - lo, hi - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((idx_hi & 1) == 0))
    code = np.where(a >= 6.0, 7, np.where(pick_hi, idx_hi, idx_lo))
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.int64)


def mxfp4_quantize(x) -> Tuple[np.ndarray, np.ndarray]:
    """(packed codes [.., K/2] uint8, scale bytes [.., K/32] uint8) of x along
    its last axis (M5); every block is finite."""
    x = f64(x)
    assert x.shape[-1] % MX_BLOCK == 0, "K must be a multiple of 32"
    X = mx_exponents(x, E2M1_EMAX)
    assert not (X == 128).any(), "MXFP4 blocks must be finite"
    scale = np.repeat(np.exp2(X.astype(np.float64)), MX_BLOCK, axis=-1)
    c = e2m1_encode(x / scale)
    packed = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    return packed, (X + 127).astype(np.uint8)


def mxfp4_dequantize(packed, sbytes) -> np.ndarray:
    p = np.asarray(packed, dtype=np.int64)
    c = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    c[..., 0::2] = p & 15
    c[..., 1::2] = p >> 4
    s = np.asarray(sbytes, dtype=np.int64)
    return e2m1_decode(c) * np.repeat(np.exp2(s.astype(np.float64) - 127.0), MX_BLOCK, axis=-1)


def mxfp4_linear(x, w, b=None) -> np.ndarray:
    """x [M, K] and w [N, K] quantized to MXFP4 along K, y = deq(x) deq(w)^T
    (+ b) in fp64 (every product is exact)."""
    y = mxfp4_dequantize(*mxfp4_quantize(x)) @ mxfp4_dequantize(*mxfp4_quantize(w)).T
    return y + f64(b) if b is not None else y
