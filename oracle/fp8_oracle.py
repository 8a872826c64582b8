"""fp64 reference of the FP8 (E4M3) linears with delayed scaling.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Follows "FP8 training
for Flux models", Configuration / FP8 model configuration: forward tensors in
the E4M3 format, the "delayed" scaling recipe with margin 0, an amax history
of 1024 entries and the "most_recent" (or "max") amax selection; attention
stays in higher precision.

Readings taken where that page is silent (each repeated at its function):
  F1 E4M3 is the OCP E4M3FN encoding: 1 sign, 4 exponent (bias 7), 3 mantissa
     bits; exponent field 0 holds subnormals m * 2^-9; the all-ones pattern
     S.1111.111 is NaN; no infinities; largest finite value 448.
  F2 a value is scaled in fp32 and rounded to the nearest E4M3 value, ties to
     the even code; magnitudes above 448 (infinities included) saturate to
     +-448; NaN stays NaN.
  F3 a quantized linear computes y = (sum_k q(x)_k q(w)_k) / (s_x s_w) + b: both
     operands are quantized with their own per-tensor scale, products are
     accumulated exactly here (fp32 on the GPU), the result is divided by both
     scales, the bias is added in high precision.
  F4 scale update after a forward, per tensor: the amax of the tensor as it was
     quantized in that forward enters the history; the selected amax is that
     entry (most_recent) or the history maximum (max); the new scale is
     fp32(448 / amax) * 2^-margin when that amax is finite and positive,
     otherwise the scale is left as it was.  Before any update the scale is 1.
  F5 fp8 covers the token-path linears of the blocks (qkv, proj, fc1, fc2 of
     each double-block stream; lin1 and lin2 of the single block); the
     modulation linears, the embeddings, the output head and attention keep
     their bf16 operands.
  F6 the "tensorwise" alternative recipe the page lists scales each tensor
     with its own current amax: s = fp32(448 / amax) of the tensor being
     quantized, no history.
  F7 fp8 attention (listed on the page, off by default, without a recipe):
     Q, K and V are each quantized with their own current scale (F6); the
     scores and the output are formed from the dequantized values
     dec(code) * fp32(1 / s).  The GPU also packs the probabilities to E4M3
     (relative error <= 2^-4 each); the oracle keeps them exact and the test
     bounds that step.
  F8 the "blockwise" alternative recipe the page lists: E4M3 elements with
     one scale per tile along K, tiles of 1 x 128 values for activations (one
     row) and 128 x 128 for weights (128 rows, the last tile of a ragged row
     count holding the rows that exist); a tile's scale 2^e is the largest
     power of two with amax * 2^e <= 448, e clamped to [-127, 127] (e = 0 for
     an all-zero tile); elements are e4m3(v * 2^e), an exact product; the
     linear is y = sum over 128-wide k blocks of 2^-(e_x + e_w) sum q_x q_w
     + b.  A tile holding a non-finite value is not defined here.
  F9 a new scale (delayed update or current scaling) is taken only when it
     and its reciprocal are finite and non-zero in fp32; a selected amax
     below about 448 / FLT_MAX, whose 448 / amax overflows, keeps the previous
     scale exactly as a zero or non-finite amax does (the page's recipe
     assumes a usable scale; an infinite one would turn zeros into NaN).
"""
from __future__ import annotations

from typing import Callable, Dict, Optional, Tuple

import numpy as np

from .flux_oracle import attention, f64, linear

__all__ = ["E4M3_MAX", "HISTORY_LEN", "e4m3_decode", "e4m3_encode", "quantize", "amax", "fp8_linear",
           "attention_fp8", "BLOCK_K", "block_exponents", "block_quantize", "block_dequantize", "block_linear",
           "scale_update", "current_scale", "fp8_linears", "TOKEN_LINEARS_DOUBLE", "TOKEN_LINEARS_SINGLE"]

E4M3_MAX = 448.0
HISTORY_LEN = 1024
TOKEN_LINEARS_DOUBLE = ("qkv", "proj", "fc1", "fc2")   # per stream (F5)
TOKEN_LINEARS_SINGLE = ("lin1", "lin2")


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3FN byte (F1), as float64; NaN for 0x7F and 0xFF."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


# the 127 non-negative finite values, codes 0x00..0x7E, in increasing order
_GRID = e4m3_decode(np.arange(0x7F))


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3FN code of each value, ties to the even code (F2).

    Saturates magnitudes above 448 (and infinities) to +-448 and keeps NaN.
    Works on exact values: a tie is decided by comparing the value with the
    exact midpoint of the two neighbouring grid points."""
    x = f64(x)
    a = np.abs(x)
    neg = np.signbit(x)
    fin = np.isfinite(a)
    a_in = np.where(fin, np.minimum(a, E4M3_MAX), 0.0)
    hi = np.searchsorted(_GRID, a_in, side="left")          # first grid point >= a
    hi = np.minimum(hi, len(_GRID) - 1)
    lo = np.maximum(hi - 1, 0)
    exact = _GRID[hi] == a_in
    mid = 0.5 * (_GRID[lo] + _GRID[hi])                      # exact: few significant bits
    pick_hi = (a_in > mid) | ((a_in == mid) & (hi % 2 == 0))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo)).astype(np.int64)
    code = np.where(np.isinf(a) | (a > E4M3_MAX), 0x7E, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize(v, scale) -> np.ndarray:
    """E4M3 codes of v under a per-tensor scale: the product fp32(v) * fp32(s)
    is formed in fp32, then rounded onto the E4M3 grid (F2)."""
    prod = np.asarray(v, dtype=np.float32) * np.float32(scale)
    return e4m3_encode(prod.astype(np.float64))


def amax(x) -> float:
    """max |x| over the whole tensor; NaN if the tensor holds a NaN."""
    a = np.abs(f64(x))
    return float(np.nan) if np.isnan(a).any() else float(a.max(initial=0.0))


def fp8_linear(x, w, b, s_x: float, s_w: float) -> np.ndarray:
    """(q(x) q(w)^T) / (s_x s_w) + b with both operands quantized (F3)."""
    xq = e4m3_decode(quantize(x, s_x))
    wq = e4m3_decode(quantize(w, s_w))
    y = (xq @ wq.T) / (np.float64(np.float32(s_x)) * np.float64(np.float32(s_w)))
    return y + f64(b) if b is not None else y


def scale_update(history: np.ndarray, amax_now: float, scale: float, algo: str = "most_recent",
                 margin: int = 0) -> Tuple[np.ndarray, float, bool]:
    """One delayed-scaling update (F4).

    history: the tensor's past amaxes, oldest first (at most HISTORY_LEN).
    Returns (history with amax_now appended and the oldest dropped beyond
    HISTORY_LEN, new scale as an fp32 value, whether amax_now was not finite)."""
    hist = np.append(np.asarray(history, dtype=np.float32), np.float32(amax_now))[-HISTORY_LEN:]
    if algo == "most_recent":
        sel = np.float32(amax_now)
    elif algo == "max":
        sel = np.float32(np.nan) if np.isnan(hist).any() else np.float32(hist.max())
    else:
        raise ValueError(algo)
    nonfinite = not np.isfinite(np.float32(amax_now))
    new = np.float32(scale)
    if np.isfinite(sel) and sel > 0:
        with np.errstate(over="ignore", divide="ignore"):
            cand = np.float32(np.float32(E4M3_MAX) / sel) * np.float32(2.0 ** -margin)
        if _usable_scale(cand):
            new = cand
    return hist, float(new), nonfinite


def _usable_scale(s) -> bool:
    """A new scale replaces the old one only when it and its reciprocal are
    finite, non-zero fp32 values (reading F9: a selected amax so small that
    448 / amax overflows fp32 keeps the previous scale, as a non-finite amax
    does; otherwise the cast would multiply zeros by infinity)."""
    s = np.float32(s)
    with np.errstate(over="ignore", divide="ignore"):
        inv = np.float32(1.0) / s
    return bool(np.isfinite(s) and s > 0 and np.isfinite(inv))


def current_scale(x, scale_before: float = 1.0) -> float:
    """Current ("tensorwise") scaling, the recipe the page lists beside delayed
    scaling (F6): the scale of a tensor comes from its own amax,
    fp32(448 / fp32(amax)); a zero or non-finite amax, or one whose scale
    overflows fp32 (F9), keeps scale_before."""
    a = np.float32(amax(x))
    if np.isfinite(a) and a > 0:
        with np.errstate(over="ignore", divide="ignore"):
            cand = np.float32(np.float32(E4M3_MAX) / a)
        if _usable_scale(cand):
            return float(cand)
    return float(np.float32(scale_before))


def fp8_linears(scales: Dict[str, Tuple[float, float]],
                seen: Optional[Dict[str, float]] = None) -> Callable:
    """Linear hook for the block functions of the oracle: the token-path
    linears named in `scales` ({name: (s_x, s_w)}, names like "img_qkv",
    "txt_fc2", "lin1") run as fp8_linear; any other name runs in full
    precision.  `seen` collects amax(x) of each quantized input."""
    def lin(name: str, x, w, b):
        if name not in scales:
            return linear(x, w, b)
        if seen is not None:
            seen[name] = amax(x)
        s_x, s_w = scales[name]
        return fp8_linear(x, w, b, s_x, s_w)
    return lin


def attention_fp8(q, k, v):
    """Softmax attention on E4M3 operands (F7): q, k, v [B, L, H, Dh] are
    quantized with their current scales and dequantized with fp32(1 / s);
    returns (o [B, Lq, H * Dh], (s_q, s_k, s_v))."""
    scales = tuple(current_scale(x) for x in (q, k, v))
    deq = [e4m3_decode(quantize(x, sx)) * float(np.float32(1.0) / np.float32(sx)) for x, sx in zip((q, k, v), scales)]
    return attention(*deq), scales


# ------------------------------- blockwise (F8) -------------------------------
BLOCK_K = 128


def block_exponents(x, tile_rows: int) -> np.ndarray:
    """Exponent e of every tile_rows x 128 tile of x [R, K] (F8), int64
    [ceil(R / tile_rows), K / 128]: the largest integer with amax * 2^e <= 448."""
    x = f64(x)
    R, K = x.shape
    assert K % BLOCK_K == 0 and tile_rows >= 1
    assert np.isfinite(x).all(), "blockwise tiles must be finite"
    nt = -(-R // tile_rows)
    a = np.zeros((nt, K // BLOCK_K))
    for t in range(nt):
        blk = np.abs(x[t * tile_rows:(t + 1) * tile_rows])
        a[t] = blk.reshape(blk.shape[0], K // BLOCK_K, BLOCK_K).max(axis=(0, 2))
    # a = m 2^E with m in [0.5, 1): a 2^e <= 448 = 0.875 2^9  <=>  m 2^(E + e) <= 0.875 2^9
    m, E = np.frexp(np.where(a > 0, a, 1.0))
    e = np.where(m <= 0.875, 9 - E, 8 - E).astype(np.int64)
    e = np.where(a > 0, e, 0)
    return np.clip(e, -127, 127)


def block_quantize(x, tile_rows: int) -> Tuple[np.ndarray, np.ndarray]:
    """(E4M3 codes [R, K], tile exponents) of x under F8."""
    x = f64(x)
    e = block_exponents(x, tile_rows)
    per_row = np.repeat(e, tile_rows, axis=0)[: x.shape[0]]
    return e4m3_encode(x * np.repeat(np.exp2(per_row.astype(np.float64)), BLOCK_K, axis=1)), e


def block_dequantize(codes, e, tile_rows: int) -> np.ndarray:
    codes = np.asarray(codes)
    per_row = np.repeat(np.asarray(e, dtype=np.int64), tile_rows, axis=0)[: codes.shape[0]]
    return e4m3_decode(codes) * np.repeat(np.exp2(-per_row.astype(np.float64)), BLOCK_K, axis=1)


def block_linear(x, w, b=None) -> np.ndarray:
    """x [M, K] in 1 x 128 tiles and w [N, K] in 128 x 128 tiles (F8),
    y = deq(x) deq(w)^T (+ b) in fp64: every product of two E4M3 values and
    two powers of two is exact, so this is F8's block sum up to fp64 rounding."""
    xq, ex = block_quantize(x, 1)
    wq, ew = block_quantize(w, 128)
    y = block_dequantize(xq, ex, 1) @ block_dequantize(wq, ew, 128).T
    return y + f64(b) if b is not None else y
