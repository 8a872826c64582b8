"""Pins of the MXFP8 oracle (oracle/mx_oracle.py): the shared exponent's
defining bounds, exact round trips of values on the scaled E4M3 grid (every
finite code, many exponents), zero, saturation and non-finite blocks, the
E4M3 error bound, and the block-scaled linear against a pure-Python sum over
blocks ("FP8 training for Flux models", Configuration: the mxfp8 recipe; the
OCP MX v1.0 format it names)."""
import math

import numpy as np
import pytest

from oracle import fp8_oracle as Q
from oracle import mx_oracle as MX

RNG = np.random.default_rng(2024)
FINITE_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_shared_exponent_bounds():
    # 2^8 <= amax / 2^X < 2^9 whenever X is not clamped
    mags = np.exp2(RNG.uniform(-110, 110, size=(200, 32)))
    x = mags * RNG.choice([-1.0, 1.0], size=mags.shape)
    X = MX.mx_exponents(x)
    r = np.abs(x).max(axis=-1) / np.exp2(X[:, 0].astype(float))
    assert np.all(r >= 256.0) and np.all(r < 512.0)
    # clamping at the ends of the E8M0 range
    assert MX.mx_exponents(np.full((1, 32), 2.0 ** -140))[0, 0] == -127
    assert MX.mx_exponents(np.full((1, 32), 1e300))[0, 0] == 127


@pytest.mark.parametrize("X0", [-100, -9, -1, 0, 3, 60])
def test_roundtrip_exact_on_the_scaled_grid(X0):
    # blocks of finite codes with one element at 256 (exponent field 15) fix the
    # block exponent at X0; the values 2^X0 * dec(code) must come back exactly
    codes = RNG.choice(FINITE_CODES, size=(64, 32))
    codes[:, 0] = 0x78                      # +256
    codes[:, 1:] = np.where(np.abs(Q.e4m3_decode(codes[:, 1:])) > 448, 0x7E, codes[:, 1:])
    x = Q.e4m3_decode(codes) * 2.0 ** X0
    q, s = MX.mx_quantize(x)
    assert np.all(s == X0 + 127)
    # -0.0 keeps its sign bit; every other code is reproduced
    assert np.array_equal(q, codes)


def test_every_finite_code_in_every_position():
    for X0 in (-20, 0, 7):
        for pos in range(32):
            x = np.zeros((len(FINITE_CODES), 32))
            x[:, (pos + 1) % 32] = 448.0 * 2.0 ** X0      # anchor: exponent X0
            x[:, pos] = Q.e4m3_decode(FINITE_CODES) * 2.0 ** X0
            q, s = MX.mx_quantize(x)
            assert np.all(s == X0 + 127)
            assert np.array_equal(q[:, pos], FINITE_CODES)


def test_zero_saturation_and_nonfinite_blocks():
    q, s = MX.mx_quantize(np.zeros((1, 64)))
    assert np.all(q == 0) and np.all(s == 0)
    x = np.zeros((1, 32))
    x[0, 0], x[0, 1] = 500.0, -470.0        # floor(log2 500) = 8 -> X = 0; both clip to 448
    q, s = MX.mx_quantize(x)
    assert s[0, 0] == 127 and q[0, 0] == 0x7E and q[0, 1] == 0xFE
    x[0, 5] = np.nan
    q, s = MX.mx_quantize(x)
    assert s[0, 0] == 0xFF and (q[0, 5] & 0x7F) == 0x7F
    assert np.isnan(MX.mx_dequantize(q, s)).all()


def test_error_bound():
    x = RNG.standard_normal((128, 256)) * np.exp2(RNG.integers(-30, 30, size=(128, 1)))
    q, s = MX.mx_quantize(x)
    d = MX.mx_dequantize(q, s)
    X = np.repeat(s.astype(float) - 127, 32, axis=-1)
    scaled = np.abs(x) / np.exp2(X)
    normal = (scaled >= 2.0 ** -6) & (scaled <= 448.0)
    sub = scaled < 2.0 ** -6
    clipped = scaled > 448.0
    # half an E4M3 ulp: 2^-4 relative for normals, 2^-10 * 2^X absolute below;
    # scaled magnitudes in (448, 512) clip to 448 (at most 1/8 relative)
    assert np.all(np.abs(d - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] + 1e-300)
    assert np.all(np.abs(d - x)[sub] <= 2.0 ** -10 * np.exp2(X)[sub])
    assert np.all(np.abs(d)[clipped] == 448.0 * np.exp2(X)[clipped])
    assert np.all(np.abs(d - x)[clipped] <= 0.125 * np.abs(x)[clipped])


def test_mx_linear_against_block_sums():
    m, n, k = 5, 3, 96
    x = RNG.standard_normal((m, k)) * 3.0
    w = RNG.standard_normal((n, k)) * 0.05
    b = RNG.standard_normal(n)
    got = MX.mx_linear(x, w, b)
    xq, xs = MX.mx_quantize(x)
    wq, ws = MX.mx_quantize(w)
    for r in range(m):
        for c in range(n):
            tot = 0.0
            for kb in range(k // 32):
                part = 0.0
                for kk in range(kb * 32, kb * 32 + 32):
                    part += float(Q.e4m3_decode(xq[r, kk])) * float(Q.e4m3_decode(wq[c, kk]))
                tot += math.ldexp(part, int(xs[r, kb]) - 127 + int(ws[c, kb]) - 127)
            assert abs(got[r, c] - (tot + b[c])) <= 1e-12 * max(1.0, abs(tot))
    # and the quantized product stays close to the exact one (E4M3 precision)
    ref = x @ w.T + b
    assert np.abs(got - ref).max() <= 0.1 * np.abs(x @ w.T).max() + 1e-12


# --------------------------------- MXFP4 --------------------------------- #
def test_e2m1_grid_and_rounding():
    # the grid the format defines, every code round-trips, ties go to the even code
    assert [float(MX.e2m1_decode(c)) for c in range(8)] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [float(MX.e2m1_decode(c)) for c in range(8, 16)] == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    for c in range(16):
        if c != 8:
            assert int(MX.e2m1_encode(MX.e2m1_decode(c))) == c
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for v, want in ties.items():
        assert float(MX.e2m1_decode(MX.e2m1_encode(v))) == want, v
        assert float(MX.e2m1_decode(MX.e2m1_encode(-v))) == -want, v
    assert float(MX.e2m1_decode(MX.e2m1_encode(100.0))) == 6.0
    assert float(MX.e2m1_decode(MX.e2m1_encode(0.26))) == 0.5 and float(MX.e2m1_decode(MX.e2m1_encode(0.24))) == 0.0
    # brute force: the encoder picks a nearest grid value for every input of a fine sweep
    xs = np.linspace(-7, 7, 2801)
    got = MX.e2m1_decode(MX.e2m1_encode(xs))
    grid = np.r_[-MX._E2M1[::-1], MX._E2M1]
    best = np.abs(np.clip(xs, -6, 6)[:, None] - grid[None, :]).min(axis=1)
    assert np.allclose(np.abs(np.clip(xs, -6, 6) - got), best, atol=0)


def test_mxfp4_exponent_and_roundtrip():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((5, 96)) * np.exp2(rng.integers(-20, 20, size=(5, 1)))
    packed, s = MX.mxfp4_quantize(x)
    X = s.astype(np.int64) - 127
    a = np.abs(x.reshape(5, 3, 32)).max(axis=-1)
    # the block max lands in [4, 8) after the shift: E2M1's top binade, rounded at most to 6
    assert np.all((a / np.exp2(X) >= 4) & (a / np.exp2(X) < 8))
    # values already on the scaled grid round-trip exactly
    grid = MX._E2M1[rng.integers(0, 8, size=(2, 64))] * np.where(rng.uniform(size=(2, 64)) < 0.5, -1, 1)
    grid[:, ::32] = 6.0
    y = grid * 2.0 ** 5
    assert np.array_equal(MX.mxfp4_dequantize(*MX.mxfp4_quantize(y)), y)
    # the even-indexed element sits in the low nibble
    p, _ = MX.mxfp4_quantize(np.r_[np.full(31, 6.0), 0.5].reshape(1, 32) * 1.0)
    assert p[0, 0] == (7 | (7 << 4)) and p[0, 15] == (7 | (1 << 4))


def test_mxfp4_linear_block_sum():
    rng = np.random.default_rng(32)
    x, w = rng.standard_normal((3, 64)), rng.standard_normal((4, 64))
    y = MX.mxfp4_linear(x, w)
    xq, xs = MX.mxfp4_quantize(x)
    wq, ws = MX.mxfp4_quantize(w)
    xd, wd = MX.mxfp4_dequantize(xq, xs), MX.mxfp4_dequantize(wq, ws)
    for i in range(3):
        for j in range(4):
            s = 0.0
            for kb in range(2):
                part = sum(xd[i, 32 * kb + t] * wd[j, 32 * kb + t] for t in range(32))
                s += part
            assert abs(y[i, j] - s) <= 1e-12 * max(1.0, abs(s))
    # and within E2M1 precision of the exact product
    assert np.linalg.norm(y - x @ w.T) / np.linalg.norm(x @ w.T) < 0.3
