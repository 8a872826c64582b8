"""GPU parity of the MXFP8 linear (the "mxfp8" recipe of "FP8 training for
Flux models", Configuration; block-scaled E4M3 in the OCP MX format) against
oracle/mx_oracle.py:

  * flux_mx_quantize: codes and E8M0 scale bytes bit-exact for bf16 and fp32
    sources, ragged row counts, zero, tiny, huge and non-finite blocks;
  * flux_mxfp8_linear_fwd: bit-exact when every partial sum is exact (small
    integer codes, power-of-two scales), and within 2e-4 of the fp64 oracle
    on random data (the scaled fp8 MFMA sums the E4M3 products of a 64-wide
    step inside the instruction with less than fp32 precision), including
    ragged M and N at the Flux-12B block widths.
"""
import numpy as np
import pytest

from oracle import fp8_oracle as Q
from oracle import mx_oracle as MX
from flow_matching_diffusion_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from flow_matching_diffusion_amd import flux
    flux.lib()
    torch.cuda.set_device(0)


def F():
    from flow_matching_diffusion_amd import flux
    return flux


def _quantize_gpu(x, bf16):
    rows, k = x.shape
    if bf16:
        src = torch.from_numpy(synth.bf16_bits(synth.round_to_bf16(x)).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        src = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    codes = torch.empty((rows, k), dtype=torch.uint8, device="cuda")
    scales = torch.full((F().flux_mx_scale_bytes(rows, k),), 0xAB, dtype=torch.uint8, device="cuda")
    F().flux_mx_quantize(F().FLUX_PREC_BF16 if bf16 else F().FLUX_PREC_F32, src, rows, k, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def _host_value(x, bf16):
    return synth.round_to_bf16(x).astype(np.float64) if bf16 else x.astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("rows,k,bf16", [(1, 64, True), (77, 192, True), (300, 512, False), (256, 3072, True)])
def test_mx_quantize_bitexact(rows, k, bf16):
    _say(f"MX quantize rows={rows} k={k} bf16={bf16}")
    rng = np.random.default_rng(rows * 7 + k)
    x = rng.standard_normal((rows, k)) * np.exp2(rng.integers(-40, 40, size=(rows, 1)))
    x[0, :32] = 0.0                                      # all-zero block
    if rows > 2:
        x[1, 32:64] *= 2.0 ** -100                       # tiny block (exponent clamps to -127 in fp32)
        x[2, :32] = rng.standard_normal(32) * 1e30       # huge block
    xv = _host_value(x, bf16)
    codes, scales = _quantize_gpu(x, bf16)
    rq, rs = MX.mx_quantize(xv)
    got_s = F().mx_scales_unswizzle(scales.cpu().numpy(), rows, k)
    assert np.array_equal(got_s, rs)
    assert np.array_equal(codes.cpu().numpy(), rq)


def test_mx_quantize_nonfinite_block():
    _say("MX quantize non-finite blocks")
    x = np.ones((4, 64), dtype=np.float32)
    x[1, 3] = np.nan
    x[2, 40] = np.inf
    x[3, :] = 1e-3
    codes, scales = _quantize_gpu(x, False)
    rq, rs = MX.mx_quantize(x.astype(np.float64))
    got_s = F().mx_scales_unswizzle(scales.cpu().numpy(), 4, 64)
    assert np.array_equal(got_s, rs)
    assert got_s[1, 0] == 0xFF and got_s[2, 1] == 0xFF
    assert np.array_equal(codes.cpu().numpy(), rq)


def _linear_gpu(xq, xs, wq, ws, b, m, n, k):
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    bd = None
    if b is not None:
        bd = torch.from_numpy(synth.bf16_bits(b).view(np.int16)).cuda().view(torch.bfloat16)
    F().flux_mxfp8_linear_fwd(m, n, k, xq, xs, wq, ws, bd, y, n)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


# k = 384 and 1152 give an odd number of 128-wide k super-stages: the GEMM then
# runs on the 64-byte-stage kernel instead of the ring of operand halves
@pytest.mark.parametrize("m,n,k", [(256, 256, 256), (300, 132, 512), (300, 132, 384)])
def test_mxfp8_linear_exact_on_small_integers(m, n, k):
    # codes of integers |v| <= 8 with block exponents in [-1, 1]: every product
    # and every partial sum (at most 2^17 in steps of 2^-2) is an exactly
    # representable fp32 value
    _say(f"MXFP8 linear exact m={m} n={n} k={k}")
    rng = np.random.default_rng(m + n + k)
    xi = rng.integers(-8, 9, size=(m, k)).astype(np.float64)
    wi = rng.integers(-8, 9, size=(n, k)).astype(np.float64)
    xi[:, ::32] = 8.0
    wi[:, ::32] = 8.0                                    # anchor: block max 8 -> X = 3 - 8 = -5
    ex = rng.integers(-1, 2, size=(m, k // 32))
    ew = rng.integers(-1, 2, size=(n, k // 32))
    x = xi * np.repeat(np.exp2(ex.astype(float)), 32, axis=1)
    w = wi * np.repeat(np.exp2(ew.astype(float)), 32, axis=1)
    xq, xs = _quantize_gpu(x, False)
    wq, ws = _quantize_gpu(w, False)
    got = _linear_gpu(xq, xs, wq, ws, None, m, n, k)
    ref = MX.mx_linear(x, w)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("m,n,k", [(512, 768, 3072), (4608 + 97, 3072 + 4, 3072), (1000, 12288, 256), (520, 256, 1152)])
def test_mxfp8_linear(m, n, k):
    _say(f"MXFP8 linear m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 3 + n + k)
    x = rng.standard_normal((m, k)) * np.exp2(rng.integers(-4, 4, size=(m, 1)))
    w = rng.standard_normal((n, k)) * 0.02
    b = synth.round_to_bf16(rng.standard_normal(n) * 0.02)
    xq, xs = _quantize_gpu(x, True)
    wq, ws = _quantize_gpu(w, True)
    got = _linear_gpu(xq, xs, wq, ws, b, m, n, k)
    rows = np.arange(m) if m <= 512 else np.unique(np.r_[rng.choice(m, 96, replace=False), 0, m - 1])
    ref = MX.mx_linear(_host_value(x[rows], True), _host_value(w, True), b.astype(np.float64))
    g = got[rows]
    err = np.abs(g - ref).max() / np.abs(ref).max()
    rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
    print(f"    MXFP8 linear: max_err/max={err:.2e} rel_l2={rel:.2e}", flush=True)
    assert np.isfinite(got).all() and err <= 2e-4 and rel <= 1e-4
    # and within E4M3 precision of the exact product (the recipe itself)
    exact = _host_value(x[rows], True) @ _host_value(w, True).T + b
    assert np.linalg.norm(g - exact) / np.linalg.norm(exact) <= 5e-2
