"""GPU parity of the MXFP4 linear (OCP MX v1.0 with E2M1 elements, the fp4
member of the microscaling family named by "FP8 training for Flux models",
Configuration) against oracle/mx_oracle.py:

  * flux_mxfp4_quantize: packed codes and E8M0 scale bytes bit-exact for bf16
    and fp32 sources, ragged row counts, zero, tiny and huge blocks and values
    on every rounding midpoint of the E2M1 grid (ties to the even code);
  * flux_mxfp4_linear_fwd: bit-exact when every partial sum is exact (grid
    values with power-of-two block scales), and within 2e-4 of the fp64
    oracle on random data, including ragged M and N at the Flux-12B block
    widths and the 15360-wide input of the single block's output linear.
"""
import numpy as np
import pytest

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
    codes = torch.full((rows, k // 2), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((F().flux_mxfp4_scale_bytes(rows, k),), 0xAB, dtype=torch.uint8, device="cuda")
    F().flux_mxfp4_quantize(F().FLUX_PREC_BF16 if bf16 else F().FLUX_PREC_F32, src, rows, k, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def _host_value(x, bf16):
    return synth.round_to_bf16(x).astype(np.float64) if bf16 else x.astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("rows,k,bf16", [(1, 128, True), (77, 384, True), (300, 512, False), (256, 3072, True)])
def test_mxfp4_quantize_bitexact(rows, k, bf16):
    _say(f"MXFP4 quantize rows={rows} k={k} bf16={bf16}")
    rng = np.random.default_rng(rows * 11 + k)
    x = rng.standard_normal((rows, k)) * np.exp2(rng.integers(-40, 40, size=(rows, 1)))
    x[0, :32] = 0.0                                      # all-zero block
    # a block anchored at 6 (X = 0) holding every midpoint of the E2M1 grid
    # and its neighbours, both signs: ties go to the even code
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, 7.0, 0.24, 0.26, 4.9])
    blk = np.zeros(32)
    blk[0] = 6.0
    blk[1:1 + len(mids)] = mids
    blk[1 + len(mids):1 + 2 * len(mids)] = -mids
    x[0, 32:64] = blk
    if rows > 2:
        x[1, 32:64] *= 2.0 ** -100                       # tiny block (exponent clamps to -127 in fp32)
        x[2, :32] = rng.standard_normal(32) * 1e30       # huge block
        x[2, 64:96] = -0.0                               # negative zeros keep their sign bit
    xv = _host_value(x, bf16)
    codes, scales = _quantize_gpu(x, bf16)
    rq, rs = MX.mxfp4_quantize(xv)
    got_s = F().mxfp4_scales_unswizzle(scales.cpu().numpy(), rows, k)
    assert np.array_equal(got_s, rs)
    assert np.array_equal(codes.cpu().numpy(), rq)


def _linear_gpu(xq, xs, wq, ws, b, m, n, k):
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    bd = None
    if b is not None:
        bd = torch.from_numpy(synth.bf16_bits(b).view(np.int16)).cuda().view(torch.bfloat16)
    F().flux_mxfp4_linear_fwd(m, n, k, xq, xs, wq, ws, bd, y, n)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def _grid_operand(rng, rows, k):
    # E2M1 grid values with the block maximum anchored at 6 (X = 0), then
    # each block scaled by 2^e, e in [-1, 1]: the quantizer reproduces them
    # exactly
    g = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    v = g[rng.integers(0, 8, size=(rows, k))] * rng.choice([-1.0, 1.0], size=(rows, k))
    v[:, ::32] = 6.0
    e = rng.integers(-1, 2, size=(rows, k // 32))
    return v * np.repeat(np.exp2(e.astype(float)), 32, axis=1)


@pytest.mark.parametrize("m,n,k", [(256, 256, 512), (300, 132, 768), (64, 3072, 3072)])
def test_mxfp4_linear_exact_on_grid_values(m, n, k):
    # every product is a multiple of 2^-4 of magnitude at most 144 and every
    # partial sum stays below 2^19: all exactly representable in fp32
    _say(f"MXFP4 linear exact m={m} n={n} k={k}")
    rng = np.random.default_rng(m + n + k)
    x = _grid_operand(rng, m, k)
    w = _grid_operand(rng, n, k)
    xq, xs = _quantize_gpu(x, False)
    wq, ws = _quantize_gpu(w, False)
    got = _linear_gpu(xq, xs, wq, ws, None, m, n, k)
    ref = MX.mxfp4_linear(x, w)
    assert np.array_equal(MX.mxfp4_dequantize(*MX.mxfp4_quantize(x)), x)   # the operands are exact
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("m,n,k", [(512, 768, 3072), (4608 + 97, 3072 + 4, 3072), (333, 3072, 15360),
                                   (1000, 12288, 512)])
def test_mxfp4_linear(m, n, k):
    _say(f"MXFP4 linear m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 5 + n + k)
    x = rng.standard_normal((m, k)) * np.exp2(rng.integers(-4, 4, size=(m, 1)))
    w = rng.standard_normal((n, k)) * 0.02
    b = synth.round_to_bf16(rng.standard_normal(n) * 0.02)
    xq, xs = _quantize_gpu(x, True)
    wq, ws = _quantize_gpu(w, True)
    got = _linear_gpu(xq, xs, wq, ws, b, m, n, k)
    rows = np.arange(m) if m <= 512 else np.unique(np.r_[rng.choice(m, 96, replace=False), 0, m - 1])
    ref = MX.mxfp4_linear(_host_value(x[rows], True), _host_value(w, True), b.astype(np.float64))
    g = got[rows]
    err = np.abs(g - ref).max() / np.abs(ref).max()
    rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
    print(f"    MXFP4 linear: max_err/max={err:.2e} rel_l2={rel:.2e}", flush=True)
    assert np.isfinite(got).all() and err <= 2e-4 and rel <= 1e-4
    # and within E2M1 precision of the exact product (the recipe itself:
    # about 0.16 relative for Gaussian operands)
    exact = _host_value(x[rows], True) @ _host_value(w, True).T + b
    assert np.linalg.norm(g - exact) / np.linalg.norm(exact) <= 0.25


def test_mxfp4_linear_rejects_unsupported_k():
    _say("MXFP4 linear rejects k = 384")
    x = torch.zeros((256, 192), dtype=torch.uint8, device="cuda")
    s = torch.zeros((F().flux_mxfp4_scale_bytes(256, 384),), dtype=torch.uint8, device="cuda")
    y = torch.empty((256, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(F().FluxError) as ei:
        F().flux_mxfp4_linear_fwd(256, 256, 384, x, s, x, s, None, y, 256)
    assert ei.value.status == F().FLUX_ERR_UNSUPPORTED
