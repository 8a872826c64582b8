"""GPU parity of the blockwise E4M3 recipe ("FP8 training for Flux models",
Configuration lists "blockwise"; reading F8 of oracle/fp8_oracle.py: one
power-of-two scale per 1 x 128 activation tile or 128 x 128 weight tile):

  * flux_fp8_block_quantize: codes bit-exact and every E8M0 byte equal to
    127 - e of the oracle's tile exponent, for bf16 and fp32 sources, both
    tile shapes, ragged row counts, zero / tiny / huge tiles and the 448
    boundary; a non-finite tile gets the NaN byte 0xFF;
  * the linear (flux_mxfp8_linear_fwd on blockwise operands): bit-exact when
    every partial sum is exact, and within 2e-4 of the fp64 oracle on random
    data at the Flux-12B block widths.
"""
import numpy as np
import pytest

from oracle import fp8_oracle as Q
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


def _quantize_gpu(x, bf16, tile_rows):
    rows, k = x.shape
    if bf16:
        src = torch.from_numpy(synth.bf16_bits(synth.round_to_bf16(x)).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        src = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    codes = torch.full((rows, k), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((F().flux_mx_scale_bytes(rows, k),), 0xAB, dtype=torch.uint8, device="cuda")
    F().flux_fp8_block_quantize(F().FLUX_PREC_BF16 if bf16 else F().FLUX_PREC_F32, src, rows, k, tile_rows,
                                codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def _host_value(x, bf16):
    return synth.round_to_bf16(x).astype(np.float64) if bf16 else x.astype(np.float32).astype(np.float64)


def _expected_bytes(e, rows, tile_rows):
    per_row = np.repeat(e, tile_rows, axis=0)[:rows]
    return np.repeat((127 - per_row).astype(np.uint8), 4, axis=1)   # one byte per 32-value block


@pytest.mark.parametrize("rows,k,bf16,tile_rows", [(1, 128, True, 1), (77, 384, True, 1), (300, 512, False, 1),
                                                   (300, 512, True, 128), (256, 3072, False, 128),
                                                   (4608, 3072, True, 1)])
def test_block_quantize_bitexact(rows, k, bf16, tile_rows):
    _say(f"blockwise quantize rows={rows} k={k} bf16={bf16} tile_rows={tile_rows}")
    rng = np.random.default_rng(rows * 13 + k + tile_rows)
    x = rng.standard_normal((rows, k)) * np.exp2(rng.integers(-40, 40, size=(rows, 1)))
    x[0, :128] = 0.0                                     # all-zero tile (when tile_rows is 1)
    x[0, 128 % k] = 448.0 if k > 128 else x[0, 0]
    if rows > 2:
        x[1, :128] *= 2.0 ** -100                        # tiny tile
        x[2, :128] = rng.standard_normal(128) * 1e30     # huge tile
    xv = _host_value(x, bf16)
    codes, scales = _quantize_gpu(x, bf16, tile_rows)
    rq, re = Q.block_quantize(xv, tile_rows)
    got_s = F().mx_scales_unswizzle(scales.cpu().numpy(), rows, k)
    assert np.array_equal(got_s, _expected_bytes(re, rows, tile_rows))
    assert np.array_equal(codes.cpu().numpy(), rq)


def test_block_quantize_nonfinite_tile():
    _say("blockwise quantize non-finite tile")
    x = np.ones((4, 256), dtype=np.float32)
    x[1, 3] = np.nan
    x[2, 200] = np.inf
    codes, scales = _quantize_gpu(x, False, 1)
    got_s = F().mx_scales_unswizzle(scales.cpu().numpy(), 4, 256)
    assert (got_s[1, :4] == 0xFF).all() and (got_s[2, 4:] == 0xFF).all()
    assert (got_s[0] == 127 - 8).all() and (got_s[1, 4:] == 127 - 8).all()   # 1.0 * 2^8 = 256 <= 448
    rq, _ = Q.block_quantize(x[[0, 3]].astype(np.float64), 1)
    assert np.array_equal(codes.cpu().numpy()[[0, 3]], rq)


def _linear_gpu(xq, xs, wq, ws, b, m, n, k):
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    bd = None
    if b is not None:
        bd = torch.from_numpy(synth.bf16_bits(b).view(np.int16)).cuda().view(torch.bfloat16)
    F().flux_mxfp8_linear_fwd(m, n, k, xq, xs, wq, ws, bd, y, n)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("m,n,k", [(256, 256, 256), (300, 132, 512)])
def test_block_linear_exact_on_small_integers(m, n, k):
    # integer codes |v| <= 8 with each tile anchored at 8 (e = 5) and scaled
    # by 2^s, s in [-1, 1]: every product and partial sum is exact in fp32
    _say(f"blockwise linear exact m={m} n={n} k={k}")
    rng = np.random.default_rng(m + n + k + 1)
    xi = rng.integers(-8, 9, size=(m, k)).astype(np.float64)
    wi = rng.integers(-8, 9, size=(n, k)).astype(np.float64)
    xi[:, ::128] = 8.0
    wi[:, ::128] = 8.0
    sx = rng.integers(-1, 2, size=(m, k // 128))
    sw = np.repeat(rng.integers(-1, 2, size=(-(-n // 128), k // 128)), 128, axis=0)[:n]
    x = xi * np.repeat(np.exp2(sx.astype(float)), 128, axis=1)
    w = wi * np.repeat(np.exp2(sw.astype(float)), 128, axis=1)
    xq, xs = _quantize_gpu(x, False, 1)
    wq, ws = _quantize_gpu(w, False, 128)
    got = _linear_gpu(xq, xs, wq, ws, None, m, n, k)
    ref = Q.block_linear(x, w)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("m,n,k", [(512, 768, 3072), (4608 + 97, 3072 + 4, 3072), (333, 3072, 15360)])
def test_block_linear(m, n, k):
    _say(f"blockwise linear m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 7 + n + k)
    x = rng.standard_normal((m, k)) * np.exp2(rng.integers(-4, 4, size=(m, 1)))
    w = rng.standard_normal((n, k)) * 0.02
    b = synth.round_to_bf16(rng.standard_normal(n) * 0.02)
    xq, xs = _quantize_gpu(x, True, 1)
    wq, ws = _quantize_gpu(w, True, 128)
    got = _linear_gpu(xq, xs, wq, ws, b, m, n, k)
    rows = np.arange(m) if m <= 512 else np.unique(np.r_[rng.choice(m, 96, replace=False), 0, m - 1])
    ref = Q.block_linear(_host_value(x[rows], True), _host_value(w, True), b.astype(np.float64))
    g = got[rows]
    err = np.abs(g - ref).max() / np.abs(ref).max()
    rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
    print(f"    blockwise linear: max_err/max={err:.2e} rel_l2={rel:.2e}", flush=True)
    assert np.isfinite(got).all() and err <= 2e-4 and rel <= 1e-4
    exact = _host_value(x[rows], True) @ _host_value(w, True).T + b
    assert np.linalg.norm(g - exact) / np.linalg.norm(exact) <= 5e-2
