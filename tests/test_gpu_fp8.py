"""GPU parity of the FP8 (E4M3) path against the fp8 oracle ("FP8 training for
Flux models", Configuration: E4M3 linears, delayed scaling).

  * quantizer: bit-exact codes on every bf16 value under several scales, and
    the recorded amax exact;
  * scale update: bit-exact scale, history and flags against scale_update;
  * fp8 GEMM: bit-exact on integer operands (every partial sum exact), and
    within 2e-4 of the fp64 oracle on random codes: E4M3 products are exact,
    the fp8 MFMA sums them inside an instruction with less than fp32
    precision;
  * blocks: the delayed-scaling protocol (two forwards with updates, the
    third measured); the oracle takes the scales the GPU used.  Outputs meet
    relative L2 <= 5e-2; weight scales are bitwise fp32(448 / max|W|) and
    activation scales within 1e-2 of 448 / the oracle's own amax.
"""
import numpy as np
import pytest

import oracle as O
from oracle import fp8_oracle as Q
from flow_matching_diffusion_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL_L2_FP8 = 5e-2


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


def M():
    from flow_matching_diffusion_amd import model
    return model


def dev(a, bf16=False):
    return M().device_array(a, bf16)


def _records(n, scales=None, amax=None, hist=None, flags=None):
    """Host-built state records as a device uint8 tensor."""
    f = F()
    raw = np.zeros(n * f.FP8_TENSOR_BYTES, np.uint8)
    for i in range(n):
        words = raw[i * f.FP8_TENSOR_BYTES:(i + 1) * f.FP8_TENSOR_BYTES].view(np.uint32)
        fl = 0
        if scales is not None and scales[i] is not None:
            words[0] = np.float32(scales[i]).view(np.uint32)
            words[1] = (np.float32(1.0) / np.float32(scales[i])).view(np.uint32)
            fl |= f.FLUX_FP8_SCALE_SET
        if amax is not None:
            words[2] = np.float32(amax[i]).view(np.uint32) & np.uint32(0x7FFFFFFF)
        if flags is not None:
            fl |= flags[i]
        words[3] = fl
        if hist is not None and len(hist[i]):
            h = np.asarray(hist[i], np.float32)
            words[4] = len(h)
            words[5] = len(h) % f.FLUX_FP8_HISTORY
            words[8:8 + len(h)] = h.view(np.uint32)
    return torch.from_numpy(raw).cuda()


def _read_records(t, n):
    raw = t.cpu().numpy().tobytes()
    f = F()
    return [f.fp8_record_fields(raw[i * f.FP8_TENSOR_BYTES:(i + 1) * f.FP8_TENSOR_BYTES]) for i in range(n)]


# --------------------------------------------------------------------------- #
# quantizer
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("scale", [None, 448.0 / 3.7, 2.0 ** -3, 1000.5, 2.0 ** 20, 0.011])
def test_quantize_every_bf16_value(scale):
    _say(f"fp8 quantize all bf16 values scale={scale}")
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    src = torch.from_numpy((bits >> 16).astype(np.uint16).view(np.int16)).cuda().view(torch.bfloat16)
    rec = _records(1, [scale])
    dst = torch.empty(v.size, dtype=torch.uint8, device="cuda")
    F().flux_fp8_quantize(F().FLUX_PREC_BF16, src, v.size, rec, dst)
    torch.cuda.synchronize()
    with np.errstate(all="ignore"):
        ref = Q.quantize(v, 1.0 if scale is None else scale)
    assert np.array_equal(dst.cpu().numpy(), ref)
    r = _read_records(rec, 1)[0]
    assert np.isnan(r["amax"])                 # the bf16 NaN patterns are in the input


def test_quantize_fp32_source_ragged_and_amax():
    _say("fp8 quantize fp32 source, n % 16 != 0")
    rng = np.random.default_rng(2)
    v = (3.0 * rng.standard_normal(100_003)).astype(np.float32)
    v[:5] = [0.0, -0.0, 1e-30, -500.0, 2.0 ** -10]
    s = 448.0 / float(np.abs(v).max())
    rec = _records(1, [s])
    dst = torch.empty(v.size, dtype=torch.uint8, device="cuda")
    F().flux_fp8_quantize(F().FLUX_PREC_F32, dev(v), v.size, rec, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), Q.quantize(v, s))
    assert _read_records(rec, 1)[0]["amax"] == float(np.abs(v).max())


@pytest.mark.parametrize("bf16", [True, False])
def test_quantize_current_scaling(bf16):
    # the "tensorwise" recipe: the scale comes from this tensor's own amax
    _say(f"fp8 current scaling bf16={bf16}")
    rng = np.random.default_rng(5 if bf16 else 6)
    v = (rng.standard_normal(300_007) * 7.3).astype(np.float32)
    v[17] = -91.0
    if bf16:
        v = synth.round_to_bf16(v).astype(np.float32)
        src = torch.from_numpy(synth.bf16_bits(v).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        src = dev(v)
    rec = _records(1, [5.0])                     # a stale delayed scale that must be replaced
    dst = torch.empty(v.size, dtype=torch.uint8, device="cuda")
    F().flux_fp8_quantize_current(F().FLUX_PREC_BF16 if bf16 else F().FLUX_PREC_F32, src, v.size, rec, dst)
    torch.cuda.synchronize()
    s = Q.current_scale(v)
    r = _read_records(rec, 1)[0]
    assert r["scale"] == s and r["scale_inv"] == float(np.float32(1.0) / np.float32(s))
    assert r["amax"] == float(np.abs(v).max())
    assert np.array_equal(dst.cpu().numpy(), Q.quantize(v, s))
    # a zero tensor keeps the previous scale
    z = torch.zeros(1000, dtype=torch.float32, device="cuda")
    F().flux_fp8_quantize_current(F().FLUX_PREC_F32, z, 1000, rec, dst)
    torch.cuda.synchronize()
    assert _read_records(rec, 1)[0]["scale"] == s


# --------------------------------------------------------------------------- #
# delayed-scaling update
# --------------------------------------------------------------------------- #
def test_update_matches_oracle():
    _say("fp8 scale update")
    cases = [  # (scale before or None, amax, history, algo, margin)
        (None, 3.5, [], 0, 0), (None, 0.07312, [], 0, 2), (7.0, 0.0, [1.0], 0, 0), (7.0, np.inf, [], 0, 0),
        (7.0, np.nan, [], 1, 0), (None, 1.0, [10.0] + [1.0] * 1022, 1, 0), (None, 2.0, [10.0] + [1.0] * 1023, 1, 0),
        (3.0, 5e-39, [], 0, 0), (None, 448.0, [0.5, 900.0], 1, 1), (3.0, 1e-37, [], 0, 0),
        (None, 5e-39, [], 0, 0),
    ]
    n = len(cases)
    rec = _records(n, [c[0] for c in cases], [c[1] for c in cases], [c[2] for c in cases])
    for algo in (0, 1):
        idx = [i for i, c in enumerate(cases) if c[3] == algo]
        # one launch per (algo, margin) group over single records
        for i in idx:
            F().flux_fp8_update(rec[i * F().FP8_TENSOR_BYTES:].data_ptr(), 1, algo, cases[i][4])
    torch.cuda.synchronize()
    got = _read_records(rec, n)
    for (s0, a, h, algo, margin), g in zip(cases, got):
        hist, s, nonfinite = Q.scale_update(h, a, 1.0 if s0 is None else s0,
                                            "most_recent" if algo == 0 else "max", margin)
        assert g["scale"] == s or (s0 is None and s == 1.0 and not (g["flags"] & 1)), (a, g["scale"], s)
        assert bool(g["flags"] & F().FLUX_FP8_NONFINITE) == nonfinite
        assert g["amax"] == 0.0 and g["hist_len"] == len(hist)
        ring = np.array(g["history"][:g["hist_len"]], np.float32)
        same = (np.sort(ring) == np.sort(hist)) | (np.isnan(np.sort(ring)) & np.isnan(np.sort(hist)))
        assert same.all()
        if g["flags"] & 1:
            assert g["scale_inv"] == float(np.float32(1.0) / np.float32(g["scale"]))
            assert np.isfinite(g["scale"]) and np.isfinite(g["scale_inv"]) and g["scale_inv"] > 0
    # after an update whose 448 / amax overflowed, a cast of zeros gives zero codes (no 0 * inf = NaN)
    i = cases.index((3.0, 5e-39, [], 0, 0))
    r = rec[i * F().FP8_TENSOR_BYTES:(i + 1) * F().FP8_TENSOR_BYTES]
    z = torch.zeros(4096, dtype=torch.float32, device="cuda")
    dst = torch.full((4096,), 0x55, dtype=torch.uint8, device="cuda")
    F().flux_fp8_quantize(F().FLUX_PREC_F32, z, 4096, r, dst)
    torch.cuda.synchronize()
    assert int(dst.max().item()) == 0


# --------------------------------------------------------------------------- #
# fp8 GEMM
# --------------------------------------------------------------------------- #
def _codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38       # no NaN operands
    return c


LINEAR_SHAPES = [(80, 768, 256), (333, 1284, 512), (4100, 9216, 3072), (4608, 3072, 12288)]


@pytest.mark.parametrize("m,n,k", LINEAR_SHAPES)
def test_fp8_linear_exact_on_small_integers(m, n, k):
    """Operands that are integers in [-8, 8]: every partial sum is an integer
    below 2^24, so any correct movement of the data gives the exact result,
    whatever the order or internal precision of the accumulation."""
    _say(f"fp8 linear, integer operands, m={m} n={n} k={k}")
    rng = np.random.default_rng(7 * m + n + k)
    xi, wi = rng.integers(-8, 9, (m, k)), rng.integers(-8, 9, (n, k))
    xc, wc = Q.e4m3_encode(xi), Q.e4m3_encode(wi)
    rec = _records(2, [None, None])
    y = torch.empty((m, n), device="cuda")
    F().flux_fp8_linear_fwd(m, n, k, torch.from_numpy(xc).cuda(), k, torch.from_numpy(wc).cuda(), k,
                            rec.data_ptr(), rec.data_ptr() + F().FP8_TENSOR_BYTES, None, y, n)
    torch.cuda.synchronize()
    rows = np.arange(m) if m <= 512 else np.unique(np.r_[rng.choice(m, 96, replace=False), 0, m - 1])
    ref = xi[rows].astype(np.int64) @ wi.T.astype(np.int64)
    assert np.array_equal(y.cpu().numpy()[rows].astype(np.int64), ref)


@pytest.mark.parametrize("m,n,k", LINEAR_SHAPES)
def test_fp8_linear(m, n, k):
    """Random E4M3 codes (magnitudes 2^-9 .. 448).  Products are exact; the
    32x32x64 fp8 MFMA of the large-problem kernel sums them with less than
    fp32 precision inside an instruction (measured 4e-5 of the largest
    output), hence the bound of 2e-4 here."""
    _say(f"fp8 linear m={m} n={n} k={k}")
    rng = np.random.default_rng(m + n + k)
    xc, wc = _codes(rng, (m, k)), _codes(rng, (n, k))
    b = synth.round_to_bf16((0.5 * rng.standard_normal(n)).astype(np.float32))
    sx, sw = 448.0 / 3.1, 448.0 / 0.09
    rec = _records(2, [sx, sw])
    y = torch.empty((m, n), device="cuda")
    F().flux_fp8_linear_fwd(m, n, k, torch.from_numpy(xc).cuda(), k, torch.from_numpy(wc).cuda(), k,
                            rec.data_ptr(), rec.data_ptr() + F().FP8_TENSOR_BYTES, dev(b, True), y, n)
    torch.cuda.synchronize()
    rows = np.arange(m) if m <= 512 else np.unique(np.r_[rng.choice(m, 64, replace=False), 0, m - 1])
    sinv = float(np.float32(1.0) / np.float32(sx)) * float(np.float32(1.0) / np.float32(sw))
    ref = (Q.e4m3_decode(xc[rows]) @ Q.e4m3_decode(wc).T) * sinv + b.astype(np.float64)
    g = y.cpu().numpy()[rows].astype(np.float64)
    err = np.abs(g - ref).max() / np.abs(ref).max()
    rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
    print(f"    fp8 linear: max_err/max={err:.2e} rel_l2={rel:.2e}", flush=True)
    assert np.isfinite(g).all() and err <= 2e-4 and rel <= 1e-4


# --------------------------------------------------------------------------- #
# blocks under the delayed-scaling protocol
# --------------------------------------------------------------------------- #
def _run_fp8(wl, w2, w1, inp, ids, which, n_fwd=3):
    """n_fwd forwards from the same input, with the weight cast before and the
    scale update after each but the last.  Returns the last output and the
    state records (scales the last forward used, amaxes it recorded)."""
    stack = M().BlockStack(wl, [w2] if which == "double" else [], [w1] if which == "single" else [])
    x0 = np.concatenate([inp["x_img"], inp["x_txt"]], axis=1)
    vec = dev(inp["vec"])
    rope = stack.rope_table(dev(ids))
    for f in range(n_fwd):
        x = dev(x0)
        stack.fp8_cast_weights()
        if which == "double":
            stack.double_fwd(0, x, vec, rope)
        else:
            stack.single_fwd(0, x, vec, rope)
        if f < n_fwd - 1:
            stack.fp8_update()
    torch.cuda.synchronize()
    return x.cpu().numpy(), stack.fp8_records()


def _double_scales(recs):
    sc = {}
    for si, s in enumerate(("img", "txt")):
        for li, n in enumerate(Q.TOKEN_LINEARS_DOUBLE):
            sc[f"{s}_{n}"] = (recs[8 * si + 2 * li]["scale"], recs[8 * si + 2 * li + 1]["scale"])
    return sc


def _single_scales(recs):
    return {n: (recs[2 * li]["scale"], recs[2 * li + 1]["scale"]) for li, n in enumerate(Q.TOKEN_LINEARS_SINGLE)}


def _check_weight_scales(scales, w, key):
    for name, (_, s_w) in scales.items():
        amax_w = np.float32(np.abs(w[key(name)]).max())
        assert s_w == float(np.float32(448.0) / amax_w), (name, s_w)


def _check_act_scales(scales, seen, names):
    for n in names:
        s_x = scales[n][0]
        ref = 448.0 / seen[n]
        assert abs(s_x - ref) <= 1e-2 * ref, (n, s_x, ref)


def _close(g, o, what):
    g = np.asarray(g, np.float64)
    d = g - o
    a = float(np.abs(d).max())
    r = float(np.linalg.norm(d) / np.linalg.norm(o))
    print(f"    {what}: max_abs={a:.3e} rel_l2={r:.3e}", flush=True)
    assert np.isfinite(g).all() and r <= REL_L2_FP8, (what, a, r)


FP8_SMALL = synth.custom_workload("ragged_fp8", base="tiny_fp32", precision="fp8", batch=2, img_h=7, img_w=9,
                                  l_txt=11, hidden=256, heads=2, head_dim=128, mlp_hidden=512,
                                  axes_dim=(16, 56, 56))


def _fixture(wl):
    return (synth.double_block_weights(wl, 0), synth.single_block_weights(wl, 1), synth.block_inputs(wl),
            synth.joint_ids(wl))


def test_fp8_double_block_small():
    wl = FP8_SMALL
    _say("fp8 double block ragged (B=2, 63 + 11 tokens), delayed scaling")
    w2, w1, inp, ids = _fixture(wl)
    g, recs = _run_fp8(wl, w2, w1, inp, ids, "double")
    sc = _double_scales(recs)
    _check_weight_scales(sc, w2, lambda n: n + ".w")
    seen = {}
    ang = O.rope_angles(ids, wl.axes_dim, wl.theta)
    oi, ot = O.double_block(inp["x_img"], inp["x_txt"], inp["vec"], ang, w2, wl.heads, wl.eps,
                            lin=Q.fp8_linears(sc, seen))
    _check_act_scales(sc, seen, list(sc))
    _close(g[:, :wl.l_img], oi, "fp8 double img")
    _close(g[:, wl.l_img:], ot, "fp8 double txt")
    # the exact block is within the fp8 bound too (a sanity check of the recipe)
    pi, pt = O.double_block(inp["x_img"], inp["x_txt"], inp["vec"], ang, w2, wl.heads, wl.eps)
    _close(g[:, :wl.l_img], pi, "fp8 double img vs exact")


def test_fp8_single_block_small():
    wl = FP8_SMALL
    _say("fp8 single block ragged, delayed scaling")
    w2, w1, inp, ids = _fixture(wl)
    g, recs = _run_fp8(wl, w2, w1, inp, ids, "single")
    sc = _single_scales(recs)
    _check_weight_scales(sc, w1, lambda n: n + ".w")
    seen = {}
    ang = O.rope_angles(ids, wl.axes_dim, wl.theta)
    x = np.concatenate([inp["x_img"], inp["x_txt"]], axis=1)
    o = O.single_block(x, inp["vec"], ang, w1, wl.heads, wl.eps, lin=Q.fp8_linears(sc, seen))
    _check_act_scales(sc, seen, list(sc))
    _close(g, o, "fp8 single")


def test_fp8_adaln_zero_identity():
    wl = FP8_SMALL
    _say("fp8 adaLN-zero identity")
    w2, w1, inp, ids = _fixture(wl)
    z2 = {k: (np.zeros_like(v) if "_mod." in k else v) for k, v in w2.items()}
    z1 = dict(w1, **{"mod.w": np.zeros_like(w1["mod.w"]), "mod.b": np.zeros_like(w1["mod.b"])})
    x0 = np.concatenate([inp["x_img"], inp["x_txt"]], axis=1)
    assert np.array_equal(_run_fp8(wl, z2, z1, inp, ids, "double", 2)[0], x0)
    assert np.array_equal(_run_fp8(wl, z2, z1, inp, ids, "single", 2)[0], x0)


@pytest.fixture(scope="module")
def c5_case():
    wl = synth.WORKLOADS["flux12b_blocks_fp8"]
    _say("generating flux12b_blocks_fp8 weights")
    return (wl,) + _fixture(wl)


def _rows(wl, seed):
    rng = np.random.default_rng(seed)
    ri = np.unique(np.r_[rng.choice(wl.l_img, 16, replace=False), 0, wl.l_img - 1])
    rt = np.unique(np.r_[rng.choice(wl.l_txt, 6, replace=False), 0, wl.l_txt - 1])
    return ri, rt


@pytest.mark.slow
def test_fp8_double_block_c5_sampled(c5_case):
    wl, w2, w1, inp, ids = c5_case
    _say(f"fp8 double block B={wl.batch} L={wl.seq} sampled rows")
    g, recs = _run_fp8(wl, w2, w1, inp, ids, "double")
    sc = _double_scales(recs)
    _check_weight_scales(sc, w2, lambda n: n + ".w")
    ri, rt = _rows(wl, 3)
    seen = {}
    ang = O.rope_angles(ids, wl.axes_dim, wl.theta)
    oi, ot = O.double_block(inp["x_img"], inp["x_txt"], inp["vec"], ang, w2, wl.heads, wl.eps,
                            rows={"img": ri, "txt": rt}, lin=Q.fp8_linears(sc, seen))
    _check_act_scales(sc, seen, ["img_qkv", "txt_qkv"])     # the inputs evaluated on every row
    _close(g[:, ri], oi, "fp8 double img")
    _close(g[:, wl.l_img + rt], ot, "fp8 double txt")


@pytest.mark.slow
def test_fp8_single_block_c5_sampled(c5_case):
    wl, w2, w1, inp, ids = c5_case
    _say(f"fp8 single block B={wl.batch} L={wl.seq} sampled rows")
    g, recs = _run_fp8(wl, w2, w1, inp, ids, "single")
    sc = _single_scales(recs)
    _check_weight_scales(sc, w1, lambda n: n + ".w")
    ri, rt = _rows(wl, 4)
    sel = np.r_[ri, wl.l_img + rt]
    seen = {}
    ang = O.rope_angles(ids, wl.axes_dim, wl.theta)
    x = np.concatenate([inp["x_img"], inp["x_txt"]], axis=1)
    o = O.single_block(x, inp["vec"], ang, w1, wl.heads, wl.eps, rows=sel, lin=Q.fp8_linears(sc, seen))
    _check_act_scales(sc, seen, ["lin1"])
    _close(g[:, sel], o, "fp8 single")


# --------------------------- fp8 attention (F7) --------------------------- #
@pytest.mark.parametrize("B,L,H", [(1, 80, 2), (2, 333, 2), (1, 4608, 24)])
def test_attention_fp8(B, L, H):
    _say(f"fp8 attention B={B} L={L} H={H} Dh=128")
    rng = np.random.default_rng(L + 7 * H)
    D = H * 128
    q = synth.round_to_bf16(0.25 * rng.standard_normal((B, L, D)).astype(np.float32))
    k = synth.round_to_bf16(rng.standard_normal((B, L, D)).astype(np.float32))
    v = synth.round_to_bf16(rng.standard_normal((B, L, D)).astype(np.float32))
    f = F()
    rec = _records(3)
    o = torch.empty((B, L, D), dtype=torch.bfloat16, device="cuda")
    wsb = f.flux_attention_fp8_workspace_bytes(B, L, H)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    bf = lambda a: torch.from_numpy(synth.bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
    f.flux_attention_fp8_fwd(B, L, H, bf(q), bf(k), bf(v), D, o, D, rec, ws, wsb)
    torch.cuda.synchronize()
    # the recorded scales are the current scales of Q, K and V, bit for bit
    scales = tuple(Q.current_scale(x) for x in (q, k, v))
    assert tuple(r["scale"] for r in _read_records(rec, 3)) == scales
    # reference on the sampled query rows (all of them up to 512 tokens)
    rows = np.arange(L) if L <= 512 else np.unique(np.r_[rng.choice(L, 48, replace=False), 0, L - 1])
    hd = lambda a: a.reshape(a.shape[0], a.shape[1], H, 128)
    deq = lambda x, s: Q.e4m3_decode(Q.quantize(x, s)) * float(np.float32(1.0) / np.float32(s))
    ref8 = O.attention(hd(deq(q[:, rows], scales[0])), hd(deq(k, scales[1])), hd(deq(v, scales[2])))
    ref = O.attention(hd(q[:, rows]), hd(k), hd(v))
    got = o.float().cpu().numpy()[:, rows]
    rel8 = float(np.linalg.norm(got - ref8) / np.linalg.norm(ref8))
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"    fp8 attention: rel_l2 vs the fp8 oracle {rel8:.2e}, vs exact attention {rel:.2e}", flush=True)
    assert np.isfinite(got).all() and rel8 <= 5e-2 and rel <= 5e-2
