"""CPU tests of the C ABI boundary: the library loads, exports every symbol
include/flux.h declares, and rejects bad arguments on the host with the
documented status codes before anything is enqueued (no GPU is touched)."""
import ctypes as C
import os
import re

import pytest

from flow_matching_diffusion_amd import flux as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flux.h")

pytestmark = pytest.mark.skipif(not os.path.exists(F.LIB_PATH), reason="libflux.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:flux_status|size_t|int32_t|int64_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 15
    L = F.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(F.EXPORTED)


def test_status_strings():
    L = F.lib()
    assert L.flux_status_string(0) == b"ok"
    assert L.flux_status_string(3) == b"workspace too small"


def _dims(**kw):
    base = dict(batch=1, l_img=64, l_txt=16, hidden=256, heads=4, head_dim=64, mlp_hidden=1024, axes_dim=(8, 28, 28),
                precision=F.FLUX_PREC_BF16)
    base.update(kw)
    return F.make_dims(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=256, heads=8, head_dim=32, axes_dim=(8, 12, 12)), F.FLUX_ERR_UNSUPPORTED),
    (dict(hidden=300, heads=4, head_dim=75), F.FLUX_ERR_UNSUPPORTED),
    (dict(hidden=256, heads=2, head_dim=64), F.FLUX_ERR_INVALID_ARGUMENT),
    (dict(axes_dim=(8, 28, 30)), F.FLUX_ERR_INVALID_ARGUMENT),
    (dict(axes_dim=(7, 29, 28)), F.FLUX_ERR_INVALID_ARGUMENT),
    (dict(batch=0), F.FLUX_ERR_INVALID_ARGUMENT),
    (dict(l_img=0), F.FLUX_ERR_INVALID_ARGUMENT),
    (dict(mlp_hidden=100), F.FLUX_ERR_UNSUPPORTED),
    (dict(precision=7), F.FLUX_ERR_INVALID_ARGUMENT),
    (dict(l_img=(1 << 23) - 16, heads=2, head_dim=128, axes_dim=(16, 56, 56)), F.FLUX_ERR_UNSUPPORTED),
])
def test_bad_dims_rejected(kw, status):
    L = F.lib()
    d = _dims(**kw)
    assert L.flux_block_fwd(C.byref(d), None, None, None, 0, None, 0, None, None, None, 0, None) == status
    assert L.flux_last_error()
    assert L.flux_single_fwd(C.byref(d), None, None, 0, None, None, None, 0, None) == status
    assert L.flux_single_seq_fwd(C.byref(d), None, None, 0, None, None, None, 0, None) == status
    assert F.flux_workspace_bytes(d, 0) == 0 and F.flux_workspace_bytes(d, 2) == 0


def test_null_and_misaligned_pointers_rejected():
    L = F.lib()
    d = _dims()
    fake = 1 << 40                          # never dereferenced: validation fails first
    w = F.flux_stream_weights(*([fake] * 12))
    ws_need = F.flux_workspace_bytes(d, 0)
    assert ws_need > 0
    # missing residual pointer
    s = L.flux_block_fwd(C.byref(d), C.byref(w), C.byref(w), None, 64 * 256, fake, 16 * 256, fake, fake, fake,
                         ws_need, None)
    assert s == F.FLUX_ERR_INVALID_ARGUMENT
    # misaligned residual
    s = L.flux_block_fwd(C.byref(d), C.byref(w), C.byref(w), fake + 4, 64 * 256, fake, 16 * 256, fake, fake, fake,
                         ws_need, None)
    assert s == F.FLUX_ERR_INVALID_ARGUMENT and b"aligned" in L.flux_last_error()
    # batch stride smaller than a sample
    s = L.flux_block_fwd(C.byref(d), C.byref(w), C.byref(w), fake, 10, fake, 16 * 256, fake, fake, fake, ws_need,
                         None)
    assert s == F.FLUX_ERR_INVALID_ARGUMENT
    # a NULL weight
    w2 = F.flux_stream_weights(*([fake] * 12))
    w2.fc2_b = None
    s = L.flux_block_fwd(C.byref(d), C.byref(w2), C.byref(w), fake, 64 * 256, fake, 16 * 256, fake, fake, fake,
                         ws_need, None)
    assert s == F.FLUX_ERR_INVALID_ARGUMENT and b"NULL" in L.flux_last_error()
    # workspace too small / misaligned
    s = L.flux_block_fwd(C.byref(d), C.byref(w), C.byref(w), fake, 64 * 256, fake, 16 * 256, fake, fake, fake,
                         ws_need - 1, None)
    assert s == F.FLUX_ERR_WORKSPACE_TOO_SMALL
    s = L.flux_block_fwd(C.byref(d), C.byref(w), C.byref(w), fake, 64 * 256, fake, 16 * 256, fake, fake, fake + 16,
                         ws_need, None)
    assert s == F.FLUX_ERR_INVALID_ARGUMENT
    # sequential single block: the joint sequence as one stream (x stride covers l_img + l_txt rows)
    ws_seq = F.flux_workspace_bytes(d, 2)
    assert ws_seq > 0
    s = L.flux_single_seq_fwd(C.byref(d), C.byref(w), fake, 64 * 256, fake, fake, fake, ws_seq, None)
    assert s == F.FLUX_ERR_INVALID_ARGUMENT and b"bstride" in L.flux_last_error()
    s = L.flux_single_seq_fwd(C.byref(d), C.byref(w2), fake, 80 * 256, fake, fake, fake, ws_seq, None)
    assert s == F.FLUX_ERR_INVALID_ARGUMENT and b"NULL" in L.flux_last_error()
    s = L.flux_single_seq_fwd(C.byref(d), C.byref(w), fake, 80 * 256, fake, fake, fake, ws_seq - 1, None)
    assert s == F.FLUX_ERR_WORKSPACE_TOO_SMALL


def test_rf_argument_checks():
    L = F.lib()
    fake = 1 << 40
    a = F.rf_args()
    a.batch, a.n_per_sample = 2, 1000
    assert L.rf_noise_loss(C.byref(a), None) == F.FLUX_ERR_INVALID_ARGUMENT      # z0/z1/t missing
    a.z0, a.z1, a.t = fake, fake + 8000, fake + 16000
    a.z_t = fake + 4000                                                         # overlaps z0
    assert L.rf_noise_loss(C.byref(a), None) == F.FLUX_ERR_INVALID_ARGUMENT
    a.z_t = None
    a.loss = fake + 1 << 20                                                     # loss without v_pred
    assert L.rf_noise_loss(C.byref(a), None) == F.FLUX_ERR_INVALID_ARGUMENT
    a.v_pred = fake + (2 << 20)
    a.workspace, a.workspace_bytes = fake + (4 << 20), 8
    assert L.rf_noise_loss(C.byref(a), None) == F.FLUX_ERR_WORKSPACE_TOO_SMALL
    a.batch = 0
    assert L.rf_noise_loss(C.byref(a), None) == F.FLUX_ERR_INVALID_ARGUMENT


def test_embed_text_at_hidden_width_checks():
    """flux_embed_fwd without txt_in copies txt into x_txt only when the text
    is already [B, l_txt, hidden]: another width, a short batch stride or a
    misaligned pointer is rejected before anything is enqueued."""
    L = F.lib()
    fake = 1 << 40
    w = F.flux_embed_weights()
    w.img_in_w, w.img_in_b, w.time_in1_w, w.time_in1_b, w.time_in2_w, w.time_in2_b = (fake + i * 4096 for i in range(6))
    B, Cc, H, W, Lt, D = 1, 64, 2, 2, 4, 256
    z, t, x_img, vec, txt, x_txt, ws = (fake + (1 << 30) + i * (1 << 24) for i in range(7))

    def call(ctx_dim, txt_bstride, txt_ptr=txt):
        return L.flux_embed_fwd(F.FLUX_PREC_BF16, B, Cc, H, W, Lt, ctx_dim, D, 256, 0, C.byref(w), z, txt_ptr, t,
                                None, None, x_img, H * W * D, x_txt, txt_bstride, vec, ws, 8, None)
    assert call(100, Lt * D) == F.FLUX_ERR_INVALID_ARGUMENT                 # text width is not the hidden width
    assert b"l_txt, hidden" in L.flux_last_error()
    assert call(0, Lt * D - 4) == F.FLUX_ERR_INVALID_ARGUMENT               # batch stride shorter than a sample
    assert call(D, Lt * D, txt + 8) == F.FLUX_ERR_INVALID_ARGUMENT           # misaligned text
    assert call(0, Lt * D) == F.FLUX_ERR_WORKSPACE_TOO_SMALL                 # arguments fine, workspace too small


def test_linear_and_attention_argument_checks():
    L = F.lib()
    fake = 1 << 40
    assert L.flux_linear_fwd(F.FLUX_PREC_BF16, 16, 64, 100, fake, 100, fake, None, fake, 64, None) == \
        F.FLUX_ERR_UNSUPPORTED                                                  # bf16 K % 64
    assert L.flux_linear_fwd(F.FLUX_PREC_BF16, 16, 66, 64, fake, 64, fake, None, fake, 68, None) == \
        F.FLUX_ERR_UNSUPPORTED                                                  # N % 4
    assert L.flux_attention_fwd(F.FLUX_PREC_BF16, 1, 80, 4, 96, fake, fake, fake, 384, fake, 384, fake, 1 << 30,
                                None) == F.FLUX_ERR_UNSUPPORTED                # head_dim 96
    # one head's keys reach 2 GiB: the attention loads use 32-bit byte offsets
    assert L.flux_attention_fwd(F.FLUX_PREC_BF16, 1, 1 << 23, 1, 128, fake, fake, fake, 128, fake, 128, fake,
                                1 << 40, None) == F.FLUX_ERR_UNSUPPORTED
    assert L.flux_attention_fwd_train(1, 1 << 23, 1, fake, fake, fake, 128, fake, 128, fake, fake, 1 << 40,
                                      None) == F.FLUX_ERR_UNSUPPORTED
    need = F.flux_attention_workspace_bytes(F.FLUX_PREC_BF16, 1, 80, 4, 64)
    assert L.flux_attention_fwd(F.FLUX_PREC_BF16, 1, 80, 4, 64, fake, fake, fake, 256, fake, 256, fake, need - 1,
                                None) == F.FLUX_ERR_WORKSPACE_TOO_SMALL


def test_workspace_sizes_grow_with_problem():
    small = F.flux_workspace_bytes(_dims(), 0)
    big = F.flux_workspace_bytes(_dims(batch=4), 0)
    assert 0 < small < big
    assert F.flux_workspace_bytes(_dims(), 1) > 0
    assert F.flux_workspace_bytes(_dims(), 2) == F.flux_workspace_bytes(_dims(), 0)   # one-stream double block
    assert F.flux_workspace_bytes(_dims(), 3) == 0
    assert F.flux_rf_workspace_bytes(2, 1 << 20) >= 2 * 8


def test_convert_and_weights_f16_checks():
    L = F.lib()
    fake = 1 << 40
    assert L.flux_convert_bf16_to_f16(fake, fake + 8, 100, None) == F.FLUX_ERR_INVALID_ARGUMENT   # misaligned
    assert L.flux_convert_bf16_to_f16(fake, fake + 64, 100, None) == F.FLUX_ERR_INVALID_ARGUMENT  # overlap
    assert L.flux_convert_bf16_to_f16(fake, fake + 4096, 0, None) == F.FLUX_ERR_INVALID_ARGUMENT
    d = _dims(precision=F.FLUX_PREC_F32, weights_f16=1)
    assert F.flux_workspace_bytes(d, 0) == 0      # fp16-held weights need FLUX_PREC_BF16
    assert F.flux_workspace_bytes(_dims(weights_f16=1), 0) > 0


def test_mx_scale_layout_helper():
    # the binding's unswizzle inverts the byte layout flux.h documents
    import numpy as np
    rows, k = 300, 192
    rp = 512
    buf = np.zeros(F.flux_mx_scale_bytes(rows, k), dtype=np.uint8)
    assert buf.size == rp * (k // 32)
    ref = np.zeros((rp, k // 32), dtype=np.uint8)
    for row in range(rp):
        for kb in range(k // 32):
            v = (row * 7 + kb * 13) % 251
            ref[row, kb] = v
            buf[(((row // 128) * (k // 64) + kb // 2) * 2 + kb % 2) * 128 + (row % 32) * 4 + (row // 32) % 4] = v
    assert np.array_equal(F.mx_scales_unswizzle(buf, rows, k), ref[:rows])


def test_mxfp4_scale_layout_helper():
    # the binding's unswizzle inverts the MXFP4 byte layout flux.h documents
    import numpy as np
    rows, k = 300, 384
    rp = 512
    assert F.flux_mxfp4_scale_bytes(rows, 320) == 0          # k must be a multiple of 128
    buf = np.zeros(F.flux_mxfp4_scale_bytes(rows, k), dtype=np.uint8)
    assert buf.size == rp * (k // 32)
    ref = np.zeros((rp, k // 32), dtype=np.uint8)
    seen = set()
    for row in range(rp):
        for kb in range(k // 32):
            v = (row * 7 + kb * 13) % 251
            ref[row, kb] = v
            off = (((row // 128) * (k // 128) + kb // 4) * 512 + (kb % 2) * 256 + (row % 32) * 8
                   + ((kb % 4) // 2) * 4 + (row // 32) % 4)
            seen.add(off)
            buf[off] = v
    assert len(seen) == buf.size                               # the layout is a bijection
    assert np.array_equal(F.mxfp4_scales_unswizzle(buf, rows, k), ref[:rows])


def test_mx_and_blockwise_argument_checks():
    # rejected before any device work: bad tile shape, k, row count, MXFP4 linear k
    L = F.lib()
    fake = 1 << 40
    bf = F.FLUX_PREC_BF16
    assert L.flux_fp8_block_quantize(bf, fake, 256, 256, 2, fake, fake, None) == F.FLUX_ERR_INVALID_ARGUMENT
    assert L.flux_fp8_block_quantize(bf, fake, 256, 192, 1, fake, fake, None) == F.FLUX_ERR_INVALID_ARGUMENT
    assert L.flux_fp8_block_quantize(bf, fake, 8388480 + 1, 128, 128, fake, fake, None) == \
        F.FLUX_ERR_INVALID_ARGUMENT
    assert L.flux_mxfp4_quantize(bf, fake, 256, 192, fake, fake, None) == F.FLUX_ERR_INVALID_ARGUMENT
    assert L.flux_mxfp4_linear_fwd(256, 256, 384, fake, fake, fake, fake, None, fake, 256, None) == \
        F.FLUX_ERR_UNSUPPORTED
    assert L.flux_mxfp4_linear_fwd(256, 258, 512, fake, fake, fake, fake, None, fake, 260, None) == \
        F.FLUX_ERR_UNSUPPORTED                                                  # N % 4
    assert F.flux_mxfp4_scale_bytes(300, 512) == 512 * 16


def test_missing_library_fails_loudly(tmp_path):
    # with the shared library absent the binding raises instead of falling back
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from flow_matching_diffusion_amd import flux as F\n"
            "F.LIB_PATH = %r\n"
            "try:\n"
            "    F.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "    sys.exit(0)\n"
            "sys.exit(3)\n") % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                str(tmp_path / "absent" / "libflux.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "missing" in r.stdout


def test_debug_checks_setting_and_null_status():
    # the setting is host state; the status read rejects NULL before touching the device
    prev = F.flux_debug_checks(None)
    try:
        F.flux_debug_checks(True)
        assert F.flux_debug_checks(None) is True
        assert F.flux_debug_checks(False) is True
        assert F.flux_debug_checks(None) is False
    finally:
        F.flux_debug_checks(prev)
    assert F.lib().flux_debug_status(None, 0) == 1
    assert b"status" in F.lib().flux_last_error()
