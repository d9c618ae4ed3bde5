"""C-ABI boundary checks that need no GPU: the library loads, exports every function that
include/ssm_ternary.h declares, and rejects invalid calls on the host with the documented
status before anything is launched (the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest
import torch

import ternary_weight_selective_amd as tws

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_ternary.h")

OK, NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, UNSUPPORTED, DEVICE = range(8)
FAKE = 0x100000  # never dereferenced: every call below fails validation first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = tws.lib()
    declared = _declared()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(tws.EXPORTS) == declared


def test_version_and_status_strings():
    L = tws.lib()
    assert tws.ssm_abi_version() == 7
    for s in range(8):
        assert L.ssm_status_string(s)
    assert tws.ssm_packed_row_bytes(8) == 4
    assert tws.ssm_packed_row_bytes(16) == 4
    assert tws.ssm_packed_row_bytes(17) == 8
    assert tws.ssm_packed_row_bytes(4096) == 1024
    assert tws.ssm_packed_row_bytes(0) == 0


def _bl(**kw):
    a = tws.BitlinearArgs()
    a.x, a.x_dtype, a.act_bits = FAKE, tws.SSM_F32, 8
    a.m, a.k, a.ldx = 16, 64, 64
    a.norm_eps = 1e-5
    a.w_packed, a.w_scale, a.n_out, a.group_size = FAKE, FAKE, 32, 0
    a.y, a.y_dtype, a.ldy = FAKE, tws.SSM_F32, 32
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(act_bits=4), UNSUPPORTED),
    (dict(x_dtype=7), DTYPE),
    (dict(x_dtype=tws.SSM_I8, act_bits=16), DTYPE),
    (dict(y_dtype=tws.SSM_I8), DTYPE),
    (dict(k=0), SHAPE),
    (dict(k=5000, ldx=5000), SHAPE),
    (dict(m=-1), SHAPE),
    (dict(n_out=0), SHAPE),
    (dict(ldx=32), SHAPE),
    (dict(ldy=8), SHAPE),
    (dict(group_size=32), SHAPE),
    (dict(group_size=128), SHAPE),
    (dict(w_packed=None), NULL),
    (dict(w_scale=None), NULL),
    (dict(x=None), NULL),
    (dict(y=None), NULL),
    (dict(w_packed=FAKE + 2), ALIGN),
    (dict(act_bits=16, dbg_acc=FAKE), UNSUPPORTED),
    (dict(x_dtype=tws.SSM_I8), NULL),
    (dict(x_dtype=tws.SSM_I8, x_absmax=FAKE, k=40, ldx=64), UNSUPPORTED),
])
def test_bitlinear_rejects(kw, status):
    L = tws.lib()
    a = _bl(**kw)
    assert L.ssm_bitlinear_fwd(ctypes.byref(a), None, 0, None) == status
    assert L.ssm_last_error().decode()


def test_bitlinear_workspace_checks():
    L = tws.lib()
    # k <= 1024, A8, one scale: the row-block kernel needs no workspace
    assert L.ssm_bitlinear_workspace_bytes(ctypes.byref(_bl())) == 0
    # k > 1024: normalised int8 rows and absmax go through the workspace
    a = _bl(k=2048, ldx=2048)
    need = L.ssm_bitlinear_workspace_bytes(ctypes.byref(a))
    assert need >= 16 * 2048 + 16 * 4
    assert L.ssm_bitlinear_fwd(ctypes.byref(a), None, 0, None) == WORKSPACE
    assert L.ssm_bitlinear_fwd(ctypes.byref(a), FAKE, need - 1, None) == WORKSPACE
    assert L.ssm_bitlinear_workspace_bytes(ctypes.byref(_bl(k=0))) == 0


def _scan(**kw):
    a = tws.ScanArgs()
    a.batch, a.seqlen, a.nheads, a.headdim, a.d_state = 2, 64, 128, 1, 16
    a.a_per_state, a.act_dtype = 1, tws.SSM_F32
    a.x, a.ld_x, a.delta, a.ld_delta = FAKE, 128, FAKE, 128
    a.A, a.Bm, a.ld_B, a.Cm, a.ld_C = FAKE, FAKE, 16, FAKE, 16
    a.y, a.ld_y = FAKE, 128
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(d_state=12), UNSUPPORTED),
    (dict(headdim=2, ld_x=256, ld_y=256), UNSUPPORTED),
    (dict(a_per_state=0, d_state=8), UNSUPPORTED),
    (dict(a_per_state=2), SHAPE),
    (dict(act_dtype=tws.SSM_I8), DTYPE),
    (dict(ld_x=100), SHAPE),
    (dict(ld_B=8), SHAPE),
    (dict(nheads=0), SHAPE),
    (dict(batch=-1), SHAPE),
    (dict(x=None), NULL),
    (dict(A=None), NULL),
    (dict(Cm=None), NULL),
    # one sequence spanning 2 GiB of a tensor (the Mamba-1 kind kernels use 32-bit offsets)
    (dict(seqlen=1 << 22, ld_x=128), UNSUPPORTED),
    (dict(seqlen=1 << 17, ld_B=4096, ld_C=4096), UNSUPPORTED),
])
def test_scan_rejects(kw, status):
    L = tws.lib()
    a = _scan(**kw)
    assert L.ssm_selective_scan_fwd(ctypes.byref(a), None, 0, None) == status


def test_scan_empty_is_noop():
    """batch 0 or L 0: validated, nothing launched (no device needed)."""
    L = tws.lib()
    for kw in (dict(batch=0), dict(seqlen=0)):
        a = _scan(x=None, delta=None, A=None, Bm=None, Cm=None, y=None, **kw)
        assert L.ssm_selective_scan_fwd(ctypes.byref(a), None, 0, None) == OK


def test_quantize_rejects():
    L = tws.lib()
    q = L.ssm_ternary_quantize_weights
    assert q(None, 4, 16, 0, None, FAKE, FAKE, None, None, 0, None) == NULL
    assert q(FAKE, 0, 16, 0, None, FAKE, FAKE, None, None, 0, None) == SHAPE
    assert q(FAKE, 4, 100, 64, None, FAKE, FAKE, None, None, 0, None) == SHAPE
    assert q(FAKE, 4, 16, 0, None, FAKE + 1, FAKE, None, None, 0, None) == ALIGN
    assert q(FAKE, 4, 16, 0, None, FAKE, FAKE, None, None, 0, None) == WORKSPACE
    assert L.ssm_ternary_quantize_workspace_bytes(4, 256, 128, None) == 4 * 2 * 8
    assert L.ssm_ternary_quantize_workspace_bytes(4, 256, 0, None) == 4 * 8
    assert L.ssm_ternary_quantize_workspace_bytes(4, 256, 0, FAKE) == 0


def test_mixer_rejects():
    L = tws.lib()
    w = tws.MixerWeights()
    for name, _ in tws.MixerWeights._fields_:
        setattr(w, name, FAKE)
    good = tws.mixer_config(0, 64, 128, 16, dt_rank=8)
    assert L.ssm_mixer_workspace_bytes(ctypes.byref(good), 2, 64) > 0
    cases = [
        (tws.mixer_config(0, 64, 128, 16, dt_rank=8, act_bits=16), UNSUPPORTED),
        (tws.mixer_config(0, 64, 128, 16, dt_rank=0), UNSUPPORTED),
        (tws.mixer_config(0, 64, 128, 16, dt_rank=80), UNSUPPORTED),
        (tws.mixer_config(0, 64, 128, 12, dt_rank=8), UNSUPPORTED),
        (tws.mixer_config(1, 64, 128, 16, nheads=3, headdim=64), SHAPE),
        (tws.mixer_config(1, 64, 128, 16, nheads=2, headdim=64, group_size=100), SHAPE),
        (tws.mixer_config(0, 8192, 128, 16, dt_rank=8), SHAPE),
        (tws.mixer_config(5, 64, 128, 16), UNSUPPORTED),
        (tws.mixer_config(0, 64, 128, 16, dt_rank=8, gated=1, d_conv=0), SHAPE),
        (tws.mixer_config(0, 64, 128, 16, dt_rank=8, gated=1, d_conv=9), SHAPE),
        (tws.mixer_config(0, 64, 128, 16, dt_rank=8, gated=0, d_conv=4), SHAPE),
        (tws.mixer_config(0, 64, 128, 16, dt_rank=8, gated=2, d_conv=4), SHAPE),
    ]
    for cfg, status in cases:
        assert L.ssm_mixer_fwd(ctypes.byref(cfg), ctypes.byref(w), FAKE, FAKE + 4096, 2, 64, 1, FAKE, 1 << 30,
                               None) == status
    # missing weights, in-place without residual, too-small workspace
    w2 = tws.MixerWeights()
    assert L.ssm_mixer_fwd(ctypes.byref(good), ctypes.byref(w2), FAKE, FAKE, 2, 64, 1, FAKE, 1 << 30, None) == NULL
    assert L.ssm_mixer_fwd(ctypes.byref(good), ctypes.byref(w), FAKE, FAKE, 2, 64, 0, FAKE, 1 << 30, None) == SHAPE
    assert L.ssm_mixer_fwd(ctypes.byref(good), ctypes.byref(w), FAKE, FAKE + 4096, 2, 64, 1, FAKE, 16, None) == WORKSPACE
    assert L.ssm_mixer_fwd(ctypes.byref(good), ctypes.byref(w), FAKE, FAKE + 4096, 2, 64, 1, FAKE + 8, 1 << 30,
                           None) == ALIGN


def test_mixer_step_rejects():
    L = tws.lib()
    w = tws.MixerWeights()
    for name, _ in tws.MixerWeights._fields_:
        setattr(w, name, FAKE)
    good = tws.mixer_config(0, 64, 128, 16, dt_rank=8)
    step = L.ssm_mixer_step
    assert step(ctypes.byref(good), ctypes.byref(w), FAKE, FAKE + 4096, 2, None, None, 1, FAKE, 1 << 30,
                None) == NULL
    assert step(ctypes.byref(tws.mixer_config(0, 64, 128, 16, dt_rank=0)), ctypes.byref(w), FAKE, FAKE + 4096, 2,
                FAKE + 8192, None, 1, FAKE, 1 << 30, None) == UNSUPPORTED
    assert step(ctypes.byref(good), ctypes.byref(w), FAKE, FAKE + 4096, 2, FAKE + 8192, None, 1, FAKE, 16,
                None) == WORKSPACE
    assert step(ctypes.byref(good), ctypes.byref(w), FAKE, FAKE, 2, FAKE + 8192, None, 0, FAKE, 1 << 30,
                None) == SHAPE
    gated = tws.mixer_config(0, 64, 128, 16, dt_rank=8, gated=1, d_conv=4)
    assert step(ctypes.byref(gated), ctypes.byref(w), FAKE, FAKE + 4096, 2, FAKE + 8192, None, 1, FAKE, 1 << 30,
                None) == NULL  # the convolution's state is required


def test_mixer_stack_step_rejects():
    L = tws.lib()
    w = tws.MixerWeights()
    for name, _ in tws.MixerWeights._fields_:
        setattr(w, name, FAKE)
    good = tws.mixer_config(0, 64, 128, 16, dt_rank=8)
    nb = L.ssm_mixer_stack_workspace_bytes(ctypes.byref(good), 2)
    assert nb >= L.ssm_mixer_workspace_bytes(ctypes.byref(good), 2, 1) + 2 * 2 * 64 * 4
    ws = (ctypes.POINTER(tws.MixerWeights) * 2)(ctypes.pointer(w), ctypes.pointer(w))
    st = (ctypes.c_void_p * 2)(FAKE + 8192, FAKE + 16384)
    step = L.ssm_mixer_stack_step
    assert step(ctypes.byref(good), ws, 0, FAKE, FAKE + 4096, 2, st, None, 1, FAKE, nb, None) == SHAPE
    assert step(ctypes.byref(good), None, 2, FAKE, FAKE + 4096, 2, st, None, 1, FAKE, nb, None) == NULL
    assert step(ctypes.byref(good), ws, 2, FAKE, FAKE + 4096, 2, None, None, 1, FAKE, nb, None) == NULL
    assert step(ctypes.byref(good), ws, 2, FAKE, FAKE + 4096, 2, st, None, 1, FAKE, nb - 1, None) == WORKSPACE
    assert step(ctypes.byref(good), ws, 2, FAKE, FAKE + 4096, 2, st, None, 1, FAKE + 8, nb, None) == ALIGN
    assert step(ctypes.byref(good), ws, 2, FAKE, FAKE, 2, st, None, 0, FAKE, nb, None) == SHAPE
    bad = tws.mixer_config(0, 64, 128, 16, dt_rank=0)
    assert step(ctypes.byref(bad), ws, 2, FAKE, FAKE + 4096, 2, st, None, 1, FAKE, nb, None) == UNSUPPORTED
    assert L.ssm_mixer_stack_workspace_bytes(ctypes.byref(bad), 2) == 0
    # nothing to do for an empty batch
    assert step(ctypes.byref(good), ws, 2, None, None, 0, st, None, 1, FAKE, nb, None) == 0


def test_mixer_gated_needs_conv_weights_and_room():
    L = tws.lib()
    w = tws.MixerWeights()
    for name, _ in tws.MixerWeights._fields_:
        setattr(w, name, FAKE)
    w.conv_w = None
    gated = tws.mixer_config(0, 64, 128, 16, dt_rank=8, gated=1, d_conv=4)
    plain = tws.mixer_config(0, 64, 128, 16, dt_rank=8)
    assert L.ssm_mixer_fwd(ctypes.byref(gated), ctypes.byref(w), FAKE, FAKE + 4096, 2, 64, 1, FAKE, 1 << 30,
                           None) == NULL
    # the gate branch and the convolved copy need room beyond the plain mixer's workspace
    assert L.ssm_mixer_workspace_bytes(ctypes.byref(gated), 2, 64) > L.ssm_mixer_workspace_bytes(ctypes.byref(plain), 2, 64)
    assert L.ssm_mixer_fuses_front(ctypes.byref(tws.mixer_config(0, 256, 512, 16, dt_rank=16, gated=1, d_conv=4))) == 0


def test_dense_rejects():
    L = tws.lib()
    d = L.ssm_dense_fwd
    assert d(FAKE, 7, 4, 16, 16, FAKE, 8, None, 0, FAKE + 4096, 8, None) == DTYPE
    assert d(FAKE, 0, 4, 0, 16, FAKE, 8, None, 0, FAKE + 4096, 8, None) == SHAPE
    assert d(FAKE, 0, 4, 16, 8, FAKE, 8, None, 0, FAKE + 4096, 8, None) == SHAPE
    assert d(FAKE, 0, 4, 16, 16, FAKE, 8, None, 0, FAKE + 4096, 4, None) == SHAPE
    assert d(FAKE, 0, 4, 16, 16, FAKE, 8, FAKE + 8192, 4, FAKE + 4096, 8, None) == SHAPE
    assert d(FAKE, 0, 1 << 31, 16, 16, FAKE, 8, None, 0, FAKE + 4096, 8, None) == SHAPE
    assert d(FAKE, 0, 4, 16, 16, None, 8, None, 0, FAKE + 4096, 8, None) == NULL
    assert d(FAKE, 0, 4, 16, 16, FAKE, 8, None, 0, FAKE, 16, None) == SHAPE


def test_mixer_fp_proj_rejects():
    L = tws.lib()
    w = tws.MixerWeights()
    for name, _ in tws.MixerWeights._fields_:
        setattr(w, name, FAKE)
    bad = tws.mixer_config(0, 64, 128, 16, dt_rank=8, fp_proj=3)
    assert L.ssm_mixer_fwd(ctypes.byref(bad), ctypes.byref(w), FAKE, FAKE + 4096, 2, 64, 1, FAKE, 1 << 30,
                           None) == SHAPE
    for mode, missing in ((1, "fw_in"), (1, "fw_out"), (2, "fw_x"), (2, "fw_dt")):
        w2 = tws.MixerWeights()
        for name, _ in tws.MixerWeights._fields_:
            setattr(w2, name, FAKE)
        setattr(w2, missing, None)
        c = tws.mixer_config(0, 64, 128, 16, dt_rank=8, fp_proj=mode)
        assert L.ssm_mixer_fwd(ctypes.byref(c), ctypes.byref(w2), FAKE, FAKE + 4096, 2, 64, 1, FAKE, 1 << 30,
                               None) == NULL, (mode, missing)
    # ternary weights are not needed where the projections are full precision
    w3 = tws.MixerWeights()
    for name in ("fw_in", "fw_out", "fw_x", "fw_dt", "A"):
        setattr(w3, name, FAKE)
    c = tws.mixer_config(0, 64, 128, 16, dt_rank=8, fp_proj=2)
    assert L.ssm_mixer_fwd(ctypes.byref(c), ctypes.byref(w3), FAKE, FAKE + 4096, 2, 64, 1, FAKE, 16,
                           None) == WORKSPACE
    assert L.ssm_mixer_fuses_front(ctypes.byref(tws.mixer_config(0, 256, 512, 16, dt_rank=16, fp_proj=1))) == 0


def test_bitlinear_bwd_and_qat_rejects():
    L = tws.lib()
    a = tws.BitlinearBwdArgs()
    a.x, a.x_dtype, a.m, a.k, a.ldx = FAKE, 0, 4, 64, 64
    a.w_packed, a.w_scale, a.n_out = FAKE, FAKE, 32
    a.dy, a.ld_dy, a.dx, a.ld_dx = FAKE, 32, FAKE, 64
    assert L.ssm_bitlinear_bwd(None, FAKE, 1 << 20, None) == NULL
    assert L.ssm_bitlinear_bwd_workspace_bytes(ctypes.byref(a)) > 0
    assert L.ssm_bitlinear_bwd(ctypes.byref(a), FAKE, 16, None) == WORKSPACE
    for field, val, status in (("x_dtype", 2, DTYPE), ("k", 0, SHAPE), ("ld_dy", 16, SHAPE), ("ld_dx", 8, SHAPE),
                               ("group_size", 100, SHAPE), ("w_packed", None, NULL), ("dy", None, NULL),
                               ("w_packed", FAKE + 2, ALIGN)):
        b = tws.BitlinearBwdArgs.from_buffer_copy(a)
        setattr(b, field, val)
        assert L.ssm_bitlinear_bwd(ctypes.byref(b), FAKE, 1 << 30, None) == status, field
    for field in ("ldx", "ld_dy", "ld_dx"):  # a 32-row tile must stay within 32-bit offsets
        b = tws.BitlinearBwdArgs.from_buffer_copy(a)
        setattr(b, field, ((1 << 31) - 1) // 33 + 1)
        assert L.ssm_bitlinear_bwd_workspace_bytes(ctypes.byref(b)) == 0, field
        assert L.ssm_bitlinear_bwd(ctypes.byref(b), FAKE, 1 << 30, None) == UNSUPPORTED, field
    b = tws.BitlinearBwdArgs.from_buffer_copy(a)
    b.d_scale = FAKE  # needs dw and w_latent
    assert L.ssm_bitlinear_bwd(ctypes.byref(b), FAKE, 1 << 30, None) == NULL
    q = L.ssm_qat_sgd_step
    assert q(None, FAKE, FAKE, None, 4, 64, 0, 0.1, 0.1, FAKE, None, None, 0, None) == NULL
    assert q(FAKE, FAKE, FAKE, None, 4, 64, 100, 0.1, 0.1, FAKE, None, None, 0, None) == SHAPE
    assert q(FAKE, FAKE, FAKE, None, 0, 64, 0, 0.1, 0.1, FAKE, None, None, 0, None) == SHAPE


def test_scan_bwd_rejects():
    L = tws.lib()
    a = tws.ScanBwdArgs()
    a.batch, a.seqlen, a.nheads, a.d_state, a.act_dtype, a.delta_softplus = 2, 8, 64, 16, 0, 1
    for f in ("x", "delta", "A", "Bm", "Cm", "dy", "dx", "ddelta", "dA", "dB", "dC"):
        setattr(a, f, FAKE)
    a.ld_x = a.ld_delta = a.ld_dy = 64
    a.ld_B = a.ld_C = 16
    assert L.ssm_selective_scan_bwd(None, FAKE, 1 << 30, None) == NULL
    # states and adjoint carries at the chunk boundaries (one chunk of 16 steps here), partial sums
    assert L.ssm_selective_scan_bwd_workspace_bytes(ctypes.byref(a)) >= 2 * (2 * 1 * 64 * 16 * 4) + 2 * 16 * 16 * 4
    assert L.ssm_selective_scan_bwd(ctypes.byref(a), FAKE, 16, None) == WORKSPACE
    assert L.ssm_selective_scan_bwd(ctypes.byref(a), FAKE + 8, 1 << 30, None) == ALIGN
    for field, val, status in (("d_state", 12, UNSUPPORTED), ("act_dtype", 2, DTYPE), ("ld_B", 8, SHAPE),
                               ("ld_dy", 32, SHAPE), ("nheads", 0, SHAPE), ("dB", None, NULL), ("A", FAKE + 2, ALIGN),
                               ("seqlen", 65535 * 16 + 1, UNSUPPORTED)):  # more than 65535 time chunks
        b = tws.ScanBwdArgs.from_buffer_copy(a)
        setattr(b, field, val)
        assert L.ssm_selective_scan_bwd(ctypes.byref(b), FAKE, 1 << 30, None) == status, field


def test_mixer_bwd_rejects():
    L = tws.lib()
    w = tws.MixerWeights()
    for name, _ in tws.MixerWeights._fields_:
        setattr(w, name, FAKE)
    g = tws.MixerGrads()
    good = tws.mixer_config(0, 64, 128, 16, dt_rank=8)
    need = L.ssm_mixer_bwd_workspace_bytes(ctypes.byref(good), 2, 64)
    assert need >= L.ssm_mixer_workspace_bytes(ctypes.byref(good), 2, 64)
    bwd = L.ssm_mixer_bwd
    U, DOUT, DU, WS = FAKE, FAKE + 4096, FAKE + 8192, FAKE + 65536
    for cfg in (tws.mixer_config(1, 64, 128, 16, nheads=2, headdim=64),
                tws.mixer_config(0, 64, 128, 16, dt_rank=8, gated=1, d_conv=4),
                tws.mixer_config(0, 64, 128, 16, dt_rank=8, fp_proj=1),
                tws.mixer_config(0, 64, 128, 16, dt_rank=8, act_dtype=torch.bfloat16),
                tws.mixer_config(0, 64, 128, 12, dt_rank=8)):
        assert L.ssm_mixer_bwd_workspace_bytes(ctypes.byref(cfg), 2, 64) == 0
        assert bwd(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(g), U, DOUT, DU, 2, 64, 1, WS, 1 << 30,
                   None) == UNSUPPORTED
    # more time chunks than the scan backward takes
    assert L.ssm_mixer_bwd_workspace_bytes(ctypes.byref(good), 1, 65535 * 16 + 1) == 0
    assert bwd(ctypes.byref(good), ctypes.byref(w), ctypes.byref(g), U, DOUT, DU, 1, 65535 * 16 + 1, 1, WS, 1 << 40,
               None) == UNSUPPORTED
    assert bwd(ctypes.byref(good), ctypes.byref(tws.MixerWeights()), ctypes.byref(g), U, DOUT, DU, 2, 64, 1, WS,
               1 << 30, None) == NULL
    g2 = tws.MixerGrads()
    g2.ds_in, g2.dw_in = FAKE, FAKE  # a scale gradient without the latent weights
    assert bwd(ctypes.byref(good), ctypes.byref(w), ctypes.byref(g2), U, DOUT, DU, 2, 64, 1, WS, 1 << 30,
               None) == NULL
    assert bwd(ctypes.byref(good), ctypes.byref(w), ctypes.byref(g), U, DOUT, None, 2, 64, 1, WS, 1 << 30,
               None) == NULL
    assert bwd(ctypes.byref(good), ctypes.byref(w), ctypes.byref(g), U, DOUT, U, 2, 64, 1, WS, 1 << 30,
               None) == SHAPE
    assert bwd(ctypes.byref(good), ctypes.byref(w), ctypes.byref(g), U, DOUT, DU, 2, 64, 1, WS, need - 1,
               None) == WORKSPACE
    assert bwd(ctypes.byref(good), ctypes.byref(w), ctypes.byref(g), U, DOUT, DU, 2, 64, 1, WS + 64, 1 << 30,
               None) == ALIGN
    # nothing to do for an empty batch, once the workspace is there
    assert bwd(ctypes.byref(good), ctypes.byref(w), ctypes.byref(g), None, None, None, 0, 64, 1, WS, 1 << 30,
               None) == OK


def test_conv_rejects():
    L = tws.lib()
    c = L.ssm_conv1d_silu_fwd
    assert c(FAKE, 5, 2, 8, 16, 16, FAKE, 4, None, None, None, FAKE + 4096, 16, None) == DTYPE
    assert c(FAKE, 0, 2, 8, 16, 16, FAKE, 0, None, None, None, FAKE + 4096, 16, None) == SHAPE
    assert c(FAKE, 0, 2, 8, 16, 16, FAKE, 9, None, None, None, FAKE + 4096, 16, None) == SHAPE
    assert c(FAKE, 0, 2, 8, 16, 8, FAKE, 4, None, None, None, FAKE + 4096, 16, None) == SHAPE
    assert c(FAKE, 0, 2, 8, 16, 16, FAKE, 4, None, None, None, FAKE + 4096, 8, None) == SHAPE
    assert c(FAKE, 0, 2, 8, 16, 16, None, 4, None, None, None, FAKE + 4096, 16, None) == NULL
    assert c(FAKE, 0, 2, 8, 16, 16, FAKE, 4, None, None, None, FAKE, 16, None) == SHAPE
    assert c(FAKE, 0, -1, 8, 16, 16, FAKE, 4, None, None, None, FAKE + 4096, 16, None) == SHAPE


def test_mixer_fuses_front_query():
    """Host-only query: which Mamba-1 shapes run in_proj, x_proj and the dt quantisation fused."""
    L = tws.lib()
    trissm = tws.mixer_config(0, 256, 512, 16, dt_rank=16)
    assert L.ssm_mixer_fuses_front(ctypes.byref(trissm)) == 1
    assert L.ssm_mixer_fuses_front(ctypes.byref(tws.mixer_config(0, 512, 1024, 16, dt_rank=32))) == 0
    assert L.ssm_mixer_fuses_front(ctypes.byref(tws.mixer_config(1, 256, 256, 64, nheads=4, headdim=64))) == 0
    assert L.ssm_mixer_fuses_front(ctypes.byref(tws.mixer_config(0, 100, 512, 16, dt_rank=16))) == 0
    assert L.ssm_mixer_fuses_front(None) == 0


def test_mixer_fuses_front_whole_range():
    """The fused front covers d_model in {64, 128, 256, 512} x d_inner in {128, 256, 512, 1024}
    except 512 x 1024, with x_proj at most 64 wide; nothing else."""
    L = tws.lib()
    for dm in (32, 64, 96, 128, 256, 384, 512, 1024):
        for di in (64, 128, 256, 384, 512, 1024, 2048):
            c = tws.mixer_config(0, dm, di, 16, dt_rank=16)
            want = dm in (64, 128, 256, 512) and di in (128, 256, 512, 1024) and not (dm == 512 and di == 1024)
            assert L.ssm_mixer_fuses_front(ctypes.byref(c)) == int(want), (dm, di)
    # x_proj width dt_rank + 2 d_state at most 64; dt_rank within [1, 64]
    assert L.ssm_mixer_fuses_front(ctypes.byref(tws.mixer_config(0, 256, 512, 16, dt_rank=32))) == 1
    assert L.ssm_mixer_fuses_front(ctypes.byref(tws.mixer_config(0, 256, 512, 32, dt_rank=16))) == 0
    assert L.ssm_mixer_fuses_front(ctypes.byref(tws.mixer_config(0, 256, 512, 16, dt_rank=33))) == 0
    # the gated block and full-precision projections never take the fused front
    assert L.ssm_mixer_fuses_front(ctypes.byref(tws.mixer_config(0, 256, 512, 16, dt_rank=16, gated=1,
                                                                 d_conv=4))) == 0


def test_last_error_is_thread_local():
    """Each thread sees the detail of its own last failing call, not another thread's."""
    import threading
    L = tws.lib()
    barrier = threading.Barrier(2)
    seen = {}

    def worker(name, call):
        assert call() != OK
        barrier.wait()  # both threads have failed before either reads its text
        seen[name] = L.ssm_last_error().decode()
        barrier.wait()

    t1 = threading.Thread(target=worker, args=("scan", lambda: L.ssm_selective_scan_fwd(None, FAKE, 1 << 20, None)))
    t2 = threading.Thread(target=worker, args=("quant", lambda: L.ssm_ternary_quantize_weights(
        FAKE, 4, 6, 4, None, FAKE, FAKE, None, FAKE, 1 << 20, None)))
    t1.start(); t2.start(); t1.join(); t2.join()
    assert "scan" in seen["scan"] and "quantize" not in seen["scan"], seen
    assert "quantize" in seen["quant"], seen
    assert seen["scan"] != seen["quant"]
