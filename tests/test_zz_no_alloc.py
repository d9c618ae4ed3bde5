"""The scan entry point that allocates nothing (ssm_selective_scan_fwd_noalloc, for callers that
cannot allocate): the same results as ssm_selective_scan_fwd with a caller workspace, bit for
bit, on two calls in a row (the second smaller, reusing the library's scratch array), for the
shapes whose scratch holds chunk carries or segment states; and a shape beyond the scratch
size is rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import ternary_weight_selective_amd as tws
import workloads as wl
from gpu_helpers import host, to_dev

pytestmark = pytest.mark.gpu


def _args(p, dt, dt_proj=None):
    return (to_dev(p["x"], dt), None if dt_proj else to_dev(p["delta"], dt), to_dev(p["A"]), to_dev(p["Bm"], dt),
            to_dev(p["Cm"], dt), to_dev(p["D"]), to_dev(p["dt_bias"]), True)


def _both(p, dt, **kw):
    a = _args(p, dt, kw.get("dt_proj"))
    ref = tws.ssm_selective_scan_fwd(*a, return_last_state=True, **kw)
    got = tws.ssm_selective_scan_fwd(*a, return_last_state=True, noalloc=True, **kw)
    return [host(t) for t in ref], [host(t) for t in got]


@pytest.mark.parametrize("shapes,P,N,aps,dt", [
    # Mamba-1 kind: few sequences and channels, long L: time chunks with carries in the scratch
    (((2, 2048, 128), (1, 1000, 64)), 1, 16, True, torch.float32),
    # SSD kind on the matrix cores: time segments with their states in the scratch
    (((2, 1024, 4), (1, 300, 2)), 64, 128, False, torch.bfloat16),
])
def test_noalloc_scan_matches_workspace_scan(shapes, P, N, aps, dt):
    for i, (B, L, H) in enumerate(shapes):  # the second call is smaller
        p = wl.scan_problem(B, L, H, P, N, aps, seed=70 + i)
        (y, hl), (y2, hl2) = _both(p, dt)
        np.testing.assert_array_equal(y2, y)
        np.testing.assert_array_equal(hl2, hl)


def test_noalloc_scan_fused_dt_projection():
    """The dt projection computed inside the scan: its input's codes live in the scratch too."""
    cfg = wl.CONFIGS["trissm"]
    lat, _ = wl.mixer_problem(cfg, seed=3, layers=1)
    packed, scale, _ = tws.ssm_ternary_quantize_weights(to_dev(lat[0]["W_dt"]))
    for i, (B, L) in enumerate(((4, 512), (2, 100))):
        p = wl.scan_problem(B, L, cfg.d_inner, 1, cfg.d_state, True, seed=80 + i)
        dr = to_dev(wl.normal(wl.rng(81 + i), (B, L, cfg.dt_rank)))
        (y, hl), (y2, hl2) = _both(p, torch.float32, dt_proj=dict(dt_in=dr, w_dt=packed, s_dt=scale,
                                                                    dt_rank=cfg.dt_rank))
        np.testing.assert_array_equal(y2, y)
        np.testing.assert_array_equal(hl2, hl)


def test_noalloc_scan_rejects_beyond_scratch():
    """A scan needing more scratch than the library holds fails on the host, launching nothing."""
    a = tws.ScanArgs()
    F = 0x100000
    # the dt input's codes of 2^21 tokens alone take 48 MB
    a.batch, a.seqlen, a.nheads, a.headdim, a.d_state = 1, 1 << 21, 64, 1, 16
    a.a_per_state, a.act_dtype = 1, 0
    a.x, a.ld_x, a.A, a.Bm, a.ld_B, a.Cm, a.ld_C, a.y, a.ld_y = F, 64, F, F, 48, F, 48, F, 64
    a.dt_in, a.ld_dt_in, a.dt_rank, a.w_dt, a.s_dt = F, 48, 16, F, F
    L = tws.lib()
    assert L.ssm_selective_scan_workspace_bytes(ctypes.byref(a)) > 32 << 20
    assert L.ssm_selective_scan_fwd_noalloc(ctypes.byref(a), None) == 6
    assert b"noalloc" in L.ssm_last_error()
