"""GPU parity: the HIP path against the CPU oracle, element by element, through the C ABI.

Integer stages (packed weights, scales, int8 activations, absmax, int32 accumulators) are
bit-exact and checked stage-wise: the GPU stage is fed the oracle's exact stage input.
Float outputs: norm-wise relative error <= 1e-4 (fp32) or <= 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_selective_amd as tws
import workloads as wl
from gpu_helpers import (DEV, TOL, bf16_values, chain, check, gpu_config, host, oracle_config, quantize_layer,
                         rel_err, run_gpu_stack, to_dev, torch_dtype)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ S0: ternarise + pack

PROJ_SHAPES = sorted({(n, k, c.group_size) for c in wl.CONFIGS.values() for (n, k) in c.proj_shapes.values()})


@pytest.mark.parametrize("n,k,group", PROJ_SHAPES)
def test_pack_bit_exact_config_shapes(n, k, group):
    """Every projection shape of the five workloads: packed bytes, scales, zero count bit-exact."""
    w = wl.normal(wl.rng(n * 7 + k), (n, k), 0.0, 0.02)
    packed, scale, zc = tws.ssm_ternary_quantize_weights(to_dev(w), group)
    codes, oscale, zeros = oracle.quantize_weights(w, group)
    np.testing.assert_array_equal(host(packed), oracle.pack(codes))
    np.testing.assert_array_equal(host(scale).ravel(), np.asarray(oscale).ravel())
    assert int(host(zc)[0]) == zeros


@pytest.mark.parametrize("n,k,group", [(1, 1, 0), (3, 7, 0), (5, 40, 0), (33, 200, 0), (17, 384, 128), (2, 4096, 64)])
def test_pack_ragged_and_edges(n, k, group):
    """Ragged rows (k not a multiple of 16), single weights, grouped scales, exact ties."""
    g = wl.rng(k)
    w = wl.normal(g, (n, k), 0.0, 0.02)
    w[0, : min(k, 4)] = np.array([1.0, -0.5, 0.25, 0.25], np.float32)[: min(k, 4)]
    packed, scale, zc = tws.ssm_ternary_quantize_weights(to_dev(w), group)
    codes, oscale, zeros = oracle.quantize_weights(w, group)
    np.testing.assert_array_equal(host(packed), oracle.pack(codes))
    np.testing.assert_array_equal(host(scale).ravel(), np.asarray(oscale).ravel())
    assert int(host(zc)[0]) == zeros


def test_pack_zero_tensor_and_caller_scale():
    w = np.zeros((8, 64), np.float32)
    packed, scale, zc = tws.ssm_ternary_quantize_weights(to_dev(w))
    assert not host(packed).any() and host(scale)[0] == 0.0 and int(host(zc)[0]) == 8 * 64
    w = wl.normal(wl.rng(5), (16, 128), 0.0, 0.02)
    s_in = np.array([0.013], np.float32)
    packed, scale, _ = tws.ssm_ternary_quantize_weights(to_dev(w), 0, scale_in=to_dev(s_in))
    codes, _, _ = oracle.quantize_weights(w, 0, scale_in=s_in)
    np.testing.assert_array_equal(host(packed), oracle.pack(codes))
    assert host(scale)[0] == s_in[0]


# ------------------------------------------------------------------ S1-S4: BitLinear

BL_CASES = [  # (m, k, n, group, act_bits, x dtype, y dtype)
    (128, 64, 128, 0, 8, "f32", "f32"),      # bitssm_tiny in_proj
    (130, 128, 40, 0, 8, "f32", "f32"),      # x_proj, ragged m
    (67, 8, 128, 0, 8, "f32", "f32"),        # dt_proj, k = 8
    (1000, 256, 512, 0, 8, "f32", "f32"),    # trissm in_proj rows
    (515, 512, 48, 0, 8, "f32", "f32"),      # trissm x_proj
    (333, 16, 512, 0, 8, "f32", "f32"),      # trissm dt_proj
    (260, 1024, 512, 0, 8, "bf16", "bf16"),  # ternaryssm50m out_proj
    (129, 32, 1024, 0, 8, "bf16", "bf16"),   # ternaryssm50m dt_proj
    (200, 512, 256, 128, 8, "f32", "f32"),   # grouped A8
    (97, 2048, 300, 128, 16, "bf16", "bf16"),  # mamba2_ssd in_proj rows, N ragged
    (64, 4096, 256, 128, 16, "bf16", "bf16"),  # mamba2_ssd out_proj rows
    (50, 256, 64, 0, 16, "f32", "f32"),      # A16 per tensor
    (130, 512, 200, 0, 16, "bf16", "bf16"),  # A16 per tensor, bf16 out (large-tile kernel), ragged m, n
    (33, 100, 70, 0, 16, "bf16", "bf16"),    # A16, k padded to 128
    (300, 2048, 4416, 128, 16, "f32", "bf16"),  # A16 grouped, Mamba-2 in_proj width, fp32 input
    (1, 100, 70, 0, 8, "f32", "f32"),        # one row, ragged k
    (100, 2048, 4416, 0, 8, "bf16", "bf16"),  # mamba2_a8 in_proj (tiled int8 path)
    (77, 4096, 2048, 0, 8, "bf16", "bf16"),   # mamba2_a8 out_proj
    (50, 1156, 130, 0, 8, "f32", "f32"),      # large-tile int8 path, odd k-step count, k % 16 != 0
]


@pytest.mark.parametrize("m,k,n,group,bits,xd,yd", BL_CASES)
def test_bitlinear_parity(m, k, n, group, bits, xd, yd):
    g = wl.rng(m + 3 * k + 7 * n)
    x = wl.normal(g, (m, k))
    if xd == "bf16":
        x = bf16_values(x)
    w = wl.normal(g, (n, k), 0.0, 0.02)
    bias = wl.normal(g, (n,), 0.0, 0.1)
    packed, scale, _ = tws.ssm_ternary_quantize_weights(to_dev(w), group)
    codes, oscale, _ = oracle.quantize_weights(w, group)
    xdt = torch.bfloat16 if xd == "bf16" else torch.float32
    ydt = torch.bfloat16 if yd == "bf16" else torch.float32
    xt = to_dev(x, xdt)
    ref, oxq, oam, oacc = oracle.bitlinear(x, codes, oscale, group, bits, bias=bias)
    if bits == 8:
        y, xq, am, acc = tws.ssm_bitlinear_fwd(xt, packed, scale, n, act_bits=bits, group_size=group,
                                               bias=to_dev(bias), y_dtype=ydt, debug=True)
        np.testing.assert_array_equal(host(xq), oxq)          # S2 int8 codes
        np.testing.assert_array_equal(host(am), oam)          # S2 absmax
        np.testing.assert_array_equal(host(acc), oacc)        # S3 int32 accumulators
        # S4: the fp64 dequantisation rounded once gives the oracle's stored value exactly
        stored = ref.astype(np.float32)
        np.testing.assert_array_equal(host(y), bf16_values(stored) if yd == "bf16" else stored)
    else:
        y = tws.ssm_bitlinear_fwd(xt, packed, scale, n, act_bits=bits, group_size=group, bias=to_dev(bias),
                                  y_dtype=ydt)
    check(host(y), ref, TOL[yd], what=f"test_bitlinear_parity {m} {k} {n} {group} {bits}")


@pytest.mark.parametrize("m,k,n", [(8192, 4096, 2048), (8192, 4096, 2000), (16384, 512, 1024), (8195, 1024, 1024)])
def test_bitlinear_big_tiles_sampled(m, k, n):
    """The large-tile int8 contraction at the Mamba-2 out_proj shape (8192 tokens, k = 4096), where
    two 128-wide output tiles share a compute unit (n = 2000 leaves a ragged last tile), and at the
    TernarySSM in_proj shape (16384 tokens, k = 512, n = 1024), which takes the norm kernel + the
    large-tile contraction instead of the row-block kernel; 8195 rows of k = 1024 leave a ragged
    last row tile.  Rows are independent (per-row norm
    and codes), so 96 sampled rows across the row tiles are checked against the oracle: codes,
    absmax and int32 sums bit for bit, outputs exactly."""
    g = wl.rng(n + 11)
    x = bf16_values(wl.normal(g, (m, k)))
    w = wl.normal(g, (n, k), 0.0, 0.02)
    packed, scale, _ = tws.ssm_ternary_quantize_weights(to_dev(w), 0)
    codes, oscale, _ = oracle.quantize_weights(w, 0)
    y, xq, am, acc = tws.ssm_bitlinear_fwd(to_dev(x, torch.bfloat16), packed, scale, n, y_dtype=torch.bfloat16,
                                           debug=True)
    rows = np.unique(np.concatenate([np.arange(0, m, m // 89), [m - 1, m - 2, 255, 256, 4095]]))
    ref, oxq, oam, oacc = oracle.bitlinear(x[rows], codes, oscale)
    np.testing.assert_array_equal(host(xq)[rows], oxq)
    np.testing.assert_array_equal(host(am)[rows], oam)
    np.testing.assert_array_equal(host(acc)[rows], oacc)
    np.testing.assert_array_equal(host(y)[rows], bf16_values(ref.astype(np.float32)))


@pytest.mark.parametrize("m,k,n", [(256, 256, 512), (77, 1024, 64), (64, 2048, 4416),
                                   (70, 1088, 200), (40, 64, 96), (300, 1216, 260)])  # odd k-step counts
def test_bitlinear_int32_from_oracle_codes(m, k, n):
    """Stage-wise S3: the GPU contraction fed the oracle's exact int8 codes and absmax."""
    g = wl.rng(k + n)
    x = wl.normal(g, (m, k))
    w = wl.normal(g, (n, k), 0.0, 0.02)
    codes, oscale, _ = oracle.quantize_weights(w, 0)
    ref, oxq, oam, oacc = oracle.bitlinear(x, codes, oscale)
    packed = to_dev(oracle.pack(codes), torch.uint8)
    y, _, _, acc = tws.ssm_bitlinear_fwd(to_dev(oxq, torch.int8), packed, to_dev(oscale), n,
                                         x_absmax=to_dev(oam), debug=True)
    np.testing.assert_array_equal(host(acc), oacc)
    check(host(y), ref, 1e-5, what="test_bitlinear_int32_from_oracle_codes")


def test_bitlinear_edge_rows():
    """All-zero token rows give bias only; a one-hot row quantises to a single 127; m = 0 is a no-op."""
    k, n = 256, 64
    x = wl.normal(wl.rng(1), (5, k))
    x[1] = 0.0
    x[3] = 0.0
    x[3, 17] = -3.5
    w = wl.normal(wl.rng(2), (n, k), 0.0, 0.02)
    bias = wl.normal(wl.rng(3), (n,))
    packed, scale, _ = tws.ssm_ternary_quantize_weights(to_dev(w))
    codes, oscale, _ = oracle.quantize_weights(w, 0)
    y, xq, am, acc = tws.ssm_bitlinear_fwd(to_dev(x), packed, scale, n, bias=to_dev(bias), debug=True)
    ref, oxq, oam, oacc = oracle.bitlinear(x, codes, oscale, bias=bias)
    np.testing.assert_array_equal(host(xq), oxq)
    np.testing.assert_array_equal(host(acc), oacc)
    yh = host(y)
    np.testing.assert_array_equal(yh[1], bias)
    assert host(xq)[3, 17] == -127
    check(yh, ref, 1e-4, what="test_bitlinear_edge_rows")
    empty = tws.ssm_bitlinear_fwd(torch.empty((0, k), device=DEV), packed, scale, n)
    assert empty.shape == (0, n)


def test_bitlinear_residual_and_strided_input():
    """A row stride wider than k (the dt input inside the x_proj output) and a residual add."""
    g = wl.rng(9)
    wide = wl.normal(g, (300, 48))
    w = wl.normal(g, (512, 16), 0.0, 0.02)
    res = wl.normal(g, (300, 512))
    packed, scale, _ = tws.ssm_ternary_quantize_weights(to_dev(w))
    codes, oscale, _ = oracle.quantize_weights(w, 0)
    xt = to_dev(wide)
    y = tws.ssm_bitlinear_fwd(xt[:, :16], packed, scale, 512, k=16, residual=to_dev(res))
    ref, *_ = oracle.bitlinear(wide, codes, oscale, k=16)
    check(host(y), ref + res, 1e-6, what="test_bitlinear_residual_and_strided_input")


# ------------------------------------------------------------------ S5-S8: selective scan

def _scan_gpu(p, dtype=torch.float32, h0=None, last=False):
    return tws.ssm_selective_scan_fwd(to_dev(p["x"], dtype), to_dev(p["delta"], dtype), to_dev(p["A"]),
                                      to_dev(p["Bm"], dtype), to_dev(p["Cm"], dtype), to_dev(p["D"]),
                                      to_dev(p["dt_bias"]), True, None if h0 is None else to_dev(h0),
                                      return_last_state=last)


def _bf16_problem(p):
    return {k: (bf16_values(v) if k in ("x", "delta", "Bm", "Cm") else v) for k, v in p.items()}


SCAN_CASES = [  # (batch, L, H, P, N, a_per_state, dtype)
    (2, 64, 128, 1, 16, True, "f32"),
    (3, 1, 512, 1, 16, True, "f32"),
    (2, 33, 100, 1, 16, True, "f32"),      # ragged channels and time tile
    (1, 300, 64, 1, 4, True, "f32"),
    (1, 97, 64, 1, 8, True, "f32"),
    (1, 70, 32, 1, 32, True, "f32"),
    (1, 70, 16, 1, 64, True, "f32"),
    (2, 100, 256, 1, 16, True, "bf16"),
    (2, 50, 4, 64, 128, False, "f32"),     # SSD kind
    (1, 77, 3, 16, 16, False, "f32"),
    (1, 40, 2, 32, 64, False, "bf16"),
    (2, 200, 4, 64, 128, False, "bf16"),   # SSD chunked (matrix-core) path, ragged last chunk
    (1, 130, 3, 64, 64, False, "bf16"),
]


@pytest.mark.parametrize("batch,L,H,P,N,aps,dt", SCAN_CASES)
def test_scan_parity(batch, L, H, P, N, aps, dt):
    p = wl.scan_problem(batch, L, H, P, N, aps, seed=L + H)
    if dt == "bf16":
        p = _bf16_problem(p)
    h0 = wl.normal(wl.rng(4), (batch, H, P, N), 0.0, 0.5)
    ref, href = oracle.selective_scan(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["D"], p["dt_bias"], h0=h0)
    y, hl = _scan_gpu(p, torch.bfloat16 if dt == "bf16" else torch.float32, h0=h0, last=True)
    check(host(y), ref, TOL[dt], what=f"test_scan_parity {batch} {L} {H} {P} {N} {dt}")
    # the SSD chunked path (bf16 activations) carries fp32 operands of its matrix products as
    # two bf16 terms (about 16 significant bits), hence the wider bound on its final state
    check(host(hl), href, (1e-4 if dt == "bf16" else 1e-5), what=f"test_scan_parity h_last {batch} {L} {H} {P} {N} {dt}")


def test_scan_ssd_dt_without_softplus():
    """SSD kind, bf16, a chunk-eligible shape, dt taken as given (no softplus, some dt < 0): the
    library routes it to the recurrent kernel (the chunked one splits decays in a way that needs
    dt >= 0) and matches the oracle."""
    p = _bf16_problem(wl.scan_problem(2, 130, 4, 64, 64, False, seed=21))
    p["dt_bias"] = np.full_like(p["dt_bias"], 0.05)  # dt = delta + 0.05 ~ N(0.05, 0.75): mixed signs
    p["A"] = p["A"] * 0.05  # keep exp(dt A) moderate for either sign of dt
    h0 = wl.normal(wl.rng(5), (2, 4, 64, 64), 0.0, 0.5)
    ref, href = oracle.selective_scan(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["D"], p["dt_bias"], h0=h0,
                                      softplus=False)
    y, hl = tws.ssm_selective_scan_fwd(to_dev(p["x"], torch.bfloat16), to_dev(p["delta"], torch.bfloat16),
                                       to_dev(p["A"]), to_dev(p["Bm"], torch.bfloat16),
                                       to_dev(p["Cm"], torch.bfloat16), to_dev(p["D"]), to_dev(p["dt_bias"]),
                                       False, to_dev(h0), return_last_state=True)
    check(host(y), ref, TOL["bf16"], what="test_scan_ssd_dt_without_softplus y")
    check(host(hl), href, 1e-4, what="test_scan_ssd_dt_without_softplus h_last")


def test_scan_long_sequence_sampled():
    """long_scan workload (batch 8, L 8192, 512 channels, d_state 16), full size on the GPU;
    the oracle checks 24 channels of every sequence (channels are independent)."""
    cfg = wl.CONFIGS["long_scan"]
    p = wl.scan_problem(cfg.batch, cfg.seqlen, cfg.d_inner, 1, cfg.d_state, True, seed=42)
    y, hl = _scan_gpu(p, last=True)
    yh, hh = host(y), host(hl)
    ch = np.array([0, 1, 63, 64, 100, 127, 128, 200, 255, 256, 300, 311, 383, 384, 400, 447, 448, 480, 500, 505,
                   509, 510, 511, 17])
    sub = dict(p, x=p["x"][:, :, ch], delta=p["delta"][:, :, ch], A=p["A"][ch], D=p["D"][ch],
               dt_bias=p["dt_bias"][ch])
    ref, href = oracle.selective_scan(sub["x"], sub["delta"], sub["A"], sub["Bm"], sub["Cm"], sub["D"],
                                      sub["dt_bias"])
    check(yh[:, :, ch], ref, 1e-4, what="test_scan_long_sequence_sampled")
    check(hh[:, ch], href, 1e-4, what="test_scan_long_sequence_sampled")


def test_scan_causality_determinism_streaming():
    """Perturbing token t leaves y before t bitwise unchanged; two runs are bitwise equal;
    a scan of L equals a scan of L1 then L - L1 from the carried state."""
    p = wl.scan_problem(2, 200, 256, 1, 16, True, seed=7)
    y1 = host(_scan_gpu(p))
    y2 = host(_scan_gpu(p))
    np.testing.assert_array_equal(y1, y2)
    q = {k: v.copy() for k, v in p.items()}
    q["x"][:, 120] += 1.0
    q["delta"][:, 120] -= 0.5
    y3 = host(_scan_gpu(q))
    np.testing.assert_array_equal(y3[:, :120], y1[:, :120])
    assert not np.array_equal(y3[:, 120], y1[:, 120])
    a = {k: (v[:, :77] if v.ndim == 3 else v) for k, v in p.items()}
    b = {k: (v[:, 77:] if v.ndim == 3 else v) for k, v in p.items()}
    ya, ha = _scan_gpu(a, last=True)
    yb = _scan_gpu(b, h0=host(ha))
    np.testing.assert_allclose(np.concatenate([host(ya), host(yb)], 1), y1, rtol=1e-5, atol=1e-5)


def test_scan_precomputed_dt_codes_identical():
    """The scan given the dt input's codes from ssm_dt_input_quantize gives the same bits as the
    scan computing them itself (the two entry points split one computation)."""
    cfg = wl.CONFIGS["trissm"]
    B, L, Di, R, N = 3, 100, cfg.d_inner, cfg.dt_rank, cfg.d_state
    lat, _ = wl.mixer_problem(cfg, seed=5, layers=1)
    g = wl.rng(6)
    p = wl.scan_problem(B, L, Di, 1, N, True, seed=6)
    dr = wl.normal(g, (B, L, R + 2 * N))
    packed, scale, _ = tws.ssm_ternary_quantize_weights(to_dev(lat[0]["W_dt"]))
    drt = to_dev(dr)
    proj = dict(dt_in=drt[..., :R], w_dt=packed, s_dt=scale, dt_rank=R)
    args = (to_dev(p["x"]), None, to_dev(p["A"]), to_dev(p["Bm"]), to_dev(p["Cm"]), to_dev(p["D"]),
            to_dev(p["dt_bias"]), True)
    y1 = host(tws.ssm_selective_scan_fwd(*args, dt_proj=proj))
    codes, deq = tws.ssm_dt_input_quantize(drt[..., :R], R)
    _, oq, oam, _ = oracle.bitlinear(dr.reshape(B * L, -1), oracle.quantize_weights(lat[0]["W_dt"], 0)[0],
                                     oracle.quantize_weights(lat[0]["W_dt"], 0)[1], k=R)
    np.testing.assert_array_equal(host(codes)[:, :R], oq)
    np.testing.assert_array_equal(host(codes)[:, R:], 0)
    np.testing.assert_array_equal(host(deq), np.maximum(oam, np.float32(1e-5)).astype(np.float64) / 127.0)
    y2 = host(tws.ssm_selective_scan_fwd(*args, dt_proj=dict(proj, dt_codes=codes, dt_deq=deq)))
    np.testing.assert_array_equal(y1, y2)


@pytest.mark.parametrize("B,L,Di,R,dt,gated", [
    (2, 70, 96, 40, "f32", False),   # dt_rank 40: three 16-byte code words per token
    (1, 300, 96, 64, "f32", True),   # dt_rank 64 (four words), cut in two time chunks, gated
    (2, 50, 72, 48, "bf16", True),   # bf16, three words, gated, a partly filled last wave
])
def test_scan_dt_projection_wide_rank(B, L, Di, R, dt, gated):
    """d_state 16 scan with the dt projection evaluated inside it, at wide dt ranks, against the
    oracle: the dt pre-activation is the oracle's BitLinear of the dt input (int8 codes and
    int32 sums identical; the in-scan dequantisation is fp32, reading 38), then the oracle's
    scan, then the SiLU gate."""
    N = 16
    g = wl.rng(B * 1000 + L + R)
    p = wl.scan_problem(B, L, Di, 1, N, True, seed=L + R)
    dr = wl.normal(g, (B, L, R))
    w = wl.normal(g, (Di, R), 0.0, 0.02)
    z = wl.normal(g, (B, L, Di))
    x, Bm, Cm = p["x"], p["Bm"], p["Cm"]
    tdt = torch.float32
    if dt == "bf16":
        x, Bm, Cm, dr, z = (bf16_values(v) for v in (x, Bm, Cm, dr, z))
        tdt = torch.bfloat16
    packed, scale, _ = tws.ssm_ternary_quantize_weights(to_dev(w))
    codes, oscale, _ = oracle.quantize_weights(w, 0)
    pre, *_ = oracle.bitlinear(dr.reshape(B * L, R), codes, oscale)
    y = tws.ssm_selective_scan_fwd(to_dev(x, tdt), None, to_dev(p["A"]), to_dev(Bm, tdt), to_dev(Cm, tdt),
                                   to_dev(p["D"]), to_dev(p["dt_bias"]), True,
                                   dt_proj=dict(dt_in=to_dev(dr, tdt), w_dt=packed, s_dt=scale, dt_rank=R),
                                   gate=to_dev(z, tdt) if gated else None)
    ref, _ = oracle.selective_scan(x, pre.reshape(B, L, Di), p["A"], Bm, Cm, p["D"], p["dt_bias"], True)
    if gated:
        ref = ref * np.vectorize(oracle.silu)(z.astype(np.float64))
    check(host(y), ref, TOL[dt], what=f"test_scan_dt_projection_wide_rank {B} {L} {Di} {R} {dt} {gated}")


def _softplus_sweep_problem(H, P, N, aps):
    """One token per channel (L = 1, zero initial state), x = 1, B = C = the first unit vector,
    D = 0: then y = softplus(delta + bias) of each channel exactly, in any order of evaluation,
    so y shows the scan's softplus value by value over the sweep."""
    v = np.linspace(-30.0, 30.0, H).astype(np.float32)
    e0 = np.zeros((1, 1, N), np.float32)
    e0[..., 0] = 1.0
    A = -np.ones((H, N) if aps else (H,), np.float32)
    return dict(x=np.ones((1, 1, H * P), np.float32), delta=v.reshape(1, 1, H), Bm=e0, Cm=e0.copy(), A=A,
                D=np.zeros(H, np.float32), dt_bias=np.zeros(H, np.float32))


@pytest.mark.parametrize("H,P,N,aps,dt,rtol", [
    (3001, 1, 16, True, "f32", 5e-6),     # Mamba-1 kind scan (its softplus also serves the in-scan dt projection)
    (601, 4, 16, False, "f32", 5e-6),     # SSD kind, recurrent kernel
    (257, 64, 64, False, "bf16", 8e-3),   # SSD kind, chunked matrix-core kernel (bf16 output)
])
def test_scan_softplus_sweep(H, P, N, aps, dt, rtol):
    """softplus(delta + bias) across [-30, 30], element by element against the oracle's
    log1p(exp(v)) (the identity above 20): where 1 + e^v rounds at or above 2 the rounding
    correction must not be applied."""
    p = _softplus_sweep_problem(H, P, N, aps)
    if dt == "bf16":
        p = _bf16_problem(p)
    ref = np.array([oracle.softplus(float(v)) for v in p["delta"].ravel()])
    y = host(_scan_gpu(p, torch.bfloat16 if dt == "bf16" else torch.float32)).reshape(H, P)
    rel = np.abs(y - ref[:, None]) / ref[:, None]
    assert float(rel.max()) <= rtol, (float(rel.max()), float(p["delta"].ravel()[rel.max(axis=1).argmax()]))


def test_scan_bwd_softplus_sweep():
    """The backward recomputes softplus: with L = 1, zero state, x = 1, B = C = e0, D = 0 and
    dy = 1, dx = softplus(delta + bias) per channel."""
    H, N = 3001, 16
    p = _softplus_sweep_problem(H, 1, N, True)
    dy = np.ones((1, 1, H), np.float32)
    got = tws.ssm_selective_scan_bwd(to_dev(p["x"]), to_dev(p["delta"]), to_dev(p["A"]), to_dev(p["Bm"]),
                                     to_dev(p["Cm"]), to_dev(dy), D=to_dev(p["D"]), delta_bias=to_dev(p["dt_bias"]))
    ref = np.array([oracle.softplus(float(v)) for v in p["delta"].ravel()])
    dx = host(got["dx"]).ravel()
    assert float((np.abs(dx - ref) / ref).max()) <= 5e-6


def test_scan_special_cases():
    """B = 0 gives y = D x exactly; empty batch / sequence is a no-op."""
    p = wl.scan_problem(1, 50, 64, 1, 16, True, seed=8)
    p["Bm"] = np.zeros_like(p["Bm"])
    y = host(_scan_gpu(p))
    np.testing.assert_allclose(y, p["x"] * p["D"][None, None, :], rtol=1e-6, atol=0)
    e = dict(p, x=p["x"][:, :0], delta=p["delta"][:, :0], Bm=p["Bm"][:, :0], Cm=p["Cm"][:, :0])
    assert _scan_gpu(e).shape == (1, 0, 64)


# ------------------------------------------------------------------ S9: mixer

@pytest.mark.parametrize("seed", [42, 43, 44])
def test_mixer_bitssm_tiny(seed):
    """bitssm_tiny workload in full (one layer, fp32): GPU mixer vs oracle mixer."""
    cfg = wl.CONFIGS["bitssm_tiny"]
    lat, u = wl.mixer_problem(cfg, seed=seed)
    gw, ow = quantize_layer(cfg, lat[0])
    out = run_gpu_stack(cfg, [gw], u)
    ref = oracle.mixer(oracle_config(cfg), ow, u)
    check(host(out), ref, TOL["f32"], what=f"test_mixer_bitssm_tiny {seed}", **chain("f32"))


def test_mixer_causality_and_determinism():
    cfg = wl.CONFIGS["bitssm_tiny"]
    lat, u = wl.mixer_problem(cfg, seed=42)
    gw, _ = quantize_layer(cfg, lat[0])
    o1 = host(run_gpu_stack(cfg, [gw], u))
    o2 = host(run_gpu_stack(cfg, [gw], u))
    np.testing.assert_array_equal(o1, o2)
    u2 = u.copy()
    u2[:, 40] = -u2[:, 40] + 0.3
    o3 = host(run_gpu_stack(cfg, [gw], u2))
    np.testing.assert_array_equal(o3[:, :40], o1[:, :40])
    assert not np.array_equal(o3[:, 40], o1[:, 40])


def _stack_sampled(name, seqs, seed=42):
    """Full-size stack on the GPU (the launch configuration the benchmark times).  Each layer is
    checked against the oracle given the same layer input (the GPU's stored input of the
    sampled sequences; sequences are independent): that is the parity bar per mixer output,
    norm-wise and element by element.  The free-running drift (oracle stack from u, no
    re-synchronisation) is returned too: a one-ulp difference anywhere can flip an int8 code at
    a .5 boundary, and flips compound through a quantised stack, so the drift of a many-layer
    stack is held to a looser bound than one layer's output."""
    cfg = wl.CONFIGS[name]
    lat, u = wl.mixer_problem(cfg, seed=seed)
    if cfg.act_dtype == "bf16":
        u = bf16_values(u)
    pairs = [quantize_layer(cfg, l) for l in lat]
    c = gpu_config(cfg)
    h = to_dev(u, torch_dtype(cfg))
    ws = torch.empty(tws.ssm_mixer_workspace_bytes(c, cfg.batch, cfg.seqlen), dtype=torch.uint8, device=DEV)
    per_layer = []
    for li, (gw, ow) in enumerate(pairs):
        h_in = host(h)[seqs]
        h = tws.ssm_mixer_fwd(c, tws.mixer_weights(gw), h, add_residual=True, out=h, workspace=ws)
        ref = oracle.mixer(oracle_config(cfg), ow, h_in)
        m = check(host(h)[seqs], ref, TOL[cfg.act_dtype], what=f"{name} layer {li}",
                  **chain(cfg.act_dtype, cfg.act_bits == 16))
        per_layer.append(m["norm"])
    free = oracle.mixer_stack(oracle_config(cfg), [o for _, o in pairs], u[seqs])
    drift = rel_err(host(h)[seqs], free)
    print(f"{name}: per-layer rel err {['%.2e' % e for e in per_layer]}, free-running drift {drift:.2e}")
    return per_layer, drift


def test_mixer_trissm_stack_sampled():
    per_layer, drift = _stack_sampled("trissm", [0, 37, 63])
    assert drift <= 0.05, drift


def test_mixer_long_scan_sampled():
    # one layer: the free-running output is the layer's own, held to the per-layer bar
    per_layer, drift = _stack_sampled("long_scan", [5])
    assert drift <= TOL["f32"], drift


def test_mixer_ternaryssm50m_stack_sampled():
    per_layer, drift = _stack_sampled("ternaryssm50m", [0, 15])
    assert drift <= 0.1, drift


def test_mixer_mamba2_ssd_sampled():
    per_layer, drift = _stack_sampled("mamba2_ssd", [2])
    assert drift <= TOL["bf16"], drift


def _boundary_dist(y_rows):
    """Distance of each x_hat * sigma of the rows' A8 quantiser input from the nearest .5."""
    out = []
    for r in np.asarray(y_rows, np.float32):
        xh = oracle.norm_row(r)
        sig = np.float32(127.0) / np.maximum(np.abs(xh).max(), np.float32(1e-5))
        t = np.abs(xh * sig).astype(np.float64)
        out.append(np.abs((t - np.floor(t)) - 0.5))
    return np.stack(out)


@pytest.mark.parametrize("name,seqs", [("trissm", [0, 37, 63]), ("bitssm_tiny", [0, 1]),
                                       ("ternaryssm50m", [3, 14])])
def test_mixer_stages_bit_exact(name, seqs):
    """The integer steps inside the mixer's kernels (the fused front of the TriSSM shape: in_proj,
    x_proj and the dt input's codes in one kernel; the dt projection inside the scan), stage by
    stage at the full workload shape on the sampled sequences: each stage fed the GPU's previous
    stage equals the oracle bit for bit (x, p and out are the A8 BitLinear's fp64 epilogue,
    rounded once; codes, absmax factors and int32 sums are integers).  The scan output y is
    float (1e-4 elementwise).  Codes of out_proj's input computed from the oracle's y and from
    the GPU's y may differ only within 1e-3 of a .5 rounding boundary (counted)."""
    cfg = wl.CONFIGS[name]
    lat, u = wl.mixer_problem(cfg, seed=42, layers=1)
    if cfg.act_dtype == "bf16":
        u = bf16_values(u)
    gw, ow = quantize_layer(cfg, lat[0])
    c = gpu_config(cfg)
    out, st = tws.ssm_mixer_fwd_stages(c, tws.mixer_weights(gw), to_dev(u, torch_dtype(cfg)), add_residual=True)
    B, L, Di, R, N = cfg.batch, cfg.seqlen, cfg.d_inner, cfg.dt_rank, cfg.d_state
    rows = np.concatenate([np.arange(b * L, (b + 1) * L) for b in seqs])
    rnd = (lambda a: bf16_values(a)) if cfg.act_dtype == "bf16" else (lambda a: a.astype(np.float32))
    u2 = u.reshape(B * L, -1)
    x, p, y = host(st["x"])[rows], host(st["p"])[rows], host(st["y"])[rows]
    xr, *_ = oracle.bitlinear(u2[rows], ow["c_in"], ow["s_in"])
    np.testing.assert_array_equal(x, rnd(xr), err_msg="x = in_proj(u)")
    pr, *_ = oracle.bitlinear(x, ow["c_x"], ow["s_x"])
    np.testing.assert_array_equal(p, rnd(pr), err_msg="p = x_proj(x)")
    z, dq, dam, dacc = oracle.bitlinear(p, ow["c_dt"], ow["s_dt"], k=R)
    np.testing.assert_array_equal(host(st["dt_codes"])[rows], dq, err_msg="dt input codes")
    np.testing.assert_array_equal(host(st["dt_deq"])[rows], np.maximum(dam, np.float32(1e-5)).astype(np.float64) / 127.0,
                                  err_msg="dt input dequantisation factors")
    np.testing.assert_array_equal(host(st["dt_acc"])[rows], dacc, err_msg="dt projection int32 sums")
    o = host(out).reshape(B * L, -1)[rows]
    orr, *_ = oracle.bitlinear(y, ow["c_out"], ow["s_out"])
    np.testing.assert_array_equal(o, rnd(orr + u2[rows].astype(np.float64)), err_msg="out = u + out_proj(y)")
    # the scan, fed the GPU's x, B, C and the dt projection's values (floats)
    sh = (len(seqs), L)
    yr, _ = oracle.selective_scan(x.reshape(*sh, Di), z.astype(np.float32).reshape(*sh, Di), ow["A"],
                                  p[:, R:R + N].reshape(*sh, N), p[:, R + N:].reshape(*sh, N), ow["D"], ow["dt_bias"])
    yr = rnd(yr.reshape(len(rows), Di))
    check(y, yr, TOL[cfg.act_dtype], what=f"stages {name} y")
    # Q19: out_proj's input codes from the oracle's y against those from the GPU's y
    _, q_gpu, _, _ = oracle.bitlinear(y, ow["c_out"], ow["s_out"])
    _, q_ref, _, _ = oracle.bitlinear(yr, ow["c_out"], ow["s_out"])
    flips = q_gpu != q_ref
    if flips.any() and cfg.act_dtype == "f32":
        # (with bf16 activations the two y differ by whole bf16 steps, which move codes anywhere)
        assert np.abs(q_gpu.astype(int) - q_ref.astype(int)).max() == 1
        dist = _boundary_dist(yr)[flips]
        assert float(dist.max()) < 1e-3, float(dist.max())
    print(f"{name}: out_proj input codes flipped at .5 boundaries: {int(flips.sum())} of {flips.size}")


def test_mixer_ssd_stages():
    """The Mamba-2 1.3B-shaped W1.58A16 SSD layer stage by stage at full size on a sampled
    sequence: the scan fed the GPU's own in_proj output v (x, B, C, dt) against the oracle's
    recurrence (bf16 outputs: 2e-2, element by element), and out = u + out_proj(y) fed the GPU's
    y against the oracle's A16 BitLinear."""
    cfg = wl.CONFIGS["mamba2_ssd"]
    lat, u = wl.mixer_problem(cfg, seed=42, layers=1)
    u = bf16_values(u)
    gw, ow = quantize_layer(cfg, lat[0])
    c = gpu_config(cfg)
    out, st = tws.ssm_mixer_fwd_stages(c, tws.mixer_weights(gw), to_dev(u, torch.bfloat16), add_residual=True,
                                       want=("p", "y"))
    B, L, Di, N, H = cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.nheads
    seq = 2
    rows = np.arange(seq * L, (seq + 1) * L)
    v = host(st["p"])[rows]
    y = host(st["y"])[rows]
    vr, *_ = oracle.bitlinear(u.reshape(B * L, -1)[rows], ow["c_in"], ow["s_in"], cfg.group_size, 16)
    check(v, bf16_values(vr), TOL["bf16"], what="ssd stages v = in_proj(u)")
    sh = (1, L)
    yr, _ = oracle.selective_scan(v[:, :Di].reshape(*sh, Di), v[:, Di + 2 * N:].reshape(*sh, H), ow["A"],
                                  v[:, Di:Di + N].reshape(*sh, N), v[:, Di + N:Di + 2 * N].reshape(*sh, N), ow["D"],
                                  ow["dt_bias"])
    m = check(y, bf16_values(yr.reshape(L, Di)), TOL["bf16"], what="ssd stages y = scan(v)")
    e = np.abs(y - yr.reshape(L, Di)) / (np.abs(yr.reshape(L, Di)) + np.sqrt(np.mean(yr ** 2)))
    t, ch = np.unravel_index(np.argmax(e), e.shape)
    print(f"scan elementwise max {m['elem_max']:.2e} at t {t} channel {ch} (head {ch // cfg.headdim})")
    orr, *_ = oracle.bitlinear(y, ow["c_out"], ow["s_out"], cfg.group_size, 16)
    o = host(out).reshape(B * L, -1)[rows]
    check(o, bf16_values(orr + u.reshape(B * L, -1)[rows].astype(np.float64)), TOL["bf16"],
          what="ssd stages out = u + out_proj(y)")


def test_mixer_ssd_small_fp32():
    """SSD kind at a small fp32 shape (several heads, ragged time tile)."""
    cfg = wl.CONFIGS["mamba2_ssd"].with_(d_model=256, d_inner=256, d_state=64, nheads=4, headdim=64, batch=2,
                                          seqlen=45, act_dtype="f32")
    lat, u = wl.mixer_problem(cfg, seed=11)
    gw, ow = quantize_layer(cfg, lat[0])
    out = run_gpu_stack(cfg, [gw], u)
    ref = oracle.mixer(oracle_config(cfg), ow, u)
    check(host(out), ref, TOL["f32"], what="test_mixer_ssd_small_fp32", **chain("f32"))


@pytest.mark.parametrize("name,over", [
    ("trissm", dict(batch=2, seqlen=3, layers=1)),          # fused front
    ("bitssm_tiny", dict(batch=3, seqlen=17)),
    ("ternaryssm50m", dict(batch=1, seqlen=5, layers=1)),   # separate in_proj / x_proj
    ("mamba2_ssd", dict(d_model=256, d_inner=256, d_state=64, nheads=4, headdim=64, batch=2, seqlen=7,
                        layers=1)),
    ("trissm_gated", dict(batch=2, seqlen=19, layers=1)),
    ("trissm_fp", dict(batch=2, seqlen=19, layers=1)),                 # stored dt
    ("mamba2_ssd_gated", dict(d_model=256, d_inner=256, d_state=64, nheads=4, headdim=64, batch=2, seqlen=7,
                              layers=1)),
])
def test_mixer_stays_inside_workspace(name, over):
    """Everything the mixer writes to its workspace lies within ssm_mixer_workspace_bytes: a
    guard region after it keeps its fill pattern."""
    cfg = wl.CONFIGS[name].with_(**over)
    lat, u = wl.mixer_problem(cfg, seed=3, layers=1)
    gw, _ = quantize_layer(cfg, lat[0])
    c = gpu_config(cfg)
    nb = tws.ssm_mixer_workspace_bytes(c, cfg.batch, cfg.seqlen)
    buf = torch.full((nb + 4096,), 0xA5, dtype=torch.uint8, device=DEV)
    h = to_dev(u, torch_dtype(cfg))
    tws.ssm_mixer_fwd(c, tws.mixer_weights(gw), h, add_residual=True, out=h, workspace=buf[:nb])
    assert bool((buf[nb:] == 0xA5).all())


# ------------------------------------------------------------------ decode step

def _decode(cfg, gw, u_host):
    """Feed u [B, L, d] to ssm_mixer_step one token at a time from a zero state."""
    c = gpu_config(cfg)
    u = to_dev(u_host, torch_dtype(cfg))
    B, L, _ = u.shape
    shape = (B, cfg.d_inner, cfg.d_state) if cfg.kind == wl.MAMBA1 else (B, cfg.nheads, cfg.headdim, cfg.d_state)
    state = torch.zeros(shape, dtype=torch.float32, device=DEV)
    cst = (torch.zeros((B, cfg.d_conv - 1, cfg.conv_channels), dtype=torch.float32, device=DEV)
           if cfg.gated and cfg.d_conv > 1 else None)
    ws = torch.empty(tws.ssm_mixer_workspace_bytes(c, B, 1), dtype=torch.uint8, device=DEV)
    mw = tws.mixer_weights(gw)
    out = torch.empty_like(u)
    for t in range(L):
        tok = u[:, t].contiguous()
        out[:, t] = tws.ssm_mixer_step(c, mw, tok, state, add_residual=True, workspace=ws, conv_state=cst)
    return out, state


DECODE_CASES = [
    ("bitssm_tiny", {}, 42),
    ("trissm_fp_inout", dict(batch=2, seqlen=12, layers=1), 14),
    ("trissm_gated", dict(batch=3, seqlen=20, layers=1), 12),
    ("mamba2_ssd_gated", dict(d_model=256, d_inner=256, d_state=64, nheads=4, headdim=64, batch=2, seqlen=14,
                              layers=1), 13),
    ("trissm", dict(batch=4, seqlen=24, layers=1), 7),
    ("ternaryssm50m", dict(batch=3, seqlen=16, layers=1), 8),
    ("mamba2_ssd", dict(d_model=256, d_inner=256, d_state=64, nheads=4, headdim=64, batch=2, seqlen=20,
                        act_dtype="f32", layers=1), 9),
    ("mamba2_ssd", dict(d_model=256, d_inner=256, d_state=128, nheads=4, headdim=64, batch=2, seqlen=12,
                        layers=1), 10),
]


@pytest.mark.parametrize("name,over,seed", DECODE_CASES)
def test_mixer_decode_step(name, over, seed):
    """Token-by-token decoding reproduces the oracle's mixer over the whole sequence, and the
    GPU's own whole-sequence forward."""
    cfg = wl.CONFIGS[name].with_(**over)
    lat, u = wl.mixer_problem(cfg, seed=seed, layers=1)
    if cfg.act_dtype == "bf16":
        u = bf16_values(u)
    gw, ow = quantize_layer(cfg, lat[0])
    out, state = _decode(cfg, gw, u)
    ref = oracle.mixer(oracle_config(cfg), ow, u)
    tol = TOL["bf16"] if cfg.act_dtype == "bf16" else TOL["f32"]
    check(host(out), ref, tol, what=f"test_mixer_decode_step {name} {seed}", **chain(cfg.act_dtype, cfg.act_bits == 16))
    full = host(run_gpu_stack(cfg, [gw], u))
    check(host(out), full, tol, what=f"test_mixer_decode_step {name} {seed} vs prefill", **chain(cfg.act_dtype, cfg.act_bits == 16))
    assert bool(torch.isfinite(state).all()) and float(state.abs().max()) > 0


DECODE_EXACT_CASES = [  # configurations the decode step runs on its own kernels
    ("trissm", dict(batch=4, seqlen=12, layers=1), 21),
    ("trissm", dict(batch=17, seqlen=5, layers=1), 22),     # two 16-row groups, the second ragged
    ("ternaryssm50m", dict(batch=3, seqlen=6, layers=1), 23),  # bf16, d_inner 1024, dt_rank 32
    ("bitssm_tiny", {}, 24),
]


@pytest.mark.parametrize("name,over,seed", DECODE_EXACT_CASES)
def test_mixer_decode_step_equals_prefill(name, over, seed):
    """The decode step's kernels evaluate every quantity as the whole-sequence path does (same
    norms, codes, int32 sums, fp64 epilogues, dt dequantisation and state recurrence), so the
    token-by-token outputs equal the prefill's bit for bit."""
    cfg = wl.CONFIGS[name].with_(**over)
    lat, u = wl.mixer_problem(cfg, seed=seed, layers=1)
    if cfg.act_dtype == "bf16":
        u = bf16_values(u)
    gw, _ = quantize_layer(cfg, lat[0])
    out, state = _decode(cfg, gw, u)
    full = host(run_gpu_stack(cfg, [gw], u))
    np.testing.assert_array_equal(host(out), full)
    assert bool(torch.isfinite(state).all())


STACK_CASES = [  # (config, overrides, layers, seed)
    ("trissm", dict(batch=3, seqlen=4), 5, 31),           # one fused launch
    ("trissm", dict(batch=1, seqlen=3), 26, 32),          # two fused launches (24 + 2 layers)
    ("trissm", dict(batch=64, seqlen=2), 12, 36),         # the decode measurement's stack
    ("ternaryssm50m", dict(batch=2, seqlen=3), 3, 33),    # bf16, d_model 512, d_inner 1024, dt_rank 32
    ("bitssm_tiny", dict(seqlen=3), 2, 37),
    ("trissm_gated", dict(batch=2, seqlen=3), 3, 34),     # layer by layer (gated block)
    ("mamba2_ssd", dict(d_model=256, d_inner=256, d_state=64, nheads=4, headdim=64, batch=2, seqlen=3), 2, 35),
]


@pytest.mark.parametrize("name,over,layers,seed", STACK_CASES)
def test_mixer_stack_step_equals_layer_steps(name, over, layers, seed):
    """ssm_mixer_stack_step equals ssm_mixer_step applied layer after layer, bit for bit, in the
    outputs of every token and in every layer's state afterwards."""
    cfg = wl.CONFIGS[name].with_(layers=layers, **over)
    lat, u = wl.mixer_problem(cfg, seed=seed, layers=layers)
    if cfg.act_dtype == "bf16":
        u = bf16_values(u)
    gws = [quantize_layer(cfg, lat[i])[0] for i in range(layers)]
    c = gpu_config(cfg)
    ud = to_dev(u, torch_dtype(cfg))
    B, L, _ = ud.shape
    shape = (B, cfg.d_inner, cfg.d_state) if cfg.kind == wl.MAMBA1 else (B, cfg.nheads, cfg.headdim, cfg.d_state)
    st1 = [torch.zeros(shape, dtype=torch.float32, device=DEV) for _ in range(layers)]
    st2 = [torch.zeros(shape, dtype=torch.float32, device=DEV) for _ in range(layers)]
    conv = cfg.gated and cfg.d_conv > 1
    cshape = (B, cfg.d_conv - 1, cfg.conv_channels)
    cs1 = [torch.zeros(cshape, dtype=torch.float32, device=DEV) if conv else None for _ in range(layers)]
    cs2 = [torch.zeros(cshape, dtype=torch.float32, device=DEV) for _ in range(layers)] if conv else None
    mws = [tws.mixer_weights(g) for g in gws]
    ws1 = torch.empty(tws.ssm_mixer_workspace_bytes(c, B, 1), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty(tws.ssm_mixer_stack_workspace_bytes(c, B), dtype=torch.uint8, device=DEV)
    for t in range(L):
        tok = ud[:, t].contiguous()
        h = tok
        for i in range(layers):
            h = tws.ssm_mixer_step(c, mws[i], h, st1[i], add_residual=True, workspace=ws1, conv_state=cs1[i])
        o = tws.ssm_mixer_stack_step(c, mws, tok, st2, add_residual=True, workspace=ws2, conv_states=cs2)
        np.testing.assert_array_equal(host(o), host(h), err_msg=f"token {t}")
    for i in range(layers):
        np.testing.assert_array_equal(host(st2[i]), host(st1[i]), err_msg=f"state of layer {i}")


# ------------------------------------------------------------------ gated block

def _ulp_diff(got, ref, bf16: bool):
    """Distance in units of the last place of the stored type (fp32 or bf16 bit patterns)."""
    g = np.asarray(got, np.float32).view(np.int32).astype(np.int64)
    r = np.asarray(ref, np.float32).view(np.int32).astype(np.int64)
    if bf16:
        g, r = g >> 16, r >> 16
    return np.abs(g - r)


CONV_CASES = [  # (batch, seqlen, channels, ldx, width, dtype, state)
    (2, 37, 100, 130, 4, "f32", None),
    (3, 70, 256, 512, 4, "bf16", None),
    (1, 5, 64, 64, 3, "f32", "separate"),
    (2, 1, 200, 400, 4, "f32", "inplace"),
    (2, 2, 72, 72, 4, "bf16", "inplace"),
    (2, 33, 48, 48, 1, "f32", None),
    (1, 64, 4352, 8512, 4, "bf16", None),  # the Mamba-2 gated block's x, B, C channels
]


@pytest.mark.parametrize("batch,L,C,ldx,K,dt,state", CONV_CASES)
def test_conv_silu_parity(batch, L, C, ldx, K, dt, state):
    """Causal convolution + SiLU: fp64 on both sides, rounded once to the stored type, so the
    values agree to the last bit except where the two fp64 exponentials straddle a rounding
    boundary (at most one unit of the last place, rarely)."""
    g = wl.rng(batch * 1000 + L * 10 + K)
    x = wl.normal(g, (batch, L, ldx))
    if dt == "bf16":
        x = bf16_values(x)
    w = g.uniform(-0.5, 0.5, (C, K)).astype(np.float32)
    b = g.uniform(-0.5, 0.5, (C,)).astype(np.float32)
    st = wl.normal(g, (batch, K - 1, C)) if state else None
    if st is not None and dt == "bf16":
        st = bf16_values(st)
    ref, ref_st = oracle.conv_silu(x[:, :, :C], w, b, state=st, act_dtype=oracle.BF16 if dt == "bf16" else oracle.F32)
    xd = to_dev(x, torch.bfloat16 if dt == "bf16" else torch.float32)
    sin = to_dev(st) if st is not None else None
    sout = (sin if state == "inplace" else torch.empty_like(sin)) if st is not None else None
    got = tws.ssm_conv1d_silu_fwd(xd, to_dev(w), to_dev(b), state_in=sin, state_out=sout, channels=C)
    d = _ulp_diff(host(got), ref, dt == "bf16")
    assert d.max() <= 1 and np.mean(d > 0) <= 1e-3, (d.max(), np.mean(d > 0))
    if st is not None:
        np.testing.assert_array_equal(host(sout), ref_st)


def test_conv_silu_streaming_equals_whole():
    """Chunks of a sequence with the state carried give the whole sequence's values bit for bit."""
    g = wl.rng(77)
    x = wl.normal(g, (2, 50, 96))
    w = g.uniform(-0.5, 0.5, (96, 4)).astype(np.float32)
    xd = to_dev(x)
    wd = to_dev(w)
    whole = host(tws.ssm_conv1d_silu_fwd(xd, wd))
    st = torch.zeros((2, 3, 96), device=DEV)
    parts = []
    for a, b in ((0, 17), (17, 18), (18, 50)):
        parts.append(host(tws.ssm_conv1d_silu_fwd(xd[:, a:b].contiguous(), wd, state_in=st, state_out=st)))
    np.testing.assert_array_equal(np.concatenate(parts, axis=1), whole)


@pytest.mark.parametrize("kind,dt", [("m1", "f32"), ("m1", "bf16"), ("ssd", "f32"), ("ssd", "bf16")])
def test_scan_gate_parity(kind, dt):
    """The scan's gate: y * SiLU(gate), against the oracle scan's y times SiLU in fp64."""
    if kind == "m1":
        p = wl.scan_problem(2, 45, 70, 1, 16, True, seed=5)
        H, P = 70, 1
    else:
        p = wl.scan_problem(2, 130, 4, 64, 64, False, seed=6)
        H, P = 4, 64
    gate = wl.normal(wl.rng(9), (2, p["x"].shape[1], H * P), 0.0, 2.0)
    if dt == "bf16":
        p = _bf16_problem(p)
        gate = bf16_values(gate)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    y = tws.ssm_selective_scan_fwd(to_dev(p["x"], tdt), to_dev(p["delta"], tdt), to_dev(p["A"]),
                                   to_dev(p["Bm"], tdt), to_dev(p["Cm"], tdt), to_dev(p["D"]),
                                   to_dev(p["dt_bias"]), True, gate=to_dev(gate, tdt))
    ref, _ = oracle.selective_scan(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["D"], p["dt_bias"])
    sil = np.vectorize(oracle.silu)(gate.astype(np.float64))
    check(host(y), ref * sil, (TOL["bf16"] if dt == "bf16" else 1e-5), what=f"test_scan_gate_parity {kind} {dt}")


GATED_MIXER_CASES = [
    ("trissm_gated", dict(batch=2, seqlen=40, layers=1), 31),
    ("trissm_gated", dict(batch=1, seqlen=19, layers=1, act_dtype="bf16"), 32),
    ("mamba2_ssd_gated", dict(d_model=256, d_inner=256, d_state=64, nheads=4, headdim=64, batch=2, seqlen=45,
                              act_dtype="f32", layers=1), 33),
    # eight heads: every in_proj column block starts 16-byte aligned, so the chunked SSD kernel runs
    ("mamba2_ssd_gated", dict(d_model=256, d_inner=512, d_state=128, nheads=8, headdim=64, batch=2, seqlen=130,
                              layers=1), 34),
]


@pytest.mark.parametrize("name,over,seed", GATED_MIXER_CASES)
def test_mixer_gated_parity(name, over, seed):
    """The gated block (convolution + SiLU on the SSM input, SiLU gate) against the oracle."""
    cfg = wl.CONFIGS[name].with_(**over)
    lat, u = wl.mixer_problem(cfg, seed=seed, layers=1)
    if cfg.act_dtype == "bf16":
        u = bf16_values(u)
    gw, ow = quantize_layer(cfg, lat[0])
    out = run_gpu_stack(cfg, [gw], u)
    ref = oracle.mixer(oracle_config(cfg), ow, u)
    check(host(out), ref, TOL[cfg.act_dtype], what=f"test_mixer_gated_parity {name} {seed}", **chain(cfg.act_dtype, cfg.act_bits == 16))


def test_mixer_trissm_gated_stack_sampled():
    per_layer, drift = _stack_sampled("trissm_gated", [0, 41])
    assert drift <= 0.05, drift


def test_mixer_mamba2_ssd_gated_sampled():
    per_layer, drift = _stack_sampled("mamba2_ssd_gated", [1])
    assert drift <= TOL["bf16"], drift


# ------------------------------------------------------------------ full-precision projections

DENSE_CASES = [  # (m, k, n, dtype, residual, ldx)
    (100, 256, 512, "f32", False, 256),
    (77, 512, 256, "f32", True, 600),
    (64, 2048, 4416, "bf16", False, 2048),
    (33, 4096, 2048, "bf16", True, 4096),
    (1, 16, 512, "f32", False, 48),
    (50, 130, 70, "f32", True, 133),     # odd row stride and k: element-wise staging
    (40, 100, 36, "bf16", False, 100),   # k not a multiple of 8
    (300, 96, 200, "bf16", True, 96),    # several tiles each way, ragged last ones
]


@pytest.mark.parametrize("m,k,n,dt,res,ldx", DENSE_CASES)
def test_dense_parity(m, k, n, dt, res, ldx):
    """Full-precision linear layer (the library's own MFMA kernel) against the oracle's fp64 x W^T."""
    g = wl.rng(m + k + n)
    x = wl.normal(g, (m, ldx))
    W = wl.normal(g, (n, k), 0.0, 1.0 / np.sqrt(k))
    r = wl.normal(g, (m, n)) if res else None
    if dt == "bf16":
        x, W = bf16_values(x), bf16_values(W)
        r = bf16_values(r) if res else None
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    xd = to_dev(x, tdt)
    y = tws.ssm_dense_fwd(xd[:, :k], to_dev(W, tdt), residual=to_dev(r, tdt) if res else None)
    ref = oracle.dense(x, W, k=k) + (r if res else 0.0)
    # fp32: k products summed in fp32 leave a typical error near sqrt(k) 2^-24 of the output
    # scale, 4e-6 elementwise for k <= 4096; the norm-wise bound stays 1e-6
    bound = {} if dt == "bf16" else {"elem": 4e-6, "frac": 1.0}  # every element within elem
    check(host(y), ref, (4e-3 if dt == "bf16" else 1e-6), **bound, what=f"test_dense_parity {m} {k} {n} {dt}")


def test_dense_allocates_nothing():
    """The full-precision layer runs on the library's own kernels: a call leaves the device's
    free memory unchanged (no library handle, no workspace of its own)."""
    g = wl.rng(5)
    x = to_dev(wl.normal(g, (256, 512)))
    W = to_dev(wl.normal(g, (384, 512), 0.0, 0.05))
    y = torch.empty((256, 384), dtype=torch.float32, device="cuda")
    tws.ssm_ternary_quantize_weights(W)  # the library's code object is resident from here on
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    tws.ssm_dense_fwd(x, W, out=y)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, (free0, free1)
    check(host(y), oracle.dense(host(x), host(W), k=512), 1e-6, elem=4e-6, frac=1.0,
          what="test_dense_allocates_nothing")


FP_MIXER_CASES = [
    ("trissm_fp_inout", dict(batch=2, seqlen=40, layers=1), 51),
    ("trissm_fp", dict(batch=2, seqlen=40, layers=1), 52),
    ("trissm_fp", dict(batch=1, seqlen=33, layers=1, act_dtype="bf16"), 53),
    ("mamba2_ssd_fp", dict(d_model=256, d_inner=512, d_state=128, nheads=8, headdim=64, batch=2, seqlen=130,
                           layers=1), 54),
]


@pytest.mark.parametrize("name,over,seed", FP_MIXER_CASES)
def test_mixer_fp_proj_parity(name, over, seed):
    """Full-precision projections (TriSSM's in/out split; the fp_ssm baseline): the mixer output
    alone (no residual, which would dominate) against the oracle, then with the residual in place."""
    cfg = wl.CONFIGS[name].with_(**over)
    lat, u = wl.mixer_problem(cfg, seed=seed, layers=1)
    if cfg.act_dtype == "bf16":
        u = bf16_values(u)
    gw, ow = quantize_layer(cfg, lat[0])
    c = gpu_config(cfg)
    tol = TOL["bf16"] if cfg.act_dtype == "bf16" else TOL["f32"]
    h = to_dev(u, torch_dtype(cfg))
    out = tws.ssm_mixer_fwd(c, tws.mixer_weights(gw), h, add_residual=False)
    ref = oracle.mixer(oracle_config(cfg), ow, u, residual=False)
    check(host(out), ref, tol, what=f"test_mixer_fp_proj_parity {name} {seed}", **chain(cfg.act_dtype, cfg.act_bits == 16))
    out2 = tws.ssm_mixer_fwd(c, tws.mixer_weights(gw), h, add_residual=True, out=h)
    ref2 = oracle.mixer(oracle_config(cfg), ow, u, residual=True)
    check(host(out2), ref2, tol, what=f"test_mixer_fp_proj_parity {name} {seed} residual", **chain(cfg.act_dtype, cfg.act_bits == 16))


# ------------------------------------------------------------------ STE backward, QAT step

BWD_CASES = [  # (m, k, n, group, x dtype, gain)
    (100, 256, 512, 0, "f32", False),   # TriSSM in_proj shape (rows)
    (77, 512, 256, 0, "bf16", True),    # TriSSM out_proj shape, bf16 activations, gains
    (64, 256, 200, 128, "f32", False),  # grouped scales, ragged n
    (33, 1024, 64, 128, "bf16", True),
    (1, 100, 30, 0, "f32", False),      # one row, ragged k
    (2048, 256, 192, 0, "f32", False),  # dW reduction split over token chunks
    (4096, 128, 96, 128, "bf16", True),
    (50, 48, 40, 0, "f32", True),       # narrow output: four row tiles per block, rows past M
    (300, 20, 100, 0, "f32", True),     # two column tiles, ragged k and n
    (37, 1024, 70, 0, "bf16", False),   # 64 column tiles, 16 per wave
    (20, 1100, 48, 0, "f32", False),    # k > 1024: dx through the dense fp32 product
    (129, 16, 512, 0, "f32", False),    # the dt projection's shape (one column tile)
]


@pytest.mark.parametrize("m,k,n,group,xd,gain", BWD_CASES)
def test_bitlinear_bwd_parity(m, k, n, group, xd, gain):
    """Straight-through-estimator backward (dx through RMSNorm, dW, the scale gradient) against
    the oracle's fp64 evaluation of the same estimator."""
    g = wl.rng(m + 5 * k + 3 * n + group)
    x = wl.normal(g, (m, k))
    if xd == "bf16":
        x = bf16_values(x)
    w = wl.normal(g, (n, k), 0.0, 0.02)
    gn = (1.0 + 0.2 * wl.normal(g, (k,))).astype(np.float32) if gain else None
    dy = wl.normal(g, (m, n))
    packed, scale, _ = tws.ssm_ternary_quantize_weights(to_dev(w), group)
    codes, oscale, _ = oracle.quantize_weights(w, group)
    xdt = torch.bfloat16 if xd == "bf16" else torch.float32
    dx, dw, ds = tws.ssm_bitlinear_bwd(to_dev(x, xdt), packed, scale, n, to_dev(dy), group_size=group,
                                       norm_weight=to_dev(gn) if gain else None, w_latent=to_dev(w))
    ref = oracle.bitlinear_bwd(x, codes, oscale, dy, group=group, norm_w=gn, w_latent=w)
    check(host(dx), ref["dx"], 1e-5, what=f"test_bitlinear_bwd_parity dx {m} {k} {n} {group}")
    check(host(dw), ref["dw"], 1e-5, what=f"test_bitlinear_bwd_parity dw {m} {k} {n} {group}")
    # the scale gradient sums terms of both signs: compare against the sum of their magnitudes
    v = w.astype(np.float64) / (np.repeat(np.asarray(oscale, np.float64).reshape(n, -1), group, axis=1)
                                if group else float(np.asarray(oscale).ravel()[0]))
    fac = np.where(np.abs(v) <= 1.0, codes - v, codes)
    mag = np.abs(ref["dw"] * fac)
    mag = np.array([mag.sum()]) if group == 0 else mag.reshape(n, k // group, group).sum(axis=2)
    assert np.all(np.abs(host(ds).reshape(mag.shape) - ref["ds"].reshape(mag.shape)) <= 1e-5 * mag + 1e-12)


@pytest.mark.parametrize("group", [0, 128])
def test_qat_step_parity(group):
    """One QAT step: the updated weights and scales bit for bit, the codes under the learned
    scales and their zero count exactly (inputs: seeded gradients of a realistic scale)."""
    g = wl.rng(70 + group)
    n, k = 96, 256
    w = wl.normal(g, (n, k), 0.0, 0.02)
    dw = wl.normal(g, (n, k), 0.0, 1.0)
    _, s0, _ = oracle.quantize_weights(w, group)
    s0 = np.asarray(s0, np.float32)
    ds = wl.normal(g, s0.shape, 0.0, 0.5)
    lr, lr_s = 1e-3, 1e-3
    W, s, codes, zeros = oracle.qat_step(w, s0, dw, ds, lr, lr_s, group)
    wd, sd = to_dev(w), to_dev(s0.ravel())
    packed, zc = tws.ssm_qat_sgd_step(wd, sd, to_dev(dw), to_dev(np.asarray(ds).ravel()), lr, lr_s, group)
    np.testing.assert_array_equal(host(wd), W)
    np.testing.assert_array_equal(host(sd), np.asarray(s).ravel())
    np.testing.assert_array_equal(host(packed), oracle.pack(codes))
    assert int(host(zc)[0]) == zeros



SCAN_BWD_CASES = [  # (batch, L, H, N, dtype, h0)
    (2, 37, 70, 16, "f32", False),     # ragged channel tile, ragged time
    (3, 130, 128, 8, "bf16", True),
    (1, 300, 512, 16, "f32", True),
    (8, 256, 512, 16, "f32", False),   # TriSSM width and length
    (2, 20, 64, 64, "f32", True),
    (2, 100, 64, 4, "f32", True),      # 64-step time chunks, ragged last chunk
    (1, 45, 96, 32, "bf16", False),    # 8-step time chunks
]


@pytest.mark.parametrize("batch,L,H,N,dt,with_h0", SCAN_BWD_CASES)
def test_scan_bwd_parity(batch, L, H, N, dt, with_h0):
    """Backward of the Mamba-1 kind scan against the oracle's reverse accumulation: every
    gradient to 2e-4 norm-wise (fp32 accumulation over the sequence on the GPU, fp64 in the
    oracle; the forward's hardware exp2 and softplus)."""
    p = wl.scan_problem(batch, L, H, 1, N, True, seed=batch * 100 + L + N)
    g = wl.rng(batch + L + H)
    dy = wl.normal(g, (batch, L, H))
    h0 = wl.normal(g, (batch, H, 1, N), 0.0, 0.5) if with_h0 else None
    if dt == "bf16":
        p = _bf16_problem(p)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    got = tws.ssm_selective_scan_bwd(to_dev(p["x"], tdt), to_dev(p["delta"], tdt), to_dev(p["A"]),
                                     to_dev(p["Bm"], tdt), to_dev(p["Cm"], tdt), to_dev(dy), D=to_dev(p["D"]),
                                     delta_bias=to_dev(p["dt_bias"]), h0=to_dev(h0) if with_h0 else None)
    ref = oracle.selective_scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["D"], dy,
                                    delta_bias=p["dt_bias"], h0=h0)
    for k in ("dx", "ddelta", "dA", "dB", "dC", "dD", "dbias", "dh0"):
        check(host(got[k]).reshape(ref[k].shape), ref[k], 2e-4, what=f"test_scan_bwd_parity {k}")


# ------------------------------------------------------------------ mixer backward (STE)

MIXER_BWD_CASES = [  # (workload, batch, seqlen, residual, latents, gains)
    ("bitssm_tiny", 2, 64, True, True, False),
    ("bitssm_tiny", 1, 37, False, False, True),   # ragged time (one partial scan chunk), RMSNorm gains
    ("bitssm_tiny", 3, 5, True, True, True),      # shorter than one time chunk
    ("trissm", 2, 256, True, True, False),         # TriSSM width and length
    ("trissm", 64, 256, True, True, False),        # the full TriSSM training batch (64 x 256 tokens)
]


def _ds_bound(dw, codes, scale, w_lat):
    """Sum of the magnitudes of the scale gradient's terms (it sums terms of both signs)."""
    v = np.asarray(w_lat, np.float64) / float(np.asarray(scale).ravel()[0])
    fac = np.where(np.abs(v) <= 1.0, codes - v, codes)
    return float(np.abs(np.asarray(dw, np.float64) * fac).sum())


@pytest.mark.parametrize("name,batch,seqlen,residual,latents,gains", MIXER_BWD_CASES)
def test_mixer_bwd_parity(name, batch, seqlen, residual, latents, gains):
    """Backward of one Mamba-1 kind mixer layer under the straight-through estimators (forward
    evaluated again, then out_proj, scan, dt_proj, x_proj and in_proj backwards) against the
    oracle's fp64 chain: every gradient norm-wise to 5e-4 (fp32 intermediates on the GPU; an
    activation code that the forward's last-ulp differences move by one step shifts the result by
    about 1e-5), the scale gradients to 1e-4 of the sum of their terms' magnitudes."""
    cfg = wl.CONFIGS[name].with_(batch=batch, seqlen=seqlen, layers=1)
    lat, u = wl.mixer_problem(cfg, seed=batch + seqlen)
    gw, ow = quantize_layer(cfg, lat[0])
    if gains:
        g = wl.rng(seqlen)
        for pname, (_, k) in cfg.proj_shapes.items():
            gv = (1.0 + 0.2 * wl.normal(g, (k,))).astype(np.float32)
            gw["g_" + pname], ow["g_" + pname] = to_dev(gv), gv
    dout = wl.normal(wl.rng(batch * seqlen), u.shape)
    lats = {"lat_" + p: lat[0]["W_" + p] for p in cfg.proj_shapes} if latents else None
    got = tws.ssm_mixer_bwd(gpu_config(cfg), gw, to_dev(u), to_dev(dout), add_residual=residual,
                            latents={k: to_dev(v) for k, v in lats.items()} if latents else None)
    ref = oracle.mixer_bwd(oracle_config(cfg), ow, u, dout, residual=residual, latents=lats)
    for k in ("du", "dw_in", "dw_x", "dw_dt", "dw_out", "dA", "dD", "d_dt_bias"):
        check(host(got[k]).reshape(np.shape(ref[k])), ref[k], 5e-4, what=f"test_mixer_bwd_parity {name} {batch} {k}",
              elem=5e-3, frac=5e-3)
    if latents:
        for p in cfg.proj_shapes:
            bound = _ds_bound(ref["dw_" + p], ow["c_" + p], ow["s_" + p], lats["lat_" + p])
            assert abs(float(host(got["ds_" + p])[0]) - float(ref["ds_" + p][0])) <= 1e-4 * bound, p


def test_mixer_bwd_empty_and_repeatable():
    """No tokens: nothing is written and the call succeeds; two calls give identical gradients
    (fixed summation order)."""
    cfg = wl.CONFIGS["bitssm_tiny"].with_(batch=2, seqlen=40)
    lat, u = wl.mixer_problem(cfg, seed=9)
    gw, _ = quantize_layer(cfg, lat[0])
    dout = wl.normal(wl.rng(10), u.shape)
    a = tws.ssm_mixer_bwd(gpu_config(cfg), gw, to_dev(u), to_dev(dout))
    b = tws.ssm_mixer_bwd(gpu_config(cfg), gw, to_dev(u), to_dev(dout))
    for k in a:
        np.testing.assert_array_equal(host(a[k]), host(b[k]), err_msg=k)
    e = tws.ssm_mixer_bwd(gpu_config(cfg), gw, to_dev(u[:, :0]), to_dev(dout[:, :0]))
    assert e["du"].shape == (2, 0, cfg.d_model)
