"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test names the passage or the mathematical fact it checks.  None of them
re-types the oracle's own formula: they use hand-worked fixtures, closed forms,
invariants, brute force, or an independent algorithm (numpy integer/fp64
contractions, the Blelloch tree, the state-space-duality quadratic form).
"""
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(":")
            rows = [r.split() for r in rest.split(";")]
            vals[key.strip()] = rows
    return vals


def _ints(rows, base=10):
    return np.array([[int(v, base) for v in r] for r in rows])


def _floats(rows):
    return np.array([[float(v) for v in r] for r in rows], dtype=np.float32)


# ------------------------------------------------------------------ O0: ternary weights

def test_ternary_hand_examples():
    """Absmean scale and codes on hand-worked examples (tests/golden/ternary_examples.txt)."""
    g = _read_golden("ternary_examples.txt")
    w1 = _floats(g["W1"])
    codes, scale, zeros = oracle.quantize_weights(w1, 0)
    assert np.float32(scale[0]) == pytest.approx(0.19375, rel=1e-6)
    np.testing.assert_array_equal(codes, _ints(g["codes1"]))
    assert zeros == 2
    w2 = _floats(g["W2"])
    codes, scale, _ = oracle.quantize_weights(w2, 4)
    np.testing.assert_allclose(scale.ravel(), [0.225, 0.925], rtol=1e-6)
    np.testing.assert_array_equal(codes, _ints(g["codes2"]))
    codes, scale, _ = oracle.quantize_weights(_floats(g["W3"]), 0)
    assert scale[0] == 0.5
    np.testing.assert_array_equal(codes, _ints(g["codes3"]))


@pytest.mark.parametrize("shape,group", [((512, 256), 0), ((48, 512), 0), ((64, 512), 128), ((7, 384), 128)])
def test_ternary_set_membership_and_absmean(shape, group):
    """Codes lie in {-1,0,+1} (TriSSM README; TernarySSM Key Points) and the stored scale is
    mean|W| (BitNet b1.58 absmean), checked against an exactly rounded sum (math.fsum)."""
    w = wl.normal(wl.rng(3), shape, 0.0, 0.02)
    codes, scale, zeros = oracle.quantize_weights(w, group)
    assert set(np.unique(codes)).issubset({-1, 0, 1})
    assert zeros == int((codes == 0).sum())
    if group == 0:
        exact = np.float32(math.fsum(np.abs(w.astype(np.float64)).ravel()) / w.size)
        assert abs(float(scale[0]) - float(exact)) <= float(np.spacing(exact))
    else:
        for i in range(shape[0]):
            for gi in range(shape[1] // group):
                seg = np.abs(w[i, gi * group:(gi + 1) * group].astype(np.float64))
                exact = np.float32(math.fsum(seg) / group)
                assert abs(float(scale[i, gi]) - float(exact)) <= float(np.spacing(exact))


def test_ternary_codes_are_nearest_level():
    """Each code is the nearest of {-1,0,+1} to w/gamma (decided in fp64 away from the
    0.5 boundary): the definition of round-then-clamp."""
    w = wl.normal(wl.rng(4), (256, 256), 0.0, 0.02)
    codes, scale, _ = oracle.quantize_weights(w, 0)
    r = w.astype(np.float64) / float(scale[0])
    far = np.abs(np.abs(r) - 0.5) > 1e-5
    expect = np.where(r > 0.5, 1, np.where(r < -0.5, -1, 0))
    np.testing.assert_array_equal(codes[far], expect[far])


def test_ternary_sign_symmetry():
    """quantise(-W) = -codes with the same scale (round-half-even is odd-symmetric)."""
    w = wl.normal(wl.rng(5), (64, 128), 0.0, 0.02)
    c1, s1, _ = oracle.quantize_weights(w, 0)
    c2, s2, _ = oracle.quantize_weights(-w, 0)
    np.testing.assert_array_equal(c2, -c1)
    assert s1[0] == s2[0]


@pytest.mark.parametrize("j", [-3, 1, 4])
def test_ternary_power_of_two_invariance(j):
    """quantise(2^j W): same codes, scale * 2^j exactly (binary scaling is exact)."""
    w = wl.normal(wl.rng(6), (64, 256), 0.0, 0.02)
    for group in (0, 128):
        c1, s1, _ = oracle.quantize_weights(w, group)
        c2, s2, _ = oracle.quantize_weights(np.ldexp(w, j).astype(np.float32), group)
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(np.ldexp(s1, j).astype(np.float32), s2)


def test_ternary_gaussian_zero_ratio():
    """Zero ratio (named in the Ternary Mamba abstract) of Gaussian weights: a code is 0
    iff |w| < gamma/2 with gamma = sigma sqrt(2/pi), so the ratio is erf(sqrt(2/pi)/2/sqrt 2)
    = 0.3101.  131,072 weights (an in_proj of the TriSSM shape): binomial sigma 0.0013."""
    expect = math.erf(math.sqrt(2.0 / math.pi) / 2.0 / math.sqrt(2.0))
    assert expect == pytest.approx(0.3101, abs=1e-4)
    w = wl.normal(wl.rng(7), (512, 256), 0.0, 0.02)
    _, _, zeros = oracle.quantize_weights(w, 0)
    assert abs(zeros / w.size - expect) < 0.006


def test_ternary_group_equals_tensor_on_slices():
    """A per-group scale is the per-tensor rule applied to each (row, group) slice."""
    g = wl.rng(8)
    w = wl.normal(g, (5, 512), 0.0, 0.02) * np.repeat(
        np.array([0.1, 1.0, 10.0, 3.0], np.float32), 128)[None, :]
    w = w.astype(np.float32)
    codes, scale, _ = oracle.quantize_weights(w, 128)
    for i in range(5):
        for gi in range(4):
            sl = np.ascontiguousarray(w[i:i + 1, gi * 128:(gi + 1) * 128])
            c, s, _ = oracle.quantize_weights(sl, 0)
            assert s[0] == scale[i, gi]
            np.testing.assert_array_equal(c[0], codes[i, gi * 128:(gi + 1) * 128])


def test_ternary_zero_tensor_and_caller_scale():
    """All-zero weights: scale 0 and all codes 0 (the 1e-5 floor guards the division).
    A caller-supplied scale (learned scales, Ternary Mamba abstract) is used as given."""
    codes, scale, zeros = oracle.quantize_weights(np.zeros((4, 16), np.float32), 0)
    assert scale[0] == 0.0 and zeros == 64 and not codes.any()
    w = np.array([[0.5, -0.5, 0.26, -0.24]], np.float32)
    codes, scale, _ = oracle.quantize_weights(w, 0, scale_in=np.array([0.5], np.float32))
    np.testing.assert_array_equal(codes, [[1, -1, 1, 0]])  # 0.52 -> 1, -0.48 -> 0


def test_pack_golden_word():
    """Packed bytes of a fixed 16-weight word and of a k = 8 row (tests/golden/pack_word.txt)."""
    g = _read_golden("pack_word.txt")
    codes = _ints(g["codes"]).astype(np.int8)
    np.testing.assert_array_equal(oracle.pack(codes)[0], _ints(g["bytes"], 16)[0])
    codes8 = _ints(g["codes8"]).astype(np.int8)
    assert oracle.packed_row_bytes(8) == 4
    np.testing.assert_array_equal(oracle.pack(codes8)[0], _ints(g["bytes8"], 16)[0])


@pytest.mark.parametrize("n,k", [(1, 1), (3, 8), (5, 16), (7, 40), (64, 512), (4416, 32)])
def test_pack_roundtrip_and_size(n, k):
    """unpack(pack(q)) = q; n * 4 * ceil(k/16) bytes; the unused code 0b10 never appears."""
    q = wl.rng(9).integers(-1, 2, size=(n, k)).astype(np.int8)
    p = oracle.pack(q)
    assert p.shape == (n, 4 * ((k + 15) // 16))
    back, bad = oracle.unpack(p, k)
    assert bad == 0
    np.testing.assert_array_equal(back, q)
    # 2 bits per weight: the packed tensor is 1/16 the size of the fp32 latent weights
    if k % 16 == 0:
        assert p.nbytes * 16 == q.size * 4


# ------------------------------------------------------------------ O1/O2: RMSNorm + absmax int8

def test_act_quant_hand_examples():
    """RMSNorm + absmax int8 codes on hand-worked rows (tests/golden/act_quant_examples.txt)."""
    g = _read_golden("act_quant_examples.txt")
    for vk, qk in (("v1", "q1"), ("v2", "q2")):
        v = _floats(g[vk])[0]
        q, m = oracle.quant_row(oracle.norm_row(v))
        np.testing.assert_array_equal(q, _ints(g[qk])[0])


@pytest.mark.parametrize("k", [1, 8, 16, 63, 64, 65, 256, 1000, 4096])
def test_rms_scale_error_bound(k):
    """1/sqrt(mean v^2 + eps) to within fp32 rounding of the exact (fsum) value."""
    v = wl.normal(wl.rng(10 + k), (k,))
    exact = 1.0 / math.sqrt(math.fsum(float(a) * float(a) for a in v) / k + 1e-5)
    r = float(oracle.rms_scale(v, 1e-5))
    # k fp32 additions, a division, sqrt, a division: a few ulp plus k*2^-24 of the sum
    assert abs(r - exact) / exact < (4 + k) * 2.0 ** -24


def test_rms_scale_exact_on_integers():
    """Small-integer rows sum exactly in any order, so the fp32 result is exactly
    1 / sqrt(S/k + eps) evaluated in fp32 (order cannot matter)."""
    v = np.array([(i % 7) - 3 for i in range(200)], np.float32)
    S = np.float32(sum(int(a) * int(a) for a in v))
    expect = np.float32(1.0) / np.sqrt(S / np.float32(200) + np.float32(1e-5))
    assert oracle.rms_scale(v, 1e-5) == expect


def test_act_quant_properties():
    """For 2,300 random fp32 tokens (K = 64..512): max|q| = 127 exactly, |xh - q/sigma| <= 0.5/sigma,
    quant(-x) = -quant(x), and eps = 0 gives exact power-of-two invariance of the codes."""
    g = wl.rng(11)
    for k in (64, 100, 512):
        rows = wl.normal(g, (300 if k == 512 else 1000, k)) * np.exp(g.uniform(-4, 4, (1, 1))).astype(np.float32)
        for v in rows:
            xh = oracle.norm_row(v)
            q, m = oracle.quant_row(xh)
            assert np.abs(q).max() == 127
            sigma = np.float32(127.0) / max(m, np.float32(1e-5))
            # |xh*sigma - q| <= 1/2 plus the fp32 rounding of the product (<= 128 * 2^-24)
            assert np.all(np.abs(xh.astype(np.float64) - q / float(sigma)) <= (0.5 + 2.0 ** -17) / float(sigma))
            qn, _ = oracle.quant_row(oracle.norm_row(-v))
            np.testing.assert_array_equal(qn, -q)
        for v in rows[:50]:
            q1, _ = oracle.quant_row(oracle.norm_row(v, eps=0.0))
            q2, _ = oracle.quant_row(oracle.norm_row(np.ldexp(v, 3).astype(np.float32), eps=0.0))
            np.testing.assert_array_equal(q1, q2)


def test_act_quant_degenerate_rows():
    """All-zero token: absmax 0, codes 0.  One-hot token: the hot element gets 127, others 0."""
    q, m = oracle.quant_row(oracle.norm_row(np.zeros(64, np.float32)))
    assert m == 0.0 and not q.any()
    v = np.zeros(256, np.float32)
    v[17] = -3.5
    q, m = oracle.quant_row(oracle.norm_row(v))
    assert q[17] == -127 and np.count_nonzero(q) == 1
    assert m == pytest.approx(3.5 / math.sqrt(3.5 ** 2 / 256 + 1e-5), rel=1e-6)


def test_norm_gain():
    """Gains multiply the normalised row elementwise: gains of 2 double xh exactly."""
    v = wl.normal(wl.rng(12), (96,))
    a = oracle.norm_row(v)
    b = oracle.norm_row(v, g=np.full(96, 2.0, np.float32))
    np.testing.assert_array_equal(b, 2 * a)


# ------------------------------------------------------------------ O3/O4: BitLinear

def test_multiply_free_identity_exhaustive():
    """TernarySSM abstract: ternary weights make the contraction add / subtract / skip.
    All 3^4 ternary rows against 64 int8 vectors at K = 4: acc = sum_{w=+1} q - sum_{w=-1} q."""
    rows = np.array(np.meshgrid(*[[-1, 0, 1]] * 4, indexing="ij")).reshape(4, -1).T.astype(np.int8)
    g = wl.rng(13)
    xs = g.integers(-128, 128, size=(64, 4))
    xs[0] = 127
    xs[1] = -128
    for x in xs:
        # rows of v whose codes are all int8 and whose normalised absmax hits 127 on
        # the largest element: feed integer vectors scaled so quantisation is the identity
        # is not possible in general, so check the identity on the accumulators directly
        add = np.where(rows == 1, x[None, :], 0).sum(1)
        sub = np.where(rows == -1, x[None, :], 0).sum(1)
        np.testing.assert_array_equal(add - sub, rows.astype(np.int64) @ x)
    # and through the oracle's BitLinear: accumulators equal the add/sub/skip sums of its codes
    v = wl.normal(g, (64, 4))
    _, xq, _, acc = oracle.bitlinear(v, rows, np.array([0.02], np.float32))
    add = np.where(rows[None, :, :] == 1, xq[:, None, :].astype(np.int64), 0).sum(2)
    sub = np.where(rows[None, :, :] == -1, xq[:, None, :].astype(np.int64), 0).sum(2)
    np.testing.assert_array_equal(acc, add - sub)


@pytest.mark.parametrize("m,k,n,group", [(37, 256, 48, 0), (16, 8, 128, 0), (9, 512, 64, 128), (5, 1024, 40, 0)])
def test_bitlinear_a8_vs_numpy(m, k, n, group):
    """A8 BitLinear: int8 codes of each row equal the row-wise quantiser; int32
    accumulators equal an int64 numpy matmul of (codes x weight codes); |acc| <= 127 k;
    dequantised output within the quantisation bound of the fp64 unquantised product."""
    g = wl.rng(14)
    x = wl.normal(g, (m, k))
    w = wl.normal(g, (n, k), 0.0, 0.02)
    codes, scale, _ = oracle.quantize_weights(w, group)
    bias = wl.normal(g, (n,))
    y, xq, am, acc = oracle.bitlinear(x, codes, scale, group, 8, bias=bias)
    for i in range(m):
        q, mm = oracle.quant_row(oracle.norm_row(x[i]))
        np.testing.assert_array_equal(xq[i], q)
        assert am[i] == mm
    ref_acc = xq.astype(np.int64) @ codes.astype(np.int64).T
    np.testing.assert_array_equal(acc, ref_acc)
    assert np.abs(acc).max() <= 127 * k
    # dequant: y - bias = s * acc * max(m)/127 per group
    deq = np.maximum(am.astype(np.float64), 1e-5) / 127.0
    if group == 0:
        ref = acc * float(scale[0]) * deq[:, None]
        sw = np.full((n, 1), float(scale[0]))
        wf = codes.astype(np.float64) * float(scale[0])
    else:
        ng = k // group
        ref = np.zeros((m, n))
        for gi in range(ng):
            a = xq[:, gi * group:(gi + 1) * group].astype(np.int64) @ codes[:, gi * group:(gi + 1) * group].astype(np.int64).T
            ref += a * scale[:, gi].astype(np.float64)[None, :]
        ref *= deq[:, None]
        wf = codes.astype(np.float64) * np.repeat(scale.astype(np.float64), group, axis=1)
    np.testing.assert_allclose(y - bias.astype(np.float64), ref, rtol=1e-12, atol=1e-12)
    # quantisation error bound against the unquantised product s * W . xh
    xh = np.stack([oracle.norm_row(x[i]) for i in range(m)]).astype(np.float64)
    exact = xh @ wf.T
    sigma = 127.0 / np.maximum(am.astype(np.float64), 1e-5)
    bound = (np.abs(wf).sum(1)[None, :] * (0.5 / sigma)[:, None]) * (1 + 1e-5) + 1e-12
    assert np.all(np.abs((y - bias) - exact) <= bound)


@pytest.mark.parametrize("group", [0, 128])
def test_bitlinear_a16_vs_numpy(group):
    """A16 (W1.58A16, Ternary Mamba abstract): unquantised normalised activations times
    per-group-scaled ternary weights, against an fp64 numpy matmul."""
    g = wl.rng(15)
    m, k, n = 23, 512, 72
    x = wl.normal(g, (m, k))
    w = wl.normal(g, (n, k), 0.0, 0.02)
    codes, scale, _ = oracle.quantize_weights(w, group)
    y, *_ = oracle.bitlinear(x, codes, scale, group, 16)
    xh = np.stack([oracle.norm_row(x[i]) for i in range(m)]).astype(np.float64)
    if group == 0:
        wf = codes * float(scale[0])
    else:
        wf = codes * np.repeat(scale.astype(np.float64), group, axis=1)
    np.testing.assert_allclose(y, xh @ wf.T, rtol=1e-12, atol=1e-12)


def test_bitlinear_strided_input():
    """A row stride wider than k reads the first k columns only (the dt projection reads
    the first dt_rank columns of the x_proj output)."""
    g = wl.rng(16)
    wide = wl.normal(g, (11, 48))
    codes, scale, _ = oracle.quantize_weights(wl.normal(g, (64, 16), 0, 0.02), 0)
    y1, *_ = oracle.bitlinear(wide, codes, scale, k=16)
    y2, *_ = oracle.bitlinear(np.ascontiguousarray(wide[:, :16]), codes, scale)
    np.testing.assert_array_equal(y1, y2)


# ------------------------------------------------------------------ O5-O7: selective scan

def _scan(p, **kw):
    return oracle.selective_scan(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p.get("D"),
                                 p.get("dt_bias"), **kw)


@pytest.mark.parametrize("H,P,N,aps,L", [(6, 1, 16, True, 37), (3, 4, 8, False, 64), (2, 1, 4, True, 1)])
def test_scan_parallel_equals_sequential(H, P, N, aps, L):
    """TriSSM README / TernarySSM abstract: the recurrence is evaluated with a parallel
    associative scan; the Blelloch tree over (a, b) pairs equals the sequential loop."""
    p = wl.scan_problem(2, L, H, P, N, aps, seed=17)
    h0 = wl.normal(wl.rng(18), (2, H, P, N))
    y1, h1 = _scan(p, h0=h0)
    y2, h2 = _scan(p, h0=h0, method="blelloch")
    np.testing.assert_allclose(y2, y1, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(h2, h1, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("aps", [True, False])
def test_scan_quadratic_form(aps):
    """State space duality ("Transformers are SSMs", cited by SSDi8): the masked quadratic
    form sum_{s<=t} (C_t . B_s) exp(A sum_{s<r<=t} dt_r) dt_s x_s + D x_t equals the recurrence."""
    H, P = (5, 1) if aps else (3, 4)
    p = wl.scan_problem(2, 40, H, P, 8, aps, seed=19)
    y1, _ = _scan(p)
    y2, _ = _scan(p, method="quadratic")
    np.testing.assert_allclose(y1, y2, rtol=1e-10, atol=1e-10)


def test_scan_zero_B():
    """B = 0: no input reaches the state, y = D x exactly."""
    p = wl.scan_problem(2, 30, 4, 1, 16, True, seed=20)
    p["Bm"] = np.zeros_like(p["Bm"])
    y, h = _scan(p)
    np.testing.assert_array_equal(y, p["x"].astype(np.float64) * p["D"].astype(np.float64)[None, None, :])
    assert not h.any()


def test_scan_zero_A_is_prefix_sum():
    """A = 0: exp(dt A) = 1, so h_t = h0 + sum_{s<=t} dt_s x_s B_s (a cumulative sum)."""
    p = wl.scan_problem(1, 25, 3, 1, 4, True, seed=21)
    p["A"] = np.zeros_like(p["A"])
    h0 = wl.normal(wl.rng(22), (1, 3, 1, 4))
    y, h = _scan(p, h0=h0)
    dt = np.log1p(np.exp(p["delta"].astype(np.float64) + p["dt_bias"][None, None, :]))[0]  # [L, H]
    x = p["x"][0].astype(np.float64)
    B = p["Bm"][0].astype(np.float64)
    C = p["Cm"][0].astype(np.float64)
    hs = h0[0, :, 0, :][None] + np.cumsum((dt * x)[:, :, None] * B[:, None, :], axis=0)  # [L, H, N]
    yref = (hs * C[:, None, :]).sum(-1) + p["D"][None, :] * x
    np.testing.assert_allclose(y[0], yref, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(h[0, :, 0, :], hs[-1], rtol=1e-10)


def test_scan_fast_decay_limit():
    """Large dt with A = -1: exp(-dt) ~ 1e-22 forgets the past, so y_t = dt x_t (C_t.B_t) + D x_t."""
    p = wl.scan_problem(1, 20, 3, 1, 8, True, seed=23)
    p["A"] = -np.ones_like(p["A"])
    p["delta"] = np.full_like(p["delta"], 50.0)
    p["dt_bias"] = np.zeros_like(p["dt_bias"])
    y, _ = _scan(p)
    x = p["x"][0].astype(np.float64)
    cb = (p["Cm"][0].astype(np.float64) * p["Bm"][0]).sum(-1)
    yref = 50.0 * x * cb[:, None] + p["D"][None, :] * x
    np.testing.assert_allclose(y[0], yref, rtol=1e-12, atol=1e-12)


def test_scan_lti_convolution():
    """Constant dt, B, C over time (S4, cited by SSDi8): the map is a causal convolution with
    kernel K_j = sum_n C_n exp(dt A_n)^j dt B_n, checked against a direct O(L^2) convolution."""
    L, H, N = 48, 2, 6
    p = wl.scan_problem(1, L, H, 1, N, True, seed=24)
    g = wl.rng(25)
    for key in ("delta", "Bm", "Cm"):
        p[key] = np.repeat(p[key][:, :1, :], L, axis=1)
    y, _ = _scan(p)
    dt = np.log1p(np.exp(p["delta"][0, 0].astype(np.float64) + p["dt_bias"]))  # [H]
    B = p["Bm"][0, 0].astype(np.float64)
    C = p["Cm"][0, 0].astype(np.float64)
    x = p["x"][0].astype(np.float64)
    for hd in range(H):
        a = np.exp(dt[hd] * p["A"][hd].astype(np.float64))  # [N]
        kern = np.array([(C * a ** j * dt[hd] * B).sum() for j in range(L)])
        conv = np.array([sum(kern[t - s] * x[s, hd] for s in range(t + 1)) for t in range(L)])
        np.testing.assert_allclose(y[0, :, hd], conv + p["D"][hd] * x[:, hd], rtol=1e-10, atol=1e-12)
    del g


def test_scan_first_order_iir_by_hand():
    """One channel, one state, L = 3, no softplus: the first-order IIR unrolled by hand."""
    x = np.array([1.0, 2.0, -1.0], np.float32).reshape(1, 3, 1)
    dt = np.array([0.5, 1.0, 0.25], np.float32).reshape(1, 3, 1)
    B = np.array([1.0, 1.0, 2.0], np.float32).reshape(1, 3, 1)
    C = np.array([1.0, 0.5, 1.0], np.float32).reshape(1, 3, 1)
    A = np.array([[-2.0]], np.float32)
    D = np.array([0.1], np.float32)
    y, h = oracle.selective_scan(x, dt, A, B, C, D, None, softplus=False)
    h1 = 0.5 * 1 * 1
    h2 = math.exp(-2.0) * h1 + 1.0 * 2 * 1
    h3 = math.exp(-0.5) * h2 + 0.25 * -1 * 2
    d = float(D[0])  # 0.1 as stored in fp32
    np.testing.assert_allclose(y.ravel(), [h1 + d, 0.5 * h2 + 2 * d, h3 - d], rtol=1e-14)
    assert h.ravel()[0] == pytest.approx(h3, rel=1e-14)


def test_softplus():
    """softplus(0) = ln 2; identity above 20; log(1 + e^v) below (Mamba's dt activation)."""
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    assert oracle.softplus(25.0) == 25.0
    assert oracle.softplus(-3.0) == pytest.approx(math.log1p(math.exp(-3.0)), rel=1e-15)
    assert oracle.softplus(19.9) == pytest.approx(19.9 + math.log1p(math.exp(-19.9)), rel=1e-15)


def test_scan_causality_and_streaming():
    """Perturbing token t leaves y before t bitwise unchanged; a scan of L equals a scan of
    L1 followed by a scan of L - L1 started from the carried state (to fp32 state rounding)."""
    p = wl.scan_problem(2, 50, 4, 2, 8, False, seed=26)
    y, h = _scan(p)
    q = {k: v.copy() for k, v in p.items()}
    q["x"][:, 30] += 1.0
    q["delta"][:, 30] -= 0.7
    q["Bm"][:, 30] *= 2
    y2, _ = _scan(q)
    np.testing.assert_array_equal(y2[:, :30], y[:, :30])
    assert not np.array_equal(y2[:, 30], y[:, 30])
    a = {k: (v[:, :20] if v.ndim == 3 else v) for k, v in p.items()}
    b = {k: (v[:, 20:] if v.ndim == 3 else v) for k, v in p.items()}
    ya, ha = _scan(a)
    yb, hb = _scan(b, h0=ha.astype(np.float32))
    np.testing.assert_allclose(np.concatenate([ya, yb], 1), y, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(hb, h, rtol=1e-6, atol=1e-6)


# ------------------------------------------------------------------ mixer composition

def _layer_codes(cfg, lat):
    out = {"dt_bias": lat["dt_bias"], "A": lat["A"], "D": lat["D"]}
    for name in cfg.proj_shapes:
        c, s, _ = oracle.quantize_weights(lat["W_" + name], cfg.group_size)
        out["c_" + name] = c
        out["s_" + name] = s
    return out


def _cfg_dict(cfg):
    return dict(kind=cfg.kind, d_model=cfg.d_model, d_inner=cfg.d_inner, d_state=cfg.d_state, dt_rank=cfg.dt_rank,
                nheads=cfg.nheads, headdim=cfg.headdim, group_size=cfg.group_size, act_bits=cfg.act_bits,
                act_dtype=oracle.BF16 if cfg.act_dtype == "bf16" else oracle.F32, norm_eps=cfg.norm_eps)


def test_mixer_mamba1_composition():
    """TriSSM README: RMSNorm -> ternary BitLinear for the Delta, B, C projections, then the
    scan.  The oracle mixer equals the composition of the separately pinned stages."""
    cfg = wl.CONFIGS["bitssm_tiny"]
    lat, u = wl.mixer_problem(cfg, seed=42)
    w = _layer_codes(cfg, lat[0])
    out = oracle.mixer(_cfg_dict(cfg), w, u)
    M = cfg.tokens
    uu = u.reshape(M, -1)
    x, *_ = oracle.bitlinear(uu, w["c_in"], w["s_in"])
    x = x.astype(np.float32)
    p, *_ = oracle.bitlinear(x, w["c_x"], w["s_x"])
    p = p.astype(np.float32)
    R, N = cfg.dt_rank, cfg.d_state
    z, *_ = oracle.bitlinear(p, w["c_dt"], w["s_dt"], k=R)
    B = p[:, R:R + N].reshape(cfg.batch, cfg.seqlen, N)
    C = p[:, R + N:].reshape(cfg.batch, cfg.seqlen, N)
    y, _ = oracle.selective_scan(x.reshape(cfg.batch, cfg.seqlen, -1), z.astype(np.float32).reshape(cfg.batch, cfg.seqlen, -1),
                                 w["A"], B, C, w["D"], w["dt_bias"])
    o, *_ = oracle.bitlinear(y.astype(np.float32).reshape(M, -1), w["c_out"], w["s_out"])
    ref = (o + uu).astype(np.float32).astype(np.float64).reshape(out.shape)
    np.testing.assert_array_equal(out, ref)


def test_mixer_ssd_composition():
    """Ternary Mamba abstract (W1.58A16, grouped scales) on an SSD-shaped mixer: in_proj
    columns [x | B | C | dt], scalar A per head; equals the composition of pinned stages."""
    cfg = wl.CONFIGS["mamba2_ssd"].with_(d_model=256, d_inner=256, d_state=16, nheads=4, headdim=64, batch=2,
                                          seqlen=24, act_dtype="f32")
    lat, u = wl.mixer_problem(cfg, seed=42)
    w = _layer_codes(cfg, lat[0])
    out = oracle.mixer(_cfg_dict(cfg), w, u, residual=False)
    M, H, P, N = cfg.tokens, cfg.nheads, cfg.headdim, cfg.d_state
    v, *_ = oracle.bitlinear(u.reshape(M, -1), w["c_in"], w["s_in"], 128, 16)
    v = v.astype(np.float32)
    sh = (cfg.batch, cfg.seqlen)
    y, _ = oracle.selective_scan(v[:, :H * P].reshape(*sh, -1), v[:, H * P + 2 * N:].reshape(*sh, -1), w["A"],
                                 v[:, H * P:H * P + N].reshape(*sh, -1), v[:, H * P + N:H * P + 2 * N].reshape(*sh, -1),
                                 w["D"], w["dt_bias"])
    o, *_ = oracle.bitlinear(y.astype(np.float32).reshape(M, -1), w["c_out"], w["s_out"], 128, 16)
    np.testing.assert_array_equal(out, o.astype(np.float32).astype(np.float64).reshape(out.shape))


def test_mixer_stack_composition():
    """A stack of residual mixer layers (the TriSSM README's 12-layer selective SSM) is the
    layers applied in order, each to the previous layer's stored output: two layers equal two
    explicit mixer calls, in that order (the reversed order differs); with every out_proj code
    zero each layer is the identity, so a stack of them returns u exactly."""
    cfg = wl.CONFIGS["bitssm_tiny"]
    lat, u = wl.mixer_problem(cfg, seed=45, layers=2)
    w1, w2 = _layer_codes(cfg, lat[0]), _layer_codes(cfg, lat[1])
    oc = _cfg_dict(cfg)
    got = oracle.mixer_stack(oc, [w1, w2], u)
    h1 = oracle.mixer(oc, w1, u, residual=True).astype(np.float32)
    np.testing.assert_array_equal(got, oracle.mixer(oc, w2, h1, residual=True))
    rev = oracle.mixer(oc, w1, oracle.mixer(oc, w2, u, residual=True).astype(np.float32), residual=True)
    assert not np.array_equal(got, rev)
    zero = [dict(w, c_out=np.zeros_like(w["c_out"])) for w in (w1, w2, w1)]
    np.testing.assert_array_equal(oracle.mixer_stack(oc, zero, u), u.astype(np.float64))


def test_mixer_causality():
    """TriSSM README tests list causality: perturbing token t of u leaves every output before
    t bitwise unchanged (oracle, Mamba-1 and SSD kinds)."""
    for cfg in (wl.CONFIGS["bitssm_tiny"],
                wl.CONFIGS["mamba2_ssd"].with_(d_model=128, d_inner=128, d_state=16, nheads=2, headdim=64,
                                               batch=1, seqlen=32)):
        lat, u = wl.mixer_problem(cfg, seed=43)
        w = _layer_codes(cfg, lat[0])
        if cfg.act_dtype == "bf16":
            u = oracle.round_bf16(u)
        out = oracle.mixer(_cfg_dict(cfg), w, u)
        u2 = u.copy()
        u2[:, 20] = -u2[:, 20] + 0.5
        out2 = oracle.mixer(_cfg_dict(cfg), w, u2)
        np.testing.assert_array_equal(out2[:, :20], out[:, :20])
        assert not np.array_equal(out2[:, 20], out[:, 20])


def test_round_bf16():
    """bf16 rounding: nearest, ties to even, against values with a known bf16 neighbourhood."""
    one = 1.0
    ulp = 2.0 ** -7
    vals = np.array([one, one + ulp / 2, one + ulp * 1.5, one + ulp / 4, -(one + ulp * 0.75), 3.0e-39], np.float32)
    got = oracle.round_bf16(vals)
    np.testing.assert_array_equal(got[:5], np.array([one, one, one + 2 * ulp, one, -(one + ulp)], np.float32))
    assert got[5] == pytest.approx(3.0e-39, rel=2 ** -7)


# ------------------------------------------------------------------ gated block (conv + SiLU gate)

def _silu_tanh(a):
    """SiLU through library routines, not the oracle's form: a * expit(a) (scipy's logistic
    sigmoid); on |a| <= 8 also checked against the identity a (1 + tanh(a / 2)) / 2."""
    a = np.asarray(a, dtype=np.float64)
    return a * expit(a)


def test_silu_values():
    """SiLU: silu(0) = 0, silu(a) - silu(-a) = a, sigmoid(1) = e / (1 + e), and the tanh form."""
    assert oracle.silu(0.0) == 0.0
    for a in (0.3, 1.0, 2.5, 7.0, 19.0):
        assert abs((oracle.silu(a) - oracle.silu(-a)) - a) <= 4e-16 * max(1.0, a)
    assert oracle.silu(1.0) == pytest.approx(math.e / (1.0 + math.e), rel=1e-15)
    for a in np.linspace(-30.0, 30.0, 121):
        assert oracle.silu(float(a)) == pytest.approx(float(_silu_tanh(a)), rel=1e-13, abs=1e-300)
        if abs(a) <= 8.0:
            assert oracle.silu(float(a)) == pytest.approx(float(a * (1.0 + math.tanh(a / 2.0)) / 2.0), rel=1e-12)
    assert oracle.silu(-800.0) == 0.0  # exp overflow: the product underflows to zero


def _conv_ref(x, w, bias, state=None):
    """Brute force through numpy's full convolution, per (sequence, channel), fp64."""
    batch, L, _ = x.shape
    C, K = w.shape
    out = np.zeros((batch, L, C))
    for b in range(batch):
        for c in range(C):
            seq = x[b, :, c].astype(np.float64)
            pre = np.zeros(K - 1) if state is None else state[b, :, c].astype(np.float64)
            full = np.convolve(np.concatenate([pre, seq]), w[c, ::-1].astype(np.float64))
            out[b, :, c] = full[K - 1:K - 1 + L] + (0.0 if bias is None else float(bias[c]))
    return _silu_tanh(out)


@pytest.mark.parametrize("K", [1, 2, 4])
def test_conv_silu_vs_numpy_convolve(K):
    g = wl.rng(5 + K)
    x = wl.normal(g, (2, 37, 24))
    w = wl.normal(g, (20, K), 0.0, 0.5)
    bias = wl.normal(g, (20,), 0.0, 0.2)
    out, _ = oracle.conv_silu(x, w, bias)
    ref = _conv_ref(x[:, :, :20], w, bias)
    np.testing.assert_allclose(out, ref, rtol=2 ** -23, atol=1e-30)
    assert out.dtype == np.float32


def test_conv_silu_taps_direction():
    """A one-hot kernel at the last tap is SiLU of the current input; at the first tap it is
    SiLU of the input K - 1 steps back, with zeros (SiLU(0) = 0) before the sequence starts."""
    g = wl.rng(11)
    x = wl.normal(g, (1, 9, 3))
    K = 4
    w_now = np.zeros((3, K), np.float32)
    w_now[:, K - 1] = 1.0
    out, _ = oracle.conv_silu(x, w_now)
    np.testing.assert_allclose(out, _silu_tanh(x), rtol=2 ** -23)
    w_old = np.zeros((3, K), np.float32)
    w_old[:, 0] = 1.0
    out, _ = oracle.conv_silu(x, w_old)
    assert np.all(out[:, :K - 1] == 0.0)
    np.testing.assert_allclose(out[:, K - 1:], _silu_tanh(x[:, :-(K - 1)]), rtol=2 ** -23)


def test_conv_silu_streaming_state():
    """Splitting a sequence and carrying the state gives the same values bit for bit; the
    state after a sequence is its last K - 1 inputs."""
    g = wl.rng(12)
    x = wl.normal(g, (2, 30, 8))
    w = wl.normal(g, (8, 4), 0.0, 0.5)
    bias = wl.normal(g, (8,), 0.0, 0.2)
    full, st_full = oracle.conv_silu(x, w, bias)
    a, st_a = oracle.conv_silu(x[:, :11], w, bias)
    b, st_b = oracle.conv_silu(x[:, 11:], w, bias, state=st_a)
    np.testing.assert_array_equal(np.concatenate([a, b], axis=1), full)
    np.testing.assert_array_equal(st_b, st_full)
    np.testing.assert_array_equal(st_full, x[:, -3:])
    # a short piece (fewer inputs than K - 1) shifts the old state
    c, st_c = oracle.conv_silu(x[:, 11:13], w, bias, state=st_a)
    np.testing.assert_array_equal(st_c, np.concatenate([st_a[:, 2:], x[:, 11:13]], axis=1))
    np.testing.assert_array_equal(c, full[:, 11:13])


def _gated_layer(cfg, seed):
    lat, u = wl.mixer_problem(cfg, seed=seed)
    w = _layer_codes(cfg, lat[0])
    w["conv_w"], w["conv_b"] = lat[0]["conv_w"], lat[0]["conv_b"]
    return w, u


def _gated_cfg_dict(cfg):
    d = _cfg_dict(cfg)
    d.update(gated=cfg.gated, d_conv=cfg.d_conv)
    return d


GATED_SMALL = {
    "mamba1": wl.CONFIGS["bitssm_tiny"].with_(gated=1, d_conv=4, seqlen=24),
    "ssd": wl.CONFIGS["mamba2_ssd_gated"].with_(d_model=128, d_inner=128, d_state=16, nheads=2, headdim=64,
                                                  batch=2, seqlen=20, act_dtype="f32"),
}


@pytest.mark.parametrize("kind", ["mamba1", "ssd"])
def test_mixer_gated_zero_gate_is_identity(kind):
    """Gate rows of W_in all zero: SiLU(0) = 0 zeroes the scan output, out_proj of a zero row is
    zero, so the layer returns u exactly -- the gate acts between the scan and out_proj."""
    cfg = GATED_SMALL[kind]
    w, u = _gated_layer(cfg, 21)
    zg0 = w["c_in"].shape[0] - cfg.d_inner
    w["c_in"] = w["c_in"].copy()
    w["c_in"][zg0:] = 0
    out = oracle.mixer(_gated_cfg_dict(cfg), w, u)
    np.testing.assert_array_equal(out, u.astype(np.float64))
    # with the gate rows back, the layer is not the identity
    w2, _ = _gated_layer(cfg, 21)
    assert not np.array_equal(oracle.mixer(_gated_cfg_dict(cfg), w2, u), u.astype(np.float64))


@pytest.mark.parametrize("kind", ["mamba1", "ssd"])
def test_mixer_gated_zero_conv_is_identity(kind):
    """Convolution weights and bias zero: every SSM input (x; and B, C for SSD) is SiLU(0) = 0,
    so x_proj, the scan state, C h and D x all vanish and the layer returns u exactly -- the
    convolved values feed x_proj and the scan, including the D x term."""
    cfg = GATED_SMALL[kind]
    w, u = _gated_layer(cfg, 22)
    w["conv_w"] = np.zeros_like(w["conv_w"])
    w["conv_b"] = np.zeros_like(w["conv_b"])
    out = oracle.mixer(_gated_cfg_dict(cfg), w, u)
    np.testing.assert_array_equal(out, u.astype(np.float64))


@pytest.mark.parametrize("kind", ["mamba1", "ssd"])
def test_mixer_gated_delay_tap(kind):
    """Kernel one-hot at the oldest tap, no bias: the SSM sees inputs delayed by K - 1 steps and
    zeros before, so the first K - 1 outputs are u exactly and the K-th is not (causal order of
    the taps)."""
    cfg = GATED_SMALL[kind]
    w, u = _gated_layer(cfg, 23)
    K = cfg.d_conv
    cw = np.zeros_like(w["conv_w"])
    cw[:, 0] = 1.0
    w["conv_w"], w["conv_b"] = cw, np.zeros_like(w["conv_b"])
    out = oracle.mixer(_gated_cfg_dict(cfg), w, u)
    np.testing.assert_array_equal(out[:, :K - 1], u[:, :K - 1].astype(np.float64))
    assert not np.array_equal(out[:, K - 1], u[:, K - 1].astype(np.float64))


def test_mixer_gated_mamba1_composition():
    """The gated Mamba-1 layer equals in_proj -> [x | zg], conv + SiLU on x (pinned above), the
    ungated stages on the convolved x, the gate y * SiLU(zg) (tanh form here) and out_proj."""
    cfg = GATED_SMALL["mamba1"]
    w, u = _gated_layer(cfg, 24)
    out = oracle.mixer(_gated_cfg_dict(cfg), w, u)
    M, Di, R, N = cfg.tokens, cfg.d_inner, cfg.dt_rank, cfg.d_state
    sh = (cfg.batch, cfg.seqlen)
    uu = u.reshape(M, -1)
    xz, *_ = oracle.bitlinear(uu, w["c_in"], w["s_in"])
    xz = xz.astype(np.float32)
    xc, _ = oracle.conv_silu(xz[:, :Di].reshape(*sh, -1), w["conv_w"], w["conv_b"])
    xc = xc.reshape(M, Di)
    p, *_ = oracle.bitlinear(xc, w["c_x"], w["s_x"])
    p = p.astype(np.float32)
    z, *_ = oracle.bitlinear(p, w["c_dt"], w["s_dt"], k=R)
    y, _ = oracle.selective_scan(xc.reshape(*sh, -1), z.astype(np.float32).reshape(*sh, -1), w["A"],
                                 p[:, R:R + N].reshape(*sh, -1), p[:, R + N:].reshape(*sh, -1), w["D"], w["dt_bias"])
    yg = (y.reshape(M, Di) * _silu_tanh(xz[:, Di:])).astype(np.float32)
    o, *_ = oracle.bitlinear(yg, w["c_out"], w["s_out"])
    ref = (o + uu).astype(np.float32).astype(np.float64).reshape(out.shape)
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-6)


# ------------------------------------------------------------------ full-precision projections

def test_dense_vs_numpy():
    """A full-precision linear layer is x W^T: numpy's fp64 matmul, and a strided input."""
    g = wl.rng(31)
    x = wl.normal(g, (13, 40))
    W = wl.normal(g, (9, 24))
    y = oracle.dense(x, W, k=24)
    np.testing.assert_allclose(y, x[:, :24].astype(np.float64) @ W.T.astype(np.float64), rtol=1e-13, atol=1e-13)
    eye = np.eye(24, dtype=np.float32)
    np.testing.assert_array_equal(oracle.dense(x, eye, k=24), x[:, :24].astype(np.float64))


def _fp_layer(cfg, seed):
    lat, u = wl.mixer_problem(cfg, seed=seed)
    w = {"dt_bias": lat[0]["dt_bias"], "A": lat[0]["A"], "D": lat[0]["D"]}
    for name in cfg.proj_shapes:
        if cfg.is_fp(name):
            w["f_" + name] = lat[0]["W_" + name]
        else:
            c, s, _ = oracle.quantize_weights(lat[0]["W_" + name], cfg.group_size)
            w["c_" + name], w["s_" + name] = c, s
    return w, u


def _fp_cfg_dict(cfg):
    d = _cfg_dict(cfg)
    d["fp_proj"] = cfg.fp_proj
    return d


FP_SMALL = {
    "inout": wl.CONFIGS["trissm_fp_inout"].with_(d_model=64, d_inner=128, dt_rank=8, batch=2, seqlen=24, layers=1),
    "all": wl.CONFIGS["trissm_fp"].with_(d_model=64, d_inner=128, dt_rank=8, batch=2, seqlen=24, layers=1),
    "ssd": wl.CONFIGS["mamba2_ssd_fp"].with_(d_model=128, d_inner=128, d_state=16, nheads=2, headdim=64, batch=1,
                                             seqlen=20, act_dtype="f32", layers=1),
}


@pytest.mark.parametrize("mode", ["inout", "all", "ssd"])
def test_mixer_fp_zero_out_proj_is_identity(mode):
    """Full-precision out_proj weights zero: the layer returns u exactly (residual only)."""
    cfg = FP_SMALL[mode]
    w, u = _fp_layer(cfg, 41)
    w["f_out"] = np.zeros_like(w["f_out"])
    np.testing.assert_array_equal(oracle.mixer(_fp_cfg_dict(cfg), w, u), u.astype(np.float64))


@pytest.mark.parametrize("mode", ["inout", "all", "ssd"])
def test_mixer_fp_zero_in_proj_is_identity(mode):
    """Full-precision in_proj weights zero: x (and B, C for SSD) vanish, so C h and D x vanish and
    the layer returns u exactly -- in_proj feeds both x_proj and the scan."""
    cfg = FP_SMALL[mode]
    w, u = _fp_layer(cfg, 42)
    w["f_in"] = np.zeros_like(w["f_in"])
    np.testing.assert_array_equal(oracle.mixer(_fp_cfg_dict(cfg), w, u), u.astype(np.float64))


def test_mixer_fp_inout_composition():
    """TriSSM's split: x = u W_in^T (numpy), the ternary x_proj / dt / scan stages (pinned above),
    out = y W_out^T (numpy), + u."""
    cfg = FP_SMALL["inout"]
    w, u = _fp_layer(cfg, 43)
    out = oracle.mixer(_fp_cfg_dict(cfg), w, u)
    M, R, N = cfg.tokens, cfg.dt_rank, cfg.d_state
    sh = (cfg.batch, cfg.seqlen)
    uu = u.reshape(M, -1)
    x = (uu.astype(np.float64) @ w["f_in"].T.astype(np.float64)).astype(np.float32)
    p, *_ = oracle.bitlinear(x, w["c_x"], w["s_x"])
    p = p.astype(np.float32)
    z, *_ = oracle.bitlinear(p, w["c_dt"], w["s_dt"], k=R)
    y, _ = oracle.selective_scan(x.reshape(*sh, -1), z.astype(np.float32).reshape(*sh, -1), w["A"],
                                 p[:, R:R + N].reshape(*sh, -1), p[:, R + N:].reshape(*sh, -1), w["D"], w["dt_bias"])
    o = y.astype(np.float32).reshape(M, -1).astype(np.float64) @ w["f_out"].T.astype(np.float64)
    ref = (o + uu).astype(np.float32).astype(np.float64).reshape(out.shape)
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-7)


def test_mixer_fp_all_dt_stored():
    """fp_ssm baseline: the dt projection output is stored in the activation type before the
    scan reads it (a bf16 layer equals the composition with that rounding)."""
    cfg = FP_SMALL["all"].with_(act_dtype="bf16")
    w, u = _fp_layer(cfg, 44)
    u = oracle.round_bf16(u)
    out = oracle.mixer(_fp_cfg_dict(cfg), w, u)
    M, R, N = cfg.tokens, cfg.dt_rank, cfg.d_state
    sh = (cfg.batch, cfg.seqlen)
    rb = oracle.round_bf16
    uu = u.reshape(M, -1)
    x = rb((uu.astype(np.float64) @ w["f_in"].T.astype(np.float64)).astype(np.float32))
    p = rb((x.astype(np.float64) @ w["f_x"].T.astype(np.float64)).astype(np.float32))
    dt = rb((p[:, :R].astype(np.float64) @ w["f_dt"].T.astype(np.float64)).astype(np.float32))
    y, _ = oracle.selective_scan(x.reshape(*sh, -1), dt.reshape(*sh, -1), w["A"], p[:, R:R + N].reshape(*sh, -1),
                                 p[:, R + N:].reshape(*sh, -1), w["D"], w["dt_bias"])
    y = rb(y.astype(np.float32)).reshape(M, -1)
    o = y.astype(np.float64) @ w["f_out"].T.astype(np.float64)
    ref = rb((o + uu).astype(np.float32)).astype(np.float64).reshape(out.shape)
    bad = np.abs(out - ref) > 2 ** -7 * np.abs(ref) + 1e-6
    assert bad.mean() < 1e-3, bad.mean()


# ------------------------------------------------------------------ STE backward, QAT step

def _fd_grad(f, x, h=1e-6):
    """Central finite differences of a scalar function of an fp64 array."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += h
        xm[i] -= h
        g[i] = (f(xp) - f(xm)) / (2 * h)
    return g


@pytest.mark.parametrize("gain", [False, True])
def test_bwd_dx_is_rmsnorm_gradient(gain):
    """The estimator passes dx̂ = dy W̃ through the activation quantiser unchanged, so dx is the
    exact gradient of <dy, RMSNorm(x) g W̃^T> with W̃ held fixed: checked by finite differences."""
    g = wl.rng(61)
    m, k, n = 3, 16, 5
    x = wl.normal(g, (m, k))
    w = wl.normal(g, (n, k), 0.0, 0.02)
    gn = (1.0 + 0.3 * wl.normal(g, (k,))).astype(np.float32) if gain else None
    codes, s, _ = oracle.quantize_weights(w, 0)
    dy = wl.normal(g, (m, n)).astype(np.float64)
    out = oracle.bitlinear_bwd(x, codes, s, dy, norm_w=gn)
    wt = float(s[0]) * codes.astype(np.float64)
    gv = np.ones(k) if gn is None else gn.astype(np.float64)
    eps = 1e-5

    def f(xx):
        r = 1.0 / np.sqrt(np.mean(xx * xx, axis=1, keepdims=True) + eps)
        return float(np.sum(dy * ((xx * r * gv) @ wt.T)))

    fd = _fd_grad(f, x.astype(np.float64))
    # the oracle uses the forward's fp32 scale r, so agreement is to fp32 precision
    np.testing.assert_allclose(out["dx"], fd, rtol=2e-5, atol=2e-6)


def test_bwd_dw_and_dequantised_activations():
    """dW is the gradient of the bilinear form <dy, x̃ W̃^T> in W̃ (finite differences), and
    x̃ is the forward's int8 codes times max(m, 1e-5) / 127, within half a step of x̂."""
    g = wl.rng(62)
    m, k, n = 4, 8, 3
    x = wl.normal(g, (m, k))
    w = wl.normal(g, (n, k), 0.0, 0.02)
    codes, s, _ = oracle.quantize_weights(w, 0)
    dy = wl.normal(g, (m, n)).astype(np.float64)
    out = oracle.bitlinear_bwd(x, codes, s, dy)
    xt = out["x_tilde"]
    fd = _fd_grad(lambda W: float(np.sum(dy * (xt @ W.T))), float(s[0]) * codes.astype(np.float64))
    np.testing.assert_allclose(out["dw"], fd, rtol=1e-7, atol=1e-8)
    _, xq, am, _ = oracle.bitlinear(x, codes, s)
    step = np.maximum(am.astype(np.float64), 1e-5) / 127.0
    np.testing.assert_allclose(xt, xq * step[:, None], rtol=0, atol=0)
    xh = np.stack([oracle.norm_row(x[i]) for i in range(m)]).astype(np.float64)
    assert np.all(np.abs(xt - xh) <= 0.5 * step[:, None] * (1 + 1e-6))


def test_bwd_scale_gradient_by_hand():
    """Step-size rule for one scale s = 0.5, latent W = (0.2, 0.7, -1.0, 0.05): v = W / s =
    (0.4, 1.4, -2, 0.1), codes (0, 1, -1, 0); the clip is active at 1.4 and -2, so the factors
    are (0 - 0.4, 1, -1, 0 - 0.1); with dW = (1, 2, 3, 4), ds = -0.4 + 2 - 3 - 0.4 = -1.8."""
    w = np.array([[0.2, 0.7, -1.0, 0.05]], np.float32)
    s = np.array([0.5], np.float32)
    codes, _ = oracle.ternarize(w, 0, s)
    np.testing.assert_array_equal(codes, [[0, 1, -1, 0]])
    x = np.ones((1, 4), np.float32)
    dw_target = np.array([[1.0, 2.0, 3.0, 4.0]])
    # choose dy so that dW = dy^T x̃ equals dw_target: x̃ is all ones here (one token of ones)
    out = oracle.bitlinear_bwd(x, codes, s, np.array([[1.0]]), w_latent=w)
    xt = out["x_tilde"][0]
    np.testing.assert_allclose(xt, np.ones(4), rtol=1e-4)  # RMSNorm of ones is 1 / sqrt(1 + eps)
    v = w.astype(np.float64)[0] / 0.5
    fac = np.where(np.abs(v) <= 1.0, codes[0] - v, codes[0])
    assert np.allclose(fac, [-0.4, 1.0, -1.0, -0.1])
    assert abs(float(np.sum(dw_target[0] * fac)) - (-1.8)) < 1e-6  # the weights are fp32 values
    np.testing.assert_allclose(out["ds"], [np.sum(out["dw"][0] * fac)], rtol=1e-12)


def test_bwd_grouped_scale_gradient_is_per_group():
    """With groups, each scale sums only its own group's terms: the per-tensor result equals
    the sum of the per-group results when every group has the same scale."""
    g = wl.rng(63)
    m, k, n, G = 5, 256, 4, 128
    x = wl.normal(g, (m, k))
    w = wl.normal(g, (n, k), 0.0, 0.02)
    s0 = oracle.absmean(w, 0)
    sg = np.full((n, k // G), s0[0], np.float32)
    c0, _ = oracle.ternarize(w, 0, s0)
    cg, _ = oracle.ternarize(w, G, sg)
    np.testing.assert_array_equal(c0, cg)
    dy = wl.normal(g, (m, n)).astype(np.float64)
    a = oracle.bitlinear_bwd(x, c0, s0, dy, w_latent=w)
    b = oracle.bitlinear_bwd(x, cg, sg, dy, group=G, w_latent=w)
    np.testing.assert_allclose(b["dx"], a["dx"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b["ds"].sum(), a["ds"][0], rtol=1e-10)


def test_qat_step_hand_examples():
    """One QAT step on hand-worked values (tests/golden/qat_step_example.txt): the latent update
    W - lr dW, the scale update s - lr_s ds, and the codes and zero count under the new scales,
    per tensor and per group.  A sign or a factor wrong in either update changes the result."""
    g = _read_golden("qat_step_example.txt")
    for i, group in ((1, 0), (2, 2)):
        W, dW = _floats(g[f"W{i}"]), _floats(g[f"dW{i}"])
        s, ds = _floats(g[f"s{i}"]).ravel(), _floats(g[f"ds{i}"]).ravel()
        lr, lr_s = (float(v) for v in _floats(g[f"lr{i}"]).ravel())
        if group:
            s, ds = s.reshape(W.shape[0], -1), ds.reshape(W.shape[0], -1)
        Wn, sn, codes, zeros = oracle.qat_step(W, s, dW, ds, lr, lr_s, group)
        np.testing.assert_array_equal(Wn, _floats(g[f"Wnew{i}"]))
        np.testing.assert_array_equal(np.asarray(sn).ravel(), _floats(g[f"snew{i}"]).ravel())
        np.testing.assert_array_equal(codes, _ints(g[f"codes{i}"]))
        assert zeros == int(g[f"zeros{i}"][0][0])


def test_qat_step_zero_lr_and_zero_ratio():
    """lr = 0 leaves weights, scales and codes as they were; raising a scale can only turn
    codes into zeros (the zero ratio grows with the scale -- the collapse the Ternary Mamba
    abstract reports for learnable scales)."""
    g = wl.rng(64)
    w = wl.normal(g, (16, 128), 0.0, 0.02)
    codes, s, zeros = oracle.quantize_weights(w, 0)
    W, s2, c2, z2 = oracle.qat_step(w, s, np.ones_like(w), np.ones(1), 0.0, 0.0)
    np.testing.assert_array_equal(W, w)
    np.testing.assert_array_equal(c2, codes)
    assert z2 == zeros
    _, _, c3, z3 = oracle.qat_step(w, s, np.zeros_like(w), np.array([-0.5 * float(s[0])]), 0.0, 1.0)
    assert z3 > zeros
    assert np.all((c3 == 0) | (c3 == codes))


@pytest.mark.parametrize("aps,P", [(True, 1), (False, 2)])
def test_scan_bwd_matches_finite_differences(aps, P):
    """Every gradient of the scan's backward (x, delta, A, B, C, D, the delta bias, h0) against
    central finite differences of <dy, y> through the oracle's own forward, at a size where
    that is exact to ~1e-7."""
    g = wl.rng(91 + P)
    Bsz, L, H, N = 2, 5, 2, 3
    p = wl.scan_problem(Bsz, L, H, P, N, aps, seed=91 + P)
    h0 = wl.normal(g, (Bsz, H, P, N), 0.0, 0.5)
    dy = wl.normal(g, (Bsz, L, H * P)).astype(np.float64)
    out = oracle.selective_scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["D"], dy,
                                    delta_bias=p["dt_bias"], h0=h0)
    base = {k: np.asarray(v, np.float64) for k, v in p.items()}
    base["h0"] = h0.astype(np.float64)

    def loss(name, val):
        q = dict(base)
        q[name] = val
        # evaluate in fp64 through a float64 reimplementation-free path: the oracle forward
        # takes fp32 inputs, so differences are taken with steps large enough for fp32
        y, _ = oracle.selective_scan(q["x"], q["delta"], q["A"], q["Bm"], q["Cm"], q["D"], q["dt_bias"],
                                     h0=q["h0"])
        return float(np.sum(dy * y))

    names = {"x": "dx", "delta": "ddelta", "A": "dA", "Bm": "dB", "Cm": "dC", "D": "dD", "dt_bias": "dbias",
             "h0": "dh0"}
    for name, gname in names.items():
        fd = _fd_grad(lambda v: loss(name, v), base[name], h=1e-3)
        np.testing.assert_allclose(out[gname], fd, rtol=2e-3, atol=2e-4, err_msg=name)


# ------------------------------------------------------------------ mixer backward

def _bwd_layer(cfg, seed, gains=False):
    lat, u = wl.mixer_problem(cfg, seed=seed)
    w = _layer_codes(cfg, lat[0])
    if gains:
        g = wl.rng(seed + 1)
        for name, (_, k) in cfg.proj_shapes.items():
            w["g_" + name] = (1.0 + 0.2 * wl.normal(g, (k,))).astype(np.float32)
    return lat[0], w, u


def test_mixer_bwd_forward_is_the_mixer():
    """The backward evaluates the forward again: its output equals the oracle mixer's, bit for bit."""
    cfg = wl.CONFIGS["bitssm_tiny"].with_(seqlen=24)
    _, w, u = _bwd_layer(cfg, 5, gains=True)
    dout = wl.normal(wl.rng(6), u.shape)
    for res in (True, False):
        got = oracle.mixer_bwd(_cfg_dict(cfg), w, u, dout, residual=res)
        np.testing.assert_array_equal(got["out"].astype(np.float64), oracle.mixer(_cfg_dict(cfg), w, u, residual=res))


def test_mixer_bwd_zero_out_proj():
    """All-zero out_proj codes: the layer is the identity (with the residual), so du = dout exactly
    and nothing behind out_proj receives a gradient; out_proj's own weight gradient does not vanish."""
    cfg = wl.CONFIGS["bitssm_tiny"].with_(seqlen=16)
    _, w, u = _bwd_layer(cfg, 7)
    w["c_out"] = np.zeros_like(w["c_out"])
    dout = wl.normal(wl.rng(8), u.shape)
    got = oracle.mixer_bwd(_cfg_dict(cfg), w, u, dout)
    np.testing.assert_array_equal(got["du"], dout.astype(np.float64))
    for k in ("dw_in", "dw_x", "dw_dt", "dA", "dD", "d_dt_bias"):
        assert not np.any(got[k]), k
    assert np.any(got["dw_out"])


def test_mixer_bwd_a16_matches_finite_differences():
    """With the activation quantiser removed (W1.58A16 projections) the estimators pass nothing
    through a rounding, so the chain's result is the plain derivative of <dout, mixer(u)>: du, dA,
    dD and the dt bias element by element, and each projection's weight gradient along its own
    ternary codes (the derivative in that projection's scale), by central differences of the
    oracle mixer (fp32 activations; steps large against their rounding)."""
    cfg = wl.MixerConfig("fd", wl.MAMBA1, 8, 16, 4, batch=2, seqlen=5, dt_rank=4, act_bits=16)
    _, w, u = _bwd_layer(cfg, 11, gains=True)
    cd = _cfg_dict(cfg)
    dout = wl.normal(wl.rng(12), u.shape).astype(np.float64)
    got = oracle.mixer_bwd(cd, w, u, dout, residual=False)

    def loss(**over):
        q = dict(w)
        uu = over.pop("u", u)
        q.update(over)
        return float(np.sum(dout * oracle.mixer(cd, q, uu, residual=False)))

    h = 1e-3
    fd = _fd_grad(lambda v: loss(u=v.astype(np.float32)), u.astype(np.float64), h=h)
    np.testing.assert_allclose(got["du"], fd, rtol=3e-3, atol=3e-4)
    for name, gname in (("A", "dA"), ("D", "dD"), ("dt_bias", "d_dt_bias")):
        fd = _fd_grad(lambda v: loss(**{name: v.astype(np.float32)}), w[name].astype(np.float64), h=h)
        np.testing.assert_allclose(got[gname], fd, rtol=3e-3, atol=3e-4, err_msg=name)
    # the scales: Richardson-extrapolated differences with steps of 8 % and 4 % of the scale (the
    # forward's fp32 activations leave ~1e-6 noise in the loss, which smaller steps would amplify);
    # the dt projection's derivative is ~1e-4 here, so its bound is looser
    for name, tol in (("in", 3e-3), ("x", 3e-3), ("dt", 5e-2), ("out", 3e-3)):
        s = np.asarray(w["s_" + name], np.float64)
        d1, d2 = (_fd_grad(lambda v: loss(**{"s_" + name: v.astype(np.float32)}), s, h=f * float(s[0]))[0]
                  for f in (8e-2, 4e-2))
        fd = (4 * d2 - d1) / 3
        along = float(np.sum(got["dw_" + name] * w["c_" + name]))
        assert abs(along - fd) <= tol * abs(fd), (name, along, fd)
