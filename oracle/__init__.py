"""CPU oracle for the ternary selective-SSM mixer forward (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``oracle.c`` (plain C, fp64)
through ctypes and shares nothing with the HIP library.  What each function
computes, and the passage of the pages it follows, is documented in
``oracle.c``.

Parity pins: every function below is pinned in ``tests/test_oracle_pins.py``
against closed forms, brute force, invariants or the printed fixtures under
``tests/golden/``; none is "parity unpinned" except the whole-mixer numerical
values beyond the composition of pinned stages (no page prints a mixer output).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1

_c_f32p = ctypes.POINTER(ctypes.c_float)
_c_f64p = ctypes.POINTER(ctypes.c_double)
_c_i8p = ctypes.POINTER(ctypes.c_int8)
_c_u8p = ctypes.POINTER(ctypes.c_uint8)
_c_i32p = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _MixerWeights(ctypes.Structure):
    _fields_ = [("c_in", _c_i8p), ("c_x", _c_i8p), ("c_dt", _c_i8p), ("c_out", _c_i8p),
                ("s_in", _c_f32p), ("s_x", _c_f32p), ("s_dt", _c_f32p), ("s_out", _c_f32p),
                ("g_in", _c_f32p), ("g_x", _c_f32p), ("g_dt", _c_f32p), ("g_out", _c_f32p),
                ("dt_bias", _c_f32p), ("A", _c_f32p), ("D", _c_f32p), ("conv_w", _c_f32p), ("conv_b", _c_f32p),
                ("f_in", _c_f32p), ("f_x", _c_f32p), ("f_dt", _c_f32p), ("f_out", _c_f32p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_round_bf16.argtypes = [ctypes.c_float]
        L.orc_round_bf16.restype = ctypes.c_float
        L.orc_round_array.argtypes = [_c_f64p, _c_f32p, _i64, ctypes.c_int]
        L.orc_absmean.argtypes = [_c_f32p, _i64, _i64, _i64, _c_f32p]
        L.orc_ternarize.argtypes = [_c_f32p, _i64, _i64, _i64, _c_f32p, _c_i8p]
        L.orc_ternarize.restype = _i64
        L.orc_packed_row_bytes.argtypes = [_i64]
        L.orc_packed_row_bytes.restype = _i64
        L.orc_pack.argtypes = [_c_i8p, _i64, _i64, _c_u8p]
        L.orc_unpack.argtypes = [_c_u8p, _i64, _i64, _c_i8p]
        L.orc_unpack.restype = _i64
        L.orc_rms_scale.argtypes = [_c_f32p, _i64, ctypes.c_float]
        L.orc_rms_scale.restype = ctypes.c_float
        L.orc_norm_row.argtypes = [_c_f32p, _i64, _c_f32p, ctypes.c_float, _c_f32p]
        L.orc_quant_row.argtypes = [_c_f32p, _i64, _c_i8p]
        L.orc_quant_row.restype = ctypes.c_float
        L.orc_bitlinear.argtypes = [_c_f32p, _i64, _i64, _i64, _c_f32p, ctypes.c_float, ctypes.c_int,
                                    _c_i8p, _c_f32p, _i64, _i64, _c_f32p, _c_f64p, _c_i8p, _c_f32p,
                                    _c_i32p]
        L.orc_bitlinear.restype = ctypes.c_int
        L.orc_softplus.argtypes = [ctypes.c_double]
        L.orc_softplus.restype = ctypes.c_double
        scan_args = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int, _c_f32p, _c_f32p, _c_f32p, ctypes.c_int,
                     _c_f32p, _c_f32p, _c_f32p, _c_f32p]
        L.orc_selective_scan.argtypes = scan_args + [_c_f32p, _c_f64p, _c_f64p]
        L.orc_selective_scan_blelloch.argtypes = scan_args + [_c_f32p, _c_f64p, _c_f64p]
        L.orc_selective_scan_quadratic.argtypes = scan_args + [_c_f64p]
        L.orc_mixer.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                ctypes.c_int, ctypes.c_float, ctypes.POINTER(_MixerWeights), _c_f32p,
                                _i64, _i64, ctypes.c_int, ctypes.c_int, _i64, ctypes.c_int, _c_f64p]
        L.orc_dense.argtypes = [_c_f32p, _i64, _i64, _i64, _c_f32p, _i64, _c_f64p]
        L.orc_mixer.restype = ctypes.c_int
        L.orc_silu.argtypes = [ctypes.c_double]
        L.orc_silu.restype = ctypes.c_double
        L.orc_conv_silu.argtypes = [_i64, _i64, _i64, _i64, _c_f32p, _i64, _c_f32p, _c_f32p, _c_f32p, ctypes.c_int,
                                    _c_f32p, _c_f32p]
        _lib = L
    return _lib


# ---------------------------------------------------------------- helpers

def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _p(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctype)


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (results do not depend on it)."""
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


def round_bf16(a) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even), returned as fp32."""
    a = _f32(a)
    d = a.astype(np.float64)
    out = np.empty_like(a)
    lib().orc_round_array(_p(d, _c_f64p), _p(out, _c_f32p), a.size, BF16)
    return out


# ---------------------------------------------------------------- O0

def absmean(w, group: int = 0) -> np.ndarray:
    w = _f32(w)
    n, k = w.shape
    out = np.empty(1 if group == 0 else n * (k // group), dtype=np.float32)
    lib().orc_absmean(_p(w, _c_f32p), n, k, group, _p(out, _c_f32p))
    return out if group == 0 else out.reshape(n, k // group)


def ternarize(w, group: int, scale) -> tuple[np.ndarray, int]:
    w = _f32(w)
    n, k = w.shape
    scale = _f32(scale)
    codes = np.empty((n, k), dtype=np.int8)
    zeros = lib().orc_ternarize(_p(w, _c_f32p), n, k, group, _p(scale, _c_f32p), _p(codes, _c_i8p))
    return codes, int(zeros)


def quantize_weights(w, group: int = 0, scale_in=None):
    """(codes int8 [n,k], scale fp32, zero count): absmean (or caller) scale, then codes."""
    scale = absmean(w, group) if scale_in is None else _f32(scale_in)
    codes, zeros = ternarize(w, group, scale)
    return codes, scale, zeros


def packed_row_bytes(k: int) -> int:
    return int(lib().orc_packed_row_bytes(k))


def pack(codes) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    n, k = codes.shape
    out = np.empty((n, packed_row_bytes(k)), dtype=np.uint8)
    lib().orc_pack(_p(codes, _c_i8p), n, k, _p(out, _c_u8p))
    return out


def unpack(packed, k: int) -> tuple[np.ndarray, int]:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    codes = np.empty((n, k), dtype=np.int8)
    bad = lib().orc_unpack(_p(packed, _c_u8p), n, k, _p(codes, _c_i8p))
    return codes, int(bad)


# ---------------------------------------------------------------- O1 / O2

def rms_scale(v, eps: float = 1e-5) -> np.float32:
    v = _f32(v)
    return np.float32(lib().orc_rms_scale(_p(v, _c_f32p), v.size, eps))


def norm_row(v, g=None, eps: float = 1e-5) -> np.ndarray:
    v = _f32(v)
    g = None if g is None else _f32(g)
    out = np.empty_like(v)
    lib().orc_norm_row(_p(v, _c_f32p), v.size, _p(g, _c_f32p), eps, _p(out, _c_f32p))
    return out


def quant_row(xh) -> tuple[np.ndarray, np.float32]:
    xh = _f32(xh)
    q = np.empty(xh.size, dtype=np.int8)
    m = lib().orc_quant_row(_p(xh, _c_f32p), xh.size, _p(q, _c_i8p))
    return q, np.float32(m)


# ---------------------------------------------------------------- O3 / O4

def bitlinear(x, codes, w_scale, group: int = 0, act_bits: int = 8, norm_w=None, eps: float = 1e-5,
              bias=None, k: int | None = None):
    """BitLinear on rows x[m, 0:k] (x may be wider: its row stride is x.shape[1]).

    Returns (y fp64 [m,n], xq int8 [m,k] or None, absmax fp32 [m] or None, acc int32 [m,n] or None).
    """
    x = _f32(x)
    m, ldx = x.shape
    k = ldx if k is None else k
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    n = codes.shape[0]
    assert codes.shape[1] == k
    w_scale = _f32(w_scale)
    norm_w = None if norm_w is None else _f32(norm_w)
    bias = None if bias is None else _f32(bias)
    y = np.empty((m, n), dtype=np.float64)
    if act_bits == 8:
        xq = np.empty((m, k), dtype=np.int8)
        am = np.empty(m, dtype=np.float32)
        acc = np.empty((m, n), dtype=np.int32)
    else:
        xq = am = acc = None
    rc = lib().orc_bitlinear(_p(x, _c_f32p), m, k, ldx, _p(norm_w, _c_f32p), eps, act_bits,
                             _p(codes, _c_i8p), _p(w_scale, _c_f32p), n, group, _p(bias, _c_f32p),
                             _p(y, _c_f64p), _p(xq, _c_i8p), _p(am, _c_f32p), _p(acc, _c_i32p))
    if rc != 0:
        raise OverflowError("int32 accumulator overflow")
    return y, xq, am, acc


# ---------------------------------------------------------------- O5 / O6 / O7

def softplus(v: float) -> float:
    return float(lib().orc_softplus(v))


def _scan_common(x, delta, A, Bm, Cm, D, delta_bias, h0):
    x, delta, A, Bm, Cm = _f32(x), _f32(delta), _f32(A), _f32(Bm), _f32(Cm)
    batch, L, H = delta.shape
    HP = x.shape[2]
    P = HP // H
    N = Bm.shape[2]
    a_per_state = 1 if A.ndim == 2 else 0
    D = None if D is None else _f32(D)
    delta_bias = None if delta_bias is None else _f32(delta_bias)
    h0 = None if h0 is None else _f32(h0)
    return x, delta, A, Bm, Cm, D, delta_bias, h0, batch, L, H, P, N, a_per_state


def selective_scan(x, delta, A, Bm, Cm, D=None, delta_bias=None, softplus: bool = True, h0=None,
                   method: str = "loop"):
    """Selective scan. x [B,L,H*P], delta [B,L,H], A [H,N] (Mamba-1) or [H] (SSD),
    Bm/Cm [B,L,N], D [H].  Returns (y fp64 [B,L,H*P], h_last fp64 [B,H,P,N] or None).
    method: "loop" (sequential recurrence), "blelloch" (parallel associative scan),
    "quadratic" (state-space-duality masked form; h0 must be None; no h_last)."""
    (x, delta, A, Bm, Cm, D, delta_bias, h0, batch, L, H, P, N,
     aps) = _scan_common(x, delta, A, Bm, Cm, D, delta_bias, h0)
    y = np.empty((batch, L, H * P), dtype=np.float64)
    common = (batch, L, H, P, N, aps, _p(x, _c_f32p), _p(delta, _c_f32p), _p(delta_bias, _c_f32p),
              int(softplus), _p(A, _c_f32p), _p(Bm, _c_f32p), _p(Cm, _c_f32p), _p(D, _c_f32p))
    if method == "quadratic":
        assert h0 is None
        lib().orc_selective_scan_quadratic(*common, _p(y, _c_f64p))
        return y, None
    hl = np.empty((batch, H, P, N), dtype=np.float64)
    fn = lib().orc_selective_scan if method == "loop" else lib().orc_selective_scan_blelloch
    fn(*common, _p(h0, _c_f32p), _p(y, _c_f64p), _p(hl, _c_f64p))
    return y, hl


# ---------------------------------------------------------------- gated block

def silu(v: float) -> float:
    return float(lib().orc_silu(v))


def conv_silu(x, w, bias=None, state=None, act_dtype: int = 0, channels: int | None = None):
    """Causal depthwise convolution of width K = w.shape[1] along time, then SiLU (fp64,
    rounded to act_dtype).  x [B, L, ldx] (first `channels` columns used), w [C, K],
    bias [C] or None, state [B, K-1, C] or None (inputs before t = 0; zeros if None).
    Returns (out [B, L, C] fp32, state after the sequence [B, K-1, C] fp32)."""
    x = _f32(x)
    batch, L, ldx = x.shape
    w = _f32(w)
    C, K = w.shape
    if channels is not None and channels != C:
        raise ValueError("w rows must equal channels")
    b = None if bias is None else _f32(bias)
    st = None if state is None else _f32(state)
    out = np.empty((batch, L, C), dtype=np.float32)
    st_out = np.empty((batch, max(K - 1, 0), C), dtype=np.float32)
    lib().orc_conv_silu(batch, L, C, K, _p(x, _c_f32p), ldx, _p(w, _c_f32p), _p(b, _c_f32p), _p(st, _c_f32p),
                        act_dtype, _p(out, _c_f32p), _p(st_out, _c_f32p) if K > 1 else None)
    return out, st_out


# ---------------------------------------------------------------- full-precision projection

def dense(x, W, k: int | None = None) -> np.ndarray:
    """y = x[:, :k] W^T in fp64 (a full-precision linear layer: no norm, no quantisation)."""
    x = _f32(x)
    m, ldx = x.shape
    W = _f32(W)
    n, kk = W.shape
    k = kk if k is None else k
    if k != kk:
        raise ValueError("W must have k columns")
    y = np.empty((m, n), dtype=np.float64)
    lib().orc_dense(_p(x, _c_f32p), m, k, ldx, _p(W, _c_f32p), n, _p(y, _c_f64p))
    return y


# ---------------------------------------------------------------- mixer

MAMBA1, SSD = 0, 1


def mixer(cfg, weights: dict, u, residual: bool = True) -> np.ndarray:
    """One mixer layer.  cfg: mapping with kind, d_model, d_inner, d_state, dt_rank,
    nheads, headdim, group_size, act_bits, act_dtype (F32/BF16), norm_eps.
    weights: codes c_in/c_x/c_dt/c_out, scales s_*, dt_bias, A, D (gains optional g_*); for the
    gated block (cfg gated = 1, d_conv) also conv_w [Cc, d_conv] and conv_b [Cc] (optional);
    for full-precision projections (cfg fp_proj = 1: in/out, 2: all) f_in / f_x / f_dt / f_out
    [n_out, k] weight values.
    u: [B, L, d_model] values (bf16-representable when act_dtype is BF16).
    Returns out fp64 [B, L, d_model], each value already rounded to act_dtype."""
    u = _f32(u)
    batch, L, dm = u.shape
    keep = []

    def arr(name, dtype, ctype):
        a = weights.get(name)
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=dtype)
        keep.append(a)
        return a.ctypes.data_as(ctype)

    w = _MixerWeights(
        arr("c_in", np.int8, _c_i8p), arr("c_x", np.int8, _c_i8p), arr("c_dt", np.int8, _c_i8p),
        arr("c_out", np.int8, _c_i8p), arr("s_in", np.float32, _c_f32p), arr("s_x", np.float32, _c_f32p),
        arr("s_dt", np.float32, _c_f32p), arr("s_out", np.float32, _c_f32p),
        arr("g_in", np.float32, _c_f32p), arr("g_x", np.float32, _c_f32p), arr("g_dt", np.float32, _c_f32p),
        arr("g_out", np.float32, _c_f32p), arr("dt_bias", np.float32, _c_f32p),
        arr("A", np.float32, _c_f32p), arr("D", np.float32, _c_f32p), arr("conv_w", np.float32, _c_f32p),
        arr("conv_b", np.float32, _c_f32p), arr("f_in", np.float32, _c_f32p), arr("f_x", np.float32, _c_f32p),
        arr("f_dt", np.float32, _c_f32p), arr("f_out", np.float32, _c_f32p))
    out = np.empty((batch, L, dm), dtype=np.float64)
    rc = lib().orc_mixer(int(cfg["kind"]), cfg["d_model"], cfg["d_inner"], cfg["d_state"], cfg.get("dt_rank", 0),
                         cfg.get("nheads", 0), cfg.get("headdim", 0), cfg.get("group_size", 0), cfg["act_bits"],
                         cfg["act_dtype"], cfg.get("norm_eps", 1e-5), ctypes.byref(w), _p(u, _c_f32p), batch, L,
                         int(residual), int(cfg.get("gated", 0)), int(cfg.get("d_conv", 0)), int(cfg.get("fp_proj", 0)),
                         _p(out, _c_f64p))
    if rc != 0:
        raise OverflowError("int32 accumulator overflow in the mixer")
    return out


def mixer_stack(cfg, layers: list, u) -> np.ndarray:
    """out = u + mixer_l(u) applied layer after layer; returns fp64 of the stored values."""
    h = _f32(u)
    out = None
    for wts in layers:
        out = mixer(cfg, wts, h, residual=True)
        h = out.astype(np.float32)
    return out


# ---------------------------------------------------------------- O10: STE backward, one QAT step

def bitlinear_bwd(x, codes, w_scale, dy, group: int = 0, norm_w=None, eps: float = 1e-5, w_latent=None,
                  act_bits: int = 8) -> dict:
    """Backward of the A8 BitLinear with straight-through estimators (TriSSM README: BitLinear
    trained with straight-through estimators; the estimator of "Estimating or Propagating
    Gradients Through Stochastic Neurons ...", cited under "Builds on"), fp64.

    Forward being differentiated: x̂ = RMSNorm(x) g;  x̃ = q_x max(m, 1e-5) / 127 (the int8
    codes of the forward, dequantised);  W̃ = s q_w (the ternary codes times their scale);
    y = x̃ W̃^T.  The estimator passes gradients through both roundings unchanged (the absmax
    and the scale are held fixed there), so
      dx̂ = dy W̃,   dW = dy^T x̃  (the latent weights receive W̃'s gradient),
      dx  = r g dx̂ - x (r^3 / k) sum_j g_j dx̂_j x_j   (RMSNorm, r = 1 / sqrt(mean x^2 + eps)).
    Learnable scales (Ternary Mamba abstract: grouped QAT with learnable quantisation scales),
    given the latent weights: with v = W / s, dW̃/ds is q - v where |v| <= 1 and q where the
    clip is active (the step-size rule of learned-step-size quantisation), summed over each
    scale's group:  ds = sum dW (q - v or q).
    act_bits 16 (W1.58A16, no activation quantiser): x̃ is the fp32 RMSNorm output itself, and
    dx, dW are then the plain derivatives of that BitLinear.
    Returns dict(dx [m,k], dw [n,k], ds (scalar array or [n, k/group]) or None, x_tilde, r)."""
    x = _f32(x)
    m, k = x.shape
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    n = codes.shape[0]
    dy = np.asarray(dy, dtype=np.float64)
    r = np.array([rms_scale(x[i], eps) for i in range(m)], dtype=np.float32).astype(np.float64)
    if act_bits == 8:
        _, xq, am, _ = bitlinear(x, codes, w_scale, group, 8, norm_w, eps)
        xt = xq.astype(np.float64) * (np.maximum(am, np.float32(1e-5)).astype(np.float64) / 127.0)[:, None]
    else:
        xt = np.stack([norm_row(x[i], norm_w, eps) for i in range(m)]).astype(np.float64).reshape(m, k)
    sc = np.asarray(w_scale, dtype=np.float32).astype(np.float64)
    s_full = np.full((n, k), sc.ravel()[0]) if group == 0 else np.repeat(sc.reshape(n, k // group), group, axis=1)
    wt = s_full * codes.astype(np.float64)
    g = np.ones(k) if norm_w is None else np.asarray(norm_w, dtype=np.float32).astype(np.float64)
    xd = x.astype(np.float64)
    dxh = dy @ wt
    dot = np.sum(g[None, :] * dxh * xd, axis=1)
    dx = r[:, None] * (g[None, :] * dxh) - xd * (r ** 3 / k)[:, None] * dot[:, None]
    dw = dy.T @ xt
    ds = None
    if w_latent is not None:
        v = np.asarray(w_latent, dtype=np.float32).astype(np.float64) / s_full
        fac = np.where(np.abs(v) <= 1.0, codes - v, codes.astype(np.float64))
        gs = dw * fac
        ds = np.array([gs.sum()]) if group == 0 else gs.reshape(n, k // group, group).sum(axis=2)
    return dict(dx=dx, dw=dw, ds=ds, x_tilde=xt, r=r)


def qat_step(w_latent, w_scale, dw, ds, lr: float, lr_scale: float, group: int = 0):
    """One SGD step of quantisation-aware training on the latent weights and their learnable
    scales (Ternary Mamba abstract), then the codes under the updated scales:
      W <- W - lr dW,  s <- s - lr_scale ds  (each rounded once to fp32),
      q = clamp(round(W / s), -1, 1).
    Returns (W fp32, s fp32, codes int8, zero count) -- the zero count is the zero ratio the
    abstract watches (it collapses when learnable scales grow)."""
    W = (np.asarray(w_latent, np.float32).astype(np.float64) - np.float64(np.float32(lr)) * np.asarray(dw, np.float64))
    W = W.astype(np.float32)
    s = np.asarray(w_scale, np.float32).astype(np.float64) - np.float64(np.float32(lr_scale)) * np.asarray(ds, np.float64).reshape(np.shape(w_scale))
    s = s.astype(np.float32)
    codes, zeros = ternarize(W, group, s)
    return W, s, codes, zeros


def selective_scan_bwd(x, delta, A, Bm, Cm, D, dy, delta_bias=None, softplus: bool = True, h0=None) -> dict:
    """Backward of the selective scan (the recurrence of ``selective_scan``), fp64, by reverse
    accumulation through the stored states.  With dt_t = softplus(delta_t + bias),
    a_t = exp(dt_t A), h_t = a_t h_{t-1} + dt_t x_t B_t and y_t = C_t . h_t + D x_t, the
    adjoint of the state is g_t = C_t dy_t + a_{t+1} g_{t+1}; then
      dC_t = sum over channels of dy_t h_t,   dB_t = sum of g_t dt_t x_t,
      dx_t = D dy_t + dt_t sum_n g_t B_t,     d dt_t = sum_n g_t (h_{t-1} a_t A + x_t B_t),
      d delta_t = d dt_t * sigmoid(delta_t + bias) (1 above 20, where softplus is the identity),
      dA = sum_t g_t h_{t-1} a_t dt_t,  dD = sum_t dy_t x_t,  d bias = sum_t d delta_t,
      dh0 = a_0 g_0.
    Shapes as ``selective_scan``; dy like y.  Returns a dict of fp64 arrays."""
    x = np.asarray(x, np.float32).astype(np.float64)
    delta = np.asarray(delta, np.float32).astype(np.float64)
    A = np.asarray(A, np.float32).astype(np.float64)
    Bm = np.asarray(Bm, np.float32).astype(np.float64)
    Cm = np.asarray(Cm, np.float32).astype(np.float64)
    dy = np.asarray(dy, np.float64)
    batch, L, HP = x.shape
    H = delta.shape[2]
    P = HP // H
    N = Bm.shape[2]
    aps = A.ndim == 2
    Dv = np.zeros(H) if D is None else np.asarray(D, np.float32).astype(np.float64)
    bias = np.zeros(H) if delta_bias is None else np.asarray(delta_bias, np.float32).astype(np.float64)
    Ab = A[:, None, :] if aps else A[:, None, None]                      # [H, 1, N or 1]
    pre = delta + bias[None, None, :]                                    # [B, L, H]
    dt = np.where(pre > 20.0, pre, np.log1p(np.exp(np.minimum(pre, 20.0)))) if softplus else pre
    sig = np.where(pre > 20.0, 1.0, 1.0 / (1.0 + np.exp(-pre))) if softplus else np.ones_like(pre)
    xs = x.reshape(batch, L, H, P)
    dys = dy.reshape(batch, L, H, P)
    hs = np.zeros((L + 1, batch, H, P, N))                              # hs[t + 1] = h_t, hs[0] = h0
    if h0 is not None:
        hs[0] = np.asarray(h0, np.float32).astype(np.float64).reshape(batch, H, P, N)
    for t in range(L):
        a = np.exp(dt[:, t, :, None, None] * Ab[None])                  # [B, H, 1 or P, N or 1]
        hs[t + 1] = a * hs[t] + (dt[:, t, :, None, None] * xs[:, t, :, :, None]) * Bm[:, t, None, None, :]
    dx = np.zeros((batch, L, H, P))
    ddelta = np.zeros((batch, L, H))
    dB = np.zeros((batch, L, N))
    dC = np.zeros((batch, L, N))
    dA = np.zeros_like(A)
    dD = np.zeros(H)
    carry = np.zeros((batch, H, P, N))                                   # a_{t+1} g_{t+1}
    for t in range(L - 1, -1, -1):
        a = np.exp(dt[:, t, :, None, None] * Ab[None]) * np.ones((1, 1, P, N))
        g = carry + Cm[:, t, None, None, :] * dys[:, t, :, :, None]
        hprev = hs[t]
        dC[:, t] = np.einsum("bhp,bhpn->bn", dys[:, t], hs[t + 1])
        dB[:, t] = np.einsum("bhpn,bh,bhp->bn", g, dt[:, t], xs[:, t])
        dx[:, t] = Dv[None, :, None] * dys[:, t] + dt[:, t, :, None] * np.einsum("bhpn,bn->bhp", g, Bm[:, t])
        ddt = np.einsum("bhpn,bhpn->bh", g, hprev * a * (Ab[None] * np.ones((1, 1, P, N)))) + \
            np.einsum("bhpn,bhp,bn->bh", g, xs[:, t], Bm[:, t])
        ddelta[:, t] = ddt * sig[:, t]
        gA = g * hprev * a * dt[:, t, :, None, None]
        dA += gA.sum(axis=(0, 2)) if aps else gA.sum(axis=(0, 2, 3))
        dD += np.einsum("bhp,bhp->h", dys[:, t], xs[:, t])
        carry = a * g
    return dict(dx=dx.reshape(batch, L, HP), ddelta=ddelta, dA=dA, dB=dB, dC=dC, dD=dD,
                dbias=ddelta.sum(axis=(0, 1)), dh0=carry.reshape(batch, H, P, N))


def mixer_bwd(cfg, weights: dict, u, dout, residual: bool = True, latents: dict | None = None) -> dict:
    """Backward of one Mamba-1 kind mixer layer (not gated, ternary projections, fp32 activations)
    under the straight-through estimators (TriSSM README: BitLinear layers trained with
    straight-through estimators, the SSM trained end to end), fp64.

    The forward is evaluated again with the roundings of ``mixer`` (x, p and y stored as fp32; the
    dt projection output passed to the scan at fp32 width), then the chain runs backwards:
      dy  = BL_out backward (dout),          scan backward (dy) -> dx_s, d delta, dB, dC, dA, dD, d bias,
      dp  = [BL_dt backward (d delta) | dB | dC],   dx = dx_s + BL_x backward (dp),
      du  = BL_in backward (dx) (+ dout when the residual is added).
    Each BitLinear backward is ``bitlinear_bwd``; its weight gradient is that of the dequantised
    ternary weights (the latent weights' gradient), and with latents["lat_in" / "lat_x" /
    "lat_dt" / "lat_out"] its learnable-scale gradient too.  act_bits 16 in cfg evaluates the same
    chain with no activation quantiser (the surrogate whose derivative the finite-difference
    pins check).  u, dout [B, L, d_model].  Returns a dict of fp64 arrays: du, dw_in, dw_x, dw_dt,
    dw_out, dA, dD, d_dt_bias (ds_* for the latents given) and out (the forward's output)."""
    assert int(cfg["kind"]) == MAMBA1 and int(cfg.get("gated", 0)) == 0 and int(cfg.get("fp_proj", 0)) == 0
    assert int(cfg["act_dtype"]) == F32 and int(cfg.get("group_size", 0)) == 0
    ab = int(cfg["act_bits"])
    eps = cfg.get("norm_eps", 1e-5)
    u = _f32(u)
    batch, L, dm = u.shape
    M = batch * L
    Di, N, R = cfg["d_inner"], cfg["d_state"], cfg["dt_rank"]
    w = weights
    lat = latents or {}
    u2 = u.reshape(M, dm)
    dout2 = np.asarray(dout, np.float32).astype(np.float64).reshape(M, dm)
    x = bitlinear(u2, w["c_in"], w["s_in"], 0, ab, w.get("g_in"), eps)[0].astype(np.float32)
    p = bitlinear(x, w["c_x"], w["s_x"], 0, ab, w.get("g_x"), eps)[0].astype(np.float32)
    z = bitlinear(p, w["c_dt"], w["s_dt"], 0, ab, w.get("g_dt"), eps, k=R)[0].astype(np.float32)
    x3 = x.reshape(batch, L, Di)
    z3 = z.reshape(batch, L, Di)
    B3 = np.ascontiguousarray(p[:, R:R + N]).reshape(batch, L, N)
    C3 = np.ascontiguousarray(p[:, R + N:R + 2 * N]).reshape(batch, L, N)
    y = selective_scan(x3, z3, w["A"], B3, C3, w.get("D"), w.get("dt_bias"))[0].astype(np.float32).reshape(M, Di)
    out = bitlinear(y, w["c_out"], w["s_out"], 0, ab, w.get("g_out"), eps)[0]
    if residual:
        out = out + u2.astype(np.float64)

    def bl(xin, name, gy):
        return bitlinear_bwd(xin, w["c_" + name], w["s_" + name], gy, 0, w.get("g_" + name), eps,
                             lat.get("lat_" + name), act_bits=ab)

    go = bl(y, "out", dout2)
    sb = selective_scan_bwd(x3, z3, w["A"], B3, C3, w.get("D"), go["dx"].reshape(batch, L, Di),
                            delta_bias=w.get("dt_bias"))
    gd = bl(np.ascontiguousarray(p[:, :R]), "dt", sb["ddelta"].reshape(M, Di))
    dp = np.concatenate([gd["dx"], sb["dB"].reshape(M, N), sb["dC"].reshape(M, N)], axis=1)
    gx = bl(x, "x", dp)
    gi = bl(u2, "in", sb["dx"].reshape(M, Di) + gx["dx"])
    du = gi["dx"] + (dout2 if residual else 0.0)
    res = dict(du=du.reshape(batch, L, dm), dw_in=gi["dw"], dw_x=gx["dw"], dw_dt=gd["dw"], dw_out=go["dw"],
               dA=sb["dA"], dD=sb["dD"], d_dt_bias=sb["dbias"], out=out.astype(np.float32).reshape(batch, L, dm))
    for name, g in (("in", gi), ("x", gx), ("dt", gd), ("out", go)):
        if g["ds"] is not None:
            res["ds_" + name] = g["ds"]
    return res
