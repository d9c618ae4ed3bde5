"""Python binding of libssm_ternary (MI355X / gfx950 ternary selective-SSM mixer forward).

Argument marshalling only: every step runs in the HIP library behind the C ABI declared
in include/ssm_ternary.h.  PyTorch supplies device memory and the current stream.  If the
library has not been built, every entry point raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssm_ternary.so")

SSM_F32, SSM_BF16, SSM_I8 = 0, 1, 2
SSM_MIXER_MAMBA1, SSM_MIXER_SSD = 0, 1
_DTYPES = {torch.float32: SSM_F32, torch.bfloat16: SSM_BF16, torch.int8: SSM_I8}
_TORCH = {SSM_F32: torch.float32, SSM_BF16: torch.bfloat16, SSM_I8: torch.int8}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


class BitlinearArgs(ctypes.Structure):
    _fields_ = [("x", _vp), ("x_dtype", _i32), ("act_bits", _i32), ("m", _i64), ("k", _i64), ("ldx", _i64),
                ("x_absmax", _vp), ("norm_weight", _vp), ("norm_eps", ctypes.c_float), ("pad0", _i32),
                ("w_packed", _vp), ("w_scale", _vp), ("n_out", _i64), ("group_size", _i64), ("bias", _vp),
                ("residual", _vp), ("ld_res", _i64), ("y", _vp), ("y_dtype", _i32), ("pad1", _i32), ("ldy", _i64),
                ("dbg_xq", _vp), ("dbg_absmax", _vp), ("dbg_acc", _vp)]


class ScanArgs(ctypes.Structure):
    _fields_ = [("batch", _i64), ("seqlen", _i64), ("nheads", _i64), ("headdim", _i64), ("d_state", _i64),
                ("a_per_state", _i32), ("act_dtype", _i32), ("x", _vp), ("ld_x", _i64), ("delta", _vp),
                ("ld_delta", _i64), ("delta_bias", _vp), ("delta_softplus", _i32), ("pad0", _i32), ("A", _vp),
                ("Bm", _vp), ("ld_B", _i64), ("Cm", _vp), ("ld_C", _i64), ("D", _vp), ("h0", _vp),
                ("h_last", _vp), ("y", _vp), ("ld_y", _i64), ("dt_in", _vp), ("ld_dt_in", _i64), ("dt_rank", _i64),
                ("w_dt", _vp), ("s_dt", _vp), ("g_dt", _vp), ("dt_eps", ctypes.c_float), ("pad1", _i32),
                ("gate", _vp), ("ld_gate", _i64), ("dt_codes", _vp), ("dt_deq", _vp)]


class ScanBwdArgs(ctypes.Structure):
    _fields_ = [("batch", _i64), ("seqlen", _i64), ("nheads", _i64), ("d_state", _i64), ("act_dtype", _i32),
                ("delta_softplus", _i32), ("x", _vp), ("ld_x", _i64), ("delta", _vp), ("ld_delta", _i64),
                ("delta_bias", _vp), ("A", _vp), ("Bm", _vp), ("ld_B", _i64), ("Cm", _vp), ("ld_C", _i64),
                ("D", _vp), ("h0", _vp), ("dy", _vp), ("ld_dy", _i64), ("dx", _vp), ("ddelta", _vp), ("dA", _vp),
                ("dB", _vp), ("dC", _vp), ("dD", _vp), ("dbias", _vp), ("dh0", _vp)]


class BitlinearBwdArgs(ctypes.Structure):
    _fields_ = [("x", _vp), ("x_dtype", _i32), ("pad0", _i32), ("m", _i64), ("k", _i64), ("ldx", _i64),
                ("norm_weight", _vp), ("norm_eps", ctypes.c_float), ("pad1", _i32), ("w_packed", _vp),
                ("w_scale", _vp), ("n_out", _i64), ("group_size", _i64), ("w_latent", _vp), ("dy", _vp),
                ("ld_dy", _i64), ("dx", _vp), ("ld_dx", _i64), ("dw", _vp), ("d_scale", _vp)]


class MixerConfig(ctypes.Structure):
    _fields_ = [("kind", _i32), ("act_bits", _i32), ("d_model", _i64), ("d_inner", _i64), ("d_state", _i64),
                ("dt_rank", _i64), ("nheads", _i64), ("headdim", _i64), ("group_size", _i64), ("act_dtype", _i32),
                ("norm_eps", ctypes.c_float), ("gated", _i32), ("d_conv", _i32), ("fp_proj", _i32), ("pad0", _i32)]


class MixerWeights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_in", "w_x", "w_dt", "w_out", "s_in", "s_x", "s_dt", "s_out", "g_in", "g_x",
                                   "g_dt", "g_out", "dt_bias", "A", "D", "conv_w", "conv_b", "fw_in", "fw_x",
                                   "fw_dt", "fw_out")]


class MixerGrads(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("lat_in", "lat_x", "lat_dt", "lat_out", "dw_in", "dw_x", "dw_dt", "dw_out",
                                   "ds_in", "ds_x", "ds_dt", "ds_out", "dA", "dD", "d_dt_bias")]


class MixerStages(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("x", "p", "dt_codes", "dt_deq", "dt_acc", "y")]


class SsmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None
EXPORTS = ["ssm_abi_version", "ssm_status_string", "ssm_last_error", "ssm_packed_row_bytes",
           "ssm_ternary_quantize_workspace_bytes", "ssm_ternary_quantize_weights", "ssm_bitlinear_workspace_bytes",
           "ssm_bitlinear_fwd", "ssm_selective_scan_workspace_bytes", "ssm_selective_scan_fwd", "ssm_selective_scan_fwd_noalloc",
           "ssm_dt_input_quantize",
           "ssm_mixer_workspace_bytes", "ssm_mixer_fwd", "ssm_mixer_fwd_stages", "ssm_mixer_fuses_front", "ssm_mixer_step",
           "ssm_mixer_stack_workspace_bytes", "ssm_mixer_stack_step",
           "ssm_conv1d_silu_fwd", "ssm_dense_fwd", "ssm_bitlinear_bwd_workspace_bytes", "ssm_bitlinear_bwd",
           "ssm_qat_sgd_step", "ssm_selective_scan_bwd_workspace_bytes", "ssm_selective_scan_bwd",
           "ssm_mixer_bwd_workspace_bytes", "ssm_mixer_bwd"]


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                               "g.build()'` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        L.ssm_abi_version.restype = ctypes.c_int
        L.ssm_status_string.argtypes = [ctypes.c_int]
        L.ssm_status_string.restype = ctypes.c_char_p
        L.ssm_last_error.restype = ctypes.c_char_p
        L.ssm_packed_row_bytes.argtypes = [_i64]
        L.ssm_packed_row_bytes.restype = _i64
        L.ssm_ternary_quantize_workspace_bytes.argtypes = [_i64, _i64, _i64, _vp]
        L.ssm_ternary_quantize_workspace_bytes.restype = _sz
        L.ssm_ternary_quantize_weights.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.ssm_ternary_quantize_weights.restype = ctypes.c_int
        L.ssm_bitlinear_workspace_bytes.argtypes = [ctypes.POINTER(BitlinearArgs)]
        L.ssm_bitlinear_workspace_bytes.restype = _sz
        L.ssm_bitlinear_fwd.argtypes = [ctypes.POINTER(BitlinearArgs), _vp, _sz, _vp]
        L.ssm_bitlinear_fwd.restype = ctypes.c_int
        L.ssm_selective_scan_workspace_bytes.argtypes = [ctypes.POINTER(ScanArgs)]
        L.ssm_selective_scan_workspace_bytes.restype = _sz
        L.ssm_selective_scan_fwd.argtypes = [ctypes.POINTER(ScanArgs), _vp, _sz, _vp]
        L.ssm_selective_scan_fwd.restype = ctypes.c_int
        L.ssm_selective_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ScanArgs), _vp]
        L.ssm_selective_scan_fwd_noalloc.restype = ctypes.c_int
        L.ssm_dt_input_quantize.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, ctypes.c_float, _vp, _vp, _vp]
        L.ssm_dt_input_quantize.restype = ctypes.c_int
        L.ssm_mixer_workspace_bytes.argtypes = [ctypes.POINTER(MixerConfig), _i64, _i64]
        L.ssm_mixer_workspace_bytes.restype = _sz
        L.ssm_mixer_fuses_front.argtypes = [ctypes.POINTER(MixerConfig)]
        L.ssm_mixer_fuses_front.restype = ctypes.c_int32
        L.ssm_mixer_step.argtypes = [ctypes.POINTER(MixerConfig), ctypes.POINTER(MixerWeights), _vp, _vp, _i64,
                                     _vp, _vp, ctypes.c_int32, _vp, _sz, _vp]
        L.ssm_conv1d_silu_fwd.argtypes = [_vp, _i32, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _vp]
        L.ssm_conv1d_silu_fwd.restype = ctypes.c_int
        L.ssm_dense_fwd.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
        L.ssm_dense_fwd.restype = ctypes.c_int
        L.ssm_bitlinear_bwd_workspace_bytes.argtypes = [ctypes.POINTER(BitlinearBwdArgs)]
        L.ssm_bitlinear_bwd_workspace_bytes.restype = _sz
        L.ssm_bitlinear_bwd.argtypes = [ctypes.POINTER(BitlinearBwdArgs), _vp, _sz, _vp]
        L.ssm_bitlinear_bwd.restype = ctypes.c_int
        L.ssm_qat_sgd_step.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_float, ctypes.c_float, _vp, _vp,
                                       _vp, _sz, _vp]
        L.ssm_qat_sgd_step.restype = ctypes.c_int
        L.ssm_selective_scan_bwd_workspace_bytes.argtypes = [ctypes.POINTER(ScanBwdArgs)]
        L.ssm_selective_scan_bwd_workspace_bytes.restype = _sz
        L.ssm_selective_scan_bwd.argtypes = [ctypes.POINTER(ScanBwdArgs), _vp, _sz, _vp]
        L.ssm_selective_scan_bwd.restype = ctypes.c_int
        L.ssm_mixer_bwd_workspace_bytes.argtypes = [ctypes.POINTER(MixerConfig), _i64, _i64]
        L.ssm_mixer_bwd_workspace_bytes.restype = _sz
        L.ssm_mixer_bwd.argtypes = [ctypes.POINTER(MixerConfig), ctypes.POINTER(MixerWeights),
                                    ctypes.POINTER(MixerGrads), _vp, _vp, _vp, _i64, _i64, _i32, _vp, _sz, _vp]
        L.ssm_mixer_bwd.restype = ctypes.c_int
        L.ssm_mixer_step.restype = ctypes.c_int
        L.ssm_mixer_stack_workspace_bytes.argtypes = [ctypes.POINTER(MixerConfig), _i64]
        L.ssm_mixer_stack_workspace_bytes.restype = _sz
        L.ssm_mixer_stack_step.argtypes = [ctypes.POINTER(MixerConfig), ctypes.POINTER(ctypes.POINTER(MixerWeights)),
                                           _i32, _vp, _vp, _i64, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32, _vp,
                                           _sz, _vp]
        L.ssm_mixer_stack_step.restype = ctypes.c_int
        L.ssm_mixer_fwd.argtypes = [ctypes.POINTER(MixerConfig), ctypes.POINTER(MixerWeights), _vp, _vp, _i64, _i64,
                                    _i32, _vp, _sz, _vp]
        L.ssm_mixer_fwd.restype = ctypes.c_int
        L.ssm_mixer_fwd_stages.argtypes = [ctypes.POINTER(MixerConfig), ctypes.POINTER(MixerWeights), _vp, _vp, _i64,
                                           _i64, _i32, _vp, _sz, ctypes.POINTER(MixerStages), _vp]
        L.ssm_mixer_fwd_stages.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        L = lib()
        raise SsmError(status, f"{L.ssm_status_string(status).decode()}: {L.ssm_last_error().decode()}")


def _p(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _rows(t: torch.Tensor, name: str):
    """(row count, row stride) of a token-major tensor whose last dim is contiguous."""
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")
    if t.dim() == 2:
        return t.shape[0], t.stride(0)
    if t.dim() == 3:
        if t.shape[0] > 1 and t.stride(0) != t.shape[1] * t.stride(1):
            raise ValueError(f"{name}: rows of all batches must be evenly strided")
        return t.shape[0] * t.shape[1], t.stride(1)
    raise ValueError(f"{name}: expected 2 or 3 dims")


def _workspace(nbytes: int, device, workspace=None):
    if nbytes == 0:
        return None
    if workspace is not None and workspace.numel() >= nbytes:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points

def ssm_abi_version() -> int:
    return lib().ssm_abi_version()


def ssm_packed_row_bytes(k: int) -> int:
    return int(lib().ssm_packed_row_bytes(k))


def ssm_ternary_quantize_weights(w: torch.Tensor, group_size: int = 0, scale_in: torch.Tensor | None = None,
                                 stream=None):
    """Absmean ternarisation + 2-bit packing.  Returns (packed uint8 [n, row_bytes], scale fp32
    [1] or [n, k/group], zero_count int64 [1])."""
    if w.dtype != torch.float32 or w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D float32 tensor")
    n, k = w.shape
    L = lib()
    packed = torch.empty((n, ssm_packed_row_bytes(k)), dtype=torch.uint8, device=w.device)
    scale = torch.empty((1,) if group_size == 0 else (n, max(1, k // max(group_size, 1))), dtype=torch.float32,
                        device=w.device)
    zc = torch.empty(1, dtype=torch.int64, device=w.device)
    nb = L.ssm_ternary_quantize_workspace_bytes(n, k, group_size, _p(scale_in))
    ws = _workspace(nb, w.device)
    _check(L.ssm_ternary_quantize_weights(_p(w), n, k, group_size, _p(scale_in), _p(packed), _p(scale), _p(zc),
                                          _p(ws), nb, _stream(stream)))
    return packed, scale, zc


def ssm_bitlinear_fwd(x: torch.Tensor, w_packed: torch.Tensor, w_scale: torch.Tensor, n_out: int, *,
                      act_bits: int = 8, group_size: int = 0, k: int | None = None,
                      x_absmax: torch.Tensor | None = None, norm_weight: torch.Tensor | None = None,
                      norm_eps: float = 1e-5, bias: torch.Tensor | None = None,
                      residual: torch.Tensor | None = None, y_dtype: torch.dtype | None = None,
                      out: torch.Tensor | None = None, debug: bool = False, workspace: torch.Tensor | None = None,
                      stream=None):
    """RMSNorm -> (int8 absmax | bf16) -> ternary contraction -> rescale (+ bias) (+ residual).
    x: [m, >= k] (or [B, L, >= k]) rows with a contiguous last dimension.  Returns y [m, n_out]
    (or (y, xq, absmax, acc) with debug=True)."""
    m, ldx = _rows(x, "x")
    k = x.shape[-1] if k is None else k
    y_dtype = (x.dtype if x.dtype != torch.int8 else torch.float32) if y_dtype is None else y_dtype
    if out is None:
        out = torch.empty((m, n_out), dtype=y_dtype, device=x.device)
    ym, ldy = _rows(out, "out")
    a = BitlinearArgs()
    a.x, a.x_dtype, a.act_bits = _p(x), _DTYPES[x.dtype], act_bits
    a.m, a.k, a.ldx = m, k, ldx
    a.x_absmax, a.norm_weight, a.norm_eps = _p(x_absmax), _p(norm_weight), norm_eps
    a.w_packed, a.w_scale, a.n_out, a.group_size = _p(w_packed), _p(w_scale), n_out, group_size
    a.bias = _p(bias)
    if residual is not None:
        _, a.ld_res = _rows(residual, "residual")
        a.residual = _p(residual)
    a.y, a.y_dtype, a.ldy = _p(out), _DTYPES[out.dtype], ldy
    dbg = None
    if debug:
        dbg = (torch.empty((m, k), dtype=torch.int8, device=x.device),
               torch.empty(m, dtype=torch.float32, device=x.device),
               torch.empty((m, n_out), dtype=torch.int32, device=x.device))
        a.dbg_xq, a.dbg_absmax, a.dbg_acc = (_p(t) for t in dbg)
    L = lib()
    nb = L.ssm_bitlinear_workspace_bytes(ctypes.byref(a))
    ws = _workspace(nb, x.device, workspace)
    _check(L.ssm_bitlinear_fwd(ctypes.byref(a), _p(ws), nb if ws is None else ws.numel(), _stream(stream)))
    return (out, *dbg) if debug else out


def ssm_selective_scan_fwd(x: torch.Tensor, delta: torch.Tensor | None, A: torch.Tensor, Bm: torch.Tensor,
                           Cm: torch.Tensor, D: torch.Tensor | None = None, delta_bias: torch.Tensor | None = None,
                           softplus: bool = True, h0: torch.Tensor | None = None, return_last_state: bool = False,
                           out: torch.Tensor | None = None, dt_proj: dict | None = None,
                           gate: torch.Tensor | None = None, noalloc: bool = False, stream=None):
    """Selective scan (noalloc: through ssm_selective_scan_fwd_noalloc, the library's own scratch).  x [B, L, H*P], delta [B, L, H], Bm/Cm [B, L, N]; A [H, N] (Mamba-1 kind,
    P = 1) or [H] (SSD kind).  Views with a contiguous last dim and even row strides are fine.
    dt_proj (Mamba-1 kind): dict(dt_in [B, L, >= R] view, w_dt packed [H, row bytes], s_dt [1],
    dt_rank R, optional g_dt, eps): dt is the A8 BitLinear of dt_in computed inside the scan
    (delta is then ignored and may be None).  gate [B, L, H*P] (optional): y is multiplied by
    SiLU(gate) before it is stored."""
    batch, seqlen, HP = x.shape
    H = A.shape[0] if A.dim() == 2 else (delta.shape[2] if delta is not None else A.shape[0])
    N = Bm.shape[2]
    aps = 1 if A.dim() == 2 else 0
    if out is None:
        out = torch.empty((batch, seqlen, HP), dtype=x.dtype, device=x.device)
    hl = torch.empty((batch, H, HP // H, N), dtype=torch.float32, device=x.device) if return_last_state else None
    a = ScanArgs()
    a.batch, a.seqlen, a.nheads, a.headdim, a.d_state = batch, seqlen, H, HP // H, N
    a.a_per_state, a.act_dtype = aps, _DTYPES[x.dtype]
    a.x, a.ld_x = _p(x), _rows(x, "x")[1]
    if delta is not None:
        a.delta, a.ld_delta = _p(delta), _rows(delta, "delta")[1]
    if dt_proj is not None:
        a.dt_in, a.ld_dt_in = _p(dt_proj["dt_in"]), _rows(dt_proj["dt_in"], "dt_in")[1]
        a.dt_rank, a.w_dt, a.s_dt = dt_proj["dt_rank"], _p(dt_proj["w_dt"]), _p(dt_proj["s_dt"])
        a.g_dt, a.dt_eps = _p(dt_proj.get("g_dt")), dt_proj.get("eps", 1e-5)
        if dt_proj.get("dt_codes") is not None:  # precomputed by ssm_dt_input_quantize
            a.dt_codes, a.dt_deq = _p(dt_proj["dt_codes"]), _p(dt_proj["dt_deq"])
    a.delta_bias, a.delta_softplus = _p(delta_bias), int(softplus)
    a.A = _p(A)
    a.Bm, a.ld_B = _p(Bm), _rows(Bm, "Bm")[1]
    a.Cm, a.ld_C = _p(Cm), _rows(Cm, "Cm")[1]
    a.D, a.h0, a.h_last = _p(D), _p(h0), _p(hl)
    a.y, a.ld_y = _p(out), _rows(out, "out")[1]
    if gate is not None:
        a.gate, a.ld_gate = _p(gate), _rows(gate, "gate")[1]
    L = lib()
    if noalloc:
        _check(L.ssm_selective_scan_fwd_noalloc(ctypes.byref(a), _stream(stream)))
        return (out, hl) if return_last_state else out
    nb = L.ssm_selective_scan_workspace_bytes(ctypes.byref(a))
    ws = _workspace(nb, x.device)
    _check(L.ssm_selective_scan_fwd(ctypes.byref(a), _p(ws), nb, _stream(stream)))
    return (out, hl) if return_last_state else out


def ssm_dt_input_quantize(dt_in: torch.Tensor, dt_rank: int, g_dt: torch.Tensor | None = None, eps: float = 1e-5,
                          stream=None):
    """int8 codes [M, 16 ceil(R / 16)] and fp64 factors [M] of the dt input's rows (dt_in [..., >= R],
    a contiguous last dim), as the scan's dt projection computes them."""
    m, ld = _rows(dt_in, "dt_in")
    codes = torch.empty((m, 16 * ((dt_rank + 15) // 16)), dtype=torch.int8, device=dt_in.device)
    deq = torch.empty(m, dtype=torch.float64, device=dt_in.device)
    _check(lib().ssm_dt_input_quantize(_p(dt_in), _DTYPES[dt_in.dtype], m, dt_rank, ld, _p(g_dt), eps, _p(codes),
                                       _p(deq), _stream(stream)))
    return codes, deq


def mixer_config(kind: int, d_model: int, d_inner: int, d_state: int, *, dt_rank: int = 0, nheads: int = 0,
                 headdim: int = 0, act_bits: int = 8, group_size: int = 0, act_dtype: torch.dtype = torch.float32,
                 norm_eps: float = 1e-5, gated: int = 0, d_conv: int = 0, fp_proj: int = 0) -> MixerConfig:
    c = MixerConfig()
    c.gated, c.d_conv, c.fp_proj = gated, d_conv, fp_proj
    c.kind, c.act_bits = kind, act_bits
    c.d_model, c.d_inner, c.d_state, c.dt_rank = d_model, d_inner, d_state, dt_rank
    c.nheads, c.headdim, c.group_size = nheads, headdim, group_size
    c.act_dtype, c.norm_eps = _DTYPES[act_dtype], norm_eps
    return c


def ssm_mixer_fuses_front(cfg: MixerConfig) -> bool:
    return bool(lib().ssm_mixer_fuses_front(ctypes.byref(cfg)))


def ssm_mixer_workspace_bytes(cfg: MixerConfig, batch: int, seqlen: int) -> int:
    return int(lib().ssm_mixer_workspace_bytes(ctypes.byref(cfg), batch, seqlen))


def mixer_weights(w: dict) -> MixerWeights:
    """w: packed weights w_in/w_x/w_dt/w_out, scales s_*, optional gains g_*, dt_bias, A, D (device tensors)."""
    mw = MixerWeights()
    for name, _ in MixerWeights._fields_:
        setattr(mw, name, _p(w.get(name)))
    return mw


def ssm_mixer_fwd(cfg: MixerConfig, weights, u: torch.Tensor, add_residual: bool = True,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """One mixer layer on u [B, L, d_model] (contiguous).  weights: MixerWeights or dict."""
    if not u.is_contiguous():
        raise ValueError("u must be contiguous")
    batch, seqlen, _ = u.shape
    mw = weights if isinstance(weights, MixerWeights) else mixer_weights(weights)
    if out is None:
        out = torch.empty_like(u)
    L = lib()
    nb = L.ssm_mixer_workspace_bytes(ctypes.byref(cfg), batch, seqlen)
    ws = _workspace(nb, u.device, workspace)
    _check(L.ssm_mixer_fwd(ctypes.byref(cfg), ctypes.byref(mw), _p(u), _p(out), batch, seqlen, int(add_residual),
                           _p(ws), nb if ws is None else ws.numel(), _stream(stream)))
    return out


def ssm_mixer_fwd_stages(cfg: MixerConfig, weights, u: torch.Tensor, add_residual: bool = True,
                         want=("x", "p", "dt_codes", "dt_deq", "dt_acc", "y"), stream=None):
    """ssm_mixer_fwd with its stages copied out: returns (out, dict of the stages in `want`):
    x [M, d_inner], p [M, PW] (SSD: v), y [M, d_inner] in the act dtype; dt_codes int8 [M, dt_rank],
    dt_deq fp64 [M], dt_acc int32 [M, d_inner] (Mamba-1 kind)."""
    if not u.is_contiguous():
        raise ValueError("u must be contiguous")
    batch, seqlen, _ = u.shape
    M = batch * seqlen
    mw = weights if isinstance(weights, MixerWeights) else mixer_weights(weights)
    act = {SSM_F32: torch.float32, SSM_BF16: torch.bfloat16}[cfg.act_dtype]
    if cfg.kind == SSM_MIXER_MAMBA1:
        pw = cfg.dt_rank + 2 * cfg.d_state
    else:
        pw = cfg.d_inner + 2 * cfg.d_state + cfg.nheads + (cfg.d_inner if cfg.gated else 0)
    shapes = {"x": ((M, cfg.d_inner), act), "p": ((M, pw), act), "dt_codes": ((M, cfg.dt_rank), torch.int8),
              "dt_deq": ((M,), torch.float64), "dt_acc": ((M, cfg.d_inner), torch.int32), "y": ((M, cfg.d_inner), act)}
    got = {k: torch.empty(shapes[k][0], dtype=shapes[k][1], device=u.device) for k in want}
    st = MixerStages()
    for k, t in got.items():
        setattr(st, k, _p(t))
    out = torch.empty_like(u)
    L = lib()
    nb = L.ssm_mixer_workspace_bytes(ctypes.byref(cfg), batch, seqlen)
    ws = _workspace(nb, u.device)
    _check(L.ssm_mixer_fwd_stages(ctypes.byref(cfg), ctypes.byref(mw), _p(u), _p(out), batch, seqlen,
                                  int(add_residual), _p(ws), nb, ctypes.byref(st), _stream(stream)))
    return out, got


def ssm_mixer_step(cfg: MixerConfig, weights, u: torch.Tensor, state: torch.Tensor, add_residual: bool = True,
                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   conv_state: torch.Tensor | None = None, stream=None):
    """One decoding step on u [B, d_model] (one token per sequence); state (and, for the gated
    block, conv_state [B, d_conv - 1, channels]) (fp32, contiguous) are read and overwritten
    in place."""
    if not u.is_contiguous() or not state.is_contiguous():
        raise ValueError("u and state must be contiguous")
    if state.dtype != torch.float32 or (conv_state is not None and conv_state.dtype != torch.float32):
        raise ValueError("state and conv_state must be float32")
    if conv_state is not None and not conv_state.is_contiguous():
        raise ValueError("conv_state must be contiguous")
    batch = u.shape[0]
    mw = weights if isinstance(weights, MixerWeights) else mixer_weights(weights)
    if out is None:
        out = torch.empty_like(u)
    L = lib()
    nb = L.ssm_mixer_workspace_bytes(ctypes.byref(cfg), batch, 1)
    ws = _workspace(nb, u.device, workspace)
    _check(L.ssm_mixer_step(ctypes.byref(cfg), ctypes.byref(mw), _p(u), _p(out), batch, _p(state), _p(conv_state),
                            int(add_residual), _p(ws), nb if ws is None else ws.numel(), _stream(stream)))
    return out


def ssm_mixer_stack_workspace_bytes(cfg: MixerConfig, batch: int) -> int:
    return int(lib().ssm_mixer_stack_workspace_bytes(ctypes.byref(cfg), batch))


def ssm_mixer_stack_step(cfg: MixerConfig, weights: list, u: torch.Tensor, states: list, add_residual: bool = True,
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         conv_states: list | None = None, stream=None):
    """One decoding step through a stack of layers (weights[l], states[l]; the output of layer l
    feeds layer l + 1) on u [B, d_model]; every state (fp32, contiguous) is read and overwritten
    in place.  Equal to ssm_mixer_step applied layer by layer."""
    n = len(weights)
    if len(states) != n or (conv_states is not None and len(conv_states) != n):
        raise ValueError("one state (and conv_state) per layer")
    if not u.is_contiguous() or any(not t.is_contiguous() or t.dtype != torch.float32 for t in states):
        raise ValueError("u and the states must be contiguous, the states float32")
    mws = [w if isinstance(w, MixerWeights) else mixer_weights(w) for w in weights]
    wp = (ctypes.POINTER(MixerWeights) * n)(*[ctypes.pointer(m) for m in mws])
    sp = (_vp * n)(*[t.data_ptr() for t in states])
    cp = None if conv_states is None else (_vp * n)(*[_p(t) for t in conv_states])
    batch = u.shape[0]
    if out is None:
        out = torch.empty_like(u)
    L = lib()
    nb = L.ssm_mixer_stack_workspace_bytes(ctypes.byref(cfg), batch)
    ws = _workspace(nb, u.device, workspace)
    _check(L.ssm_mixer_stack_step(ctypes.byref(cfg), wp, n, _p(u), _p(out), batch, sp, cp, int(add_residual), _p(ws),
                                  nb if ws is None else ws.numel(), _stream(stream)))
    return out


def ssm_selective_scan_bwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor, Cm: torch.Tensor,
                           dy: torch.Tensor, D: torch.Tensor | None = None, delta_bias: torch.Tensor | None = None,
                           softplus: bool = True, h0: torch.Tensor | None = None, stream=None) -> dict:
    """Backward of the Mamba-1 kind scan: x, delta [B, L, H], Bm/Cm [B, L, N] (views with a
    contiguous last dim), A [H, N], dy fp32 [B, L, H].  Returns fp32 gradients dx, ddelta,
    dA, dB, dC, dD, dbias, dh0."""
    batch, L, H = x.shape
    N = Bm.shape[2]
    dev = x.device
    f = dict(dtype=torch.float32, device=dev)
    g = dict(dx=torch.empty((batch, L, H), **f), ddelta=torch.empty((batch, L, H), **f), dA=torch.empty((H, N), **f),
             dB=torch.empty((batch, L, N), **f), dC=torch.empty((batch, L, N), **f), dD=torch.empty(H, **f),
             dbias=torch.empty(H, **f), dh0=torch.empty((batch, H, N), **f))
    a = ScanBwdArgs()
    a.batch, a.seqlen, a.nheads, a.d_state = batch, L, H, N
    a.act_dtype, a.delta_softplus = _DTYPES[x.dtype], int(softplus)
    a.x, a.ld_x = _p(x), _rows(x, "x")[1]
    a.delta, a.ld_delta = _p(delta), _rows(delta, "delta")[1]
    a.delta_bias, a.A = _p(delta_bias), _p(A)
    a.Bm, a.ld_B = _p(Bm), _rows(Bm, "Bm")[1]
    a.Cm, a.ld_C = _p(Cm), _rows(Cm, "Cm")[1]
    a.D, a.h0 = _p(D), _p(h0)
    a.dy, a.ld_dy = _p(dy), _rows(dy, "dy")[1]
    for k, v in g.items():
        setattr(a, k, _p(v))
    L_ = lib()
    nb = L_.ssm_selective_scan_bwd_workspace_bytes(ctypes.byref(a))
    ws = _workspace(nb, dev)
    _check(L_.ssm_selective_scan_bwd(ctypes.byref(a), _p(ws), nb, _stream(stream)))
    return g


def ssm_mixer_bwd_workspace_bytes(cfg: MixerConfig, batch: int, seqlen: int) -> int:
    return int(lib().ssm_mixer_bwd_workspace_bytes(ctypes.byref(cfg), batch, seqlen))


def ssm_mixer_bwd(cfg: MixerConfig, weights, u: torch.Tensor, dout: torch.Tensor, add_residual: bool = True,
                  latents: dict | None = None, workspace: torch.Tensor | None = None, stream=None) -> dict:
    """Backward of one Mamba-1 kind mixer layer: u, dout fp32 [B, L, d_model] (contiguous).
    latents (optional): latent weights lat_in / lat_x / lat_dt / lat_out, which add the scale
    gradients.  Returns fp32 du, dw_in, dw_x, dw_dt, dw_out, dA, dD, d_dt_bias (and ds_* with
    latents)."""
    if not u.is_contiguous() or not dout.is_contiguous():
        raise ValueError("u and dout must be contiguous")
    if dout.dtype != torch.float32:
        raise ValueError("dout must be float32")
    batch, seqlen, dm = u.shape
    di, n, r = cfg.d_inner, cfg.d_state, cfg.dt_rank
    pw = r + 2 * n
    dev = u.device
    f = dict(dtype=torch.float32, device=dev)
    out = dict(du=torch.empty((batch, seqlen, dm), **f), dw_in=torch.empty((di, dm), **f),
               dw_x=torch.empty((pw, di), **f), dw_dt=torch.empty((di, r), **f), dw_out=torch.empty((dm, di), **f),
               dA=torch.empty((di, n), **f), dD=torch.empty(di, **f), d_dt_bias=torch.empty(di, **f))
    g = MixerGrads()
    for k in ("dw_in", "dw_x", "dw_dt", "dw_out", "dA", "dD", "d_dt_bias"):
        setattr(g, k, _p(out[k]))
    if latents:
        for k in ("in", "x", "dt", "out"):
            lat = latents.get("lat_" + k)
            if lat is not None:
                out["ds_" + k] = torch.empty(1, **f)
                setattr(g, "lat_" + k, _p(lat))
                setattr(g, "ds_" + k, _p(out["ds_" + k]))
    mw = weights if isinstance(weights, MixerWeights) else mixer_weights(weights)
    L = lib()
    nb = L.ssm_mixer_bwd_workspace_bytes(ctypes.byref(cfg), batch, seqlen)
    ws = _workspace(nb, dev, workspace)
    _check(L.ssm_mixer_bwd(ctypes.byref(cfg), ctypes.byref(mw), ctypes.byref(g), _p(u), _p(dout), _p(out["du"]),
                           batch, seqlen, int(add_residual), _p(ws), nb if ws is None else ws.numel(),
                           _stream(stream)))
    return out


def ssm_bitlinear_bwd(x: torch.Tensor, w_packed: torch.Tensor, w_scale: torch.Tensor, n_out: int,
                      dy: torch.Tensor, group_size: int = 0, norm_weight: torch.Tensor | None = None,
                      norm_eps: float = 1e-5, w_latent: torch.Tensor | None = None, want_dw: bool = True,
                      stream=None):
    """Straight-through-estimator backward of the A8 BitLinear.  x [m, k] (fp32 / bf16, rows with
    a contiguous last dim), dy [m, n_out] fp32.  Returns (dx fp32 [m, k], dw fp32 [n_out, k] or
    None, d_scale fp32 or None -- d_scale when w_latent is given)."""
    m, ldx = _rows(x, "x")
    k = x.shape[-1]
    if dy.dtype != torch.float32:
        raise ValueError("dy must be float32")
    dx = torch.empty((m, k), dtype=torch.float32, device=x.device)
    dw = torch.empty((n_out, k), dtype=torch.float32, device=x.device) if (want_dw or w_latent is not None) else None
    ns = 1 if group_size == 0 else n_out * (k // group_size)
    ds = torch.empty(ns, dtype=torch.float32, device=x.device) if w_latent is not None else None
    a = BitlinearBwdArgs()
    a.x, a.x_dtype, a.m, a.k, a.ldx = _p(x), _DTYPES[x.dtype], m, k, ldx
    a.norm_weight, a.norm_eps = _p(norm_weight), norm_eps
    a.w_packed, a.w_scale, a.n_out, a.group_size = _p(w_packed), _p(w_scale), n_out, group_size
    a.w_latent = _p(w_latent)
    a.dy, a.ld_dy = _p(dy), _rows(dy, "dy")[1]
    a.dx, a.ld_dx = _p(dx), k
    a.dw, a.d_scale = _p(dw), _p(ds)
    L = lib()
    nb = L.ssm_bitlinear_bwd_workspace_bytes(ctypes.byref(a))
    ws = _workspace(nb, x.device)
    _check(L.ssm_bitlinear_bwd(ctypes.byref(a), _p(ws), nb, _stream(stream)))
    return dx, dw, ds


def ssm_qat_sgd_step(w_latent: torch.Tensor, w_scale: torch.Tensor, dw: torch.Tensor, d_scale: torch.Tensor | None,
                     lr: float, lr_scale: float, group_size: int = 0, w_packed: torch.Tensor | None = None,
                     stream=None):
    """One QAT step in place on w_latent [n, k] and w_scale; returns (w_packed, zero count tensor)."""
    n, k = w_latent.shape
    if w_packed is None:
        w_packed = torch.empty((n, ssm_packed_row_bytes(k)), dtype=torch.uint8, device=w_latent.device)
    zc = torch.zeros(1, dtype=torch.int64, device=w_latent.device)
    _check(lib().ssm_qat_sgd_step(_p(w_latent), _p(w_scale), _p(dw), _p(d_scale), n, k, group_size, lr, lr_scale,
                                  _p(w_packed), _p(zc), None, 0, _stream(stream)))
    return w_packed, zc


def ssm_dense_fwd(x: torch.Tensor, w: torch.Tensor, residual: torch.Tensor | None = None,
                  out: torch.Tensor | None = None, stream=None):
    """Full-precision linear layer y = x W^T (+ residual); x [m, k] or [B, L, k] (contiguous last
    dim, even row strides), w [n, k] of x's dtype (fp32 or bf16)."""
    m, ldx = _rows(x, "x")
    n, k = w.shape
    if out is None:
        out = torch.empty((*x.shape[:-1], n), dtype=x.dtype, device=x.device)
    ld_res = _rows(residual, "residual")[1] if residual is not None else 0
    _check(lib().ssm_dense_fwd(_p(x), _DTYPES[x.dtype], m, k, ldx, _p(w.contiguous()), n, _p(residual), ld_res,
                               _p(out), _rows(out, "out")[1], _stream(stream)))
    return out


def ssm_conv1d_silu_fwd(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None = None,
                        state_in: torch.Tensor | None = None, state_out: torch.Tensor | None = None,
                        channels: int | None = None, out: torch.Tensor | None = None, stream=None):
    """Causal depthwise convolution of width w.shape[1] + SiLU on the first `channels` columns
    of x [B, L, ldx] (a view with a contiguous last dim).  state_in / state_out: fp32
    [B, width - 1, channels] (optional; may be the same tensor)."""
    batch, seqlen, _ = x.shape
    C = w.shape[0] if channels is None else channels
    if out is None:
        out = torch.empty((batch, seqlen, C), dtype=x.dtype, device=x.device)
    _check(lib().ssm_conv1d_silu_fwd(_p(x), _DTYPES[x.dtype], batch, seqlen, C, _rows(x, "x")[1], _p(w),
                                     int(w.shape[1]), _p(bias), _p(state_in), _p(state_out), _p(out),
                                     _rows(out, "out")[1], _stream(stream)))
    return out
