"""Shared helpers of the GPU parity tests (marshalling seeded inputs to both sides)."""
import json
import os

import numpy as np
import torch

import oracle
import ternary_weight_selective_amd as tws
import workloads as wl

DEV = torch.device("cuda:0")

# Tolerances (norm-wise relative error per output tensor): fp32 outputs 1e-4, bf16 outputs 2e-2.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def elem_err(got, ref) -> np.ndarray:
    """Per element |y - y_ref| / (|y_ref| + rms(y_ref)): a localised error (one channel, the
    last chunk of each sequence) shows at full size here, where the norm-wise ratio dilutes it."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return np.abs(got - ref) / (np.abs(ref) + (rms if rms > 0 else 1.0))


def check(got, ref, tol: float, *, elem: float | None = None, frac: float = 0.0, what: str = "") -> dict:
    """Float parity of one output tensor.
      norm-wise relative error <= tol;
      every element's elem_err <= elem (default: tol itself);
      at most a fraction `frac` of the elements above tol (default: none).
    The looser `elem` / `frac` are for outputs behind a chain of int8 quantisers, where a
    one-ulp float difference upstream may legitimately move a code across a .5 boundary and
    shift the values it feeds by a quantisation step.  Metrics are appended to the file named
    by the PARITY_LOG environment variable, when set."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    n = rel_err(got, ref)
    e = elem_err(got, ref)
    emax = float(e.max()) if e.size else 0.0
    above = float(np.mean(e > tol)) if e.size else 0.0
    elem = tol if elem is None else elem
    m = {"what": what, "norm": n, "elem_max": emax, "frac_above_tol": above, "tol": tol, "elem": elem,
         "frac": frac, "size": int(e.size)}
    path = os.environ.get("PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(m) + "\n")
    assert n <= tol, m
    assert emax <= elem, m
    assert above <= frac, m
    return m


# Outputs behind a chain of rounded stages, compared end to end (whole mixer layers):
#  fp32: int8 quantisers in the chain; an element may be off by a few quantisation steps of
#   the codes a boundary flip moved (a step of out_proj's codes is s_w max|y| / 127, about 5e-4
#   of the output's rms at the TriSSM shape), and such elements must stay rare;
#  bf16: every stored activation is rounded to bf16 and the A16 projections take x_hat as bf16,
#   so dt, B, C and x differ by bf16 steps before the scan, and the decays exp(A sum dt) scale a
#   dt difference by |A sum dt|: single elements of a layer's output move by a few 1e-2 while
#   each stage fed the previous stage's values stays within 2e-2 (tested stage by stage).
CHAIN = {"f32": {"elem": 5e-3, "frac": 5e-3}, "bf16_a16": {"elem": 6e-2, "frac": 1e-3}}


def chain(dtype_name: str, a16: bool = False) -> dict:
    """Bounds for a whole layer's output; bf16 outputs of int8-activation layers keep the bf16
    bound itself (their projections' stored outputs are exact up to the final rounding)."""
    if dtype_name == "f32":
        return CHAIN["f32"]
    return CHAIN["bf16_a16"] if a16 else {}


def to_dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dtype)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def bf16_values(a) -> np.ndarray:
    """The values a bf16 tensor made from `a` holds (torch's round-to-nearest-even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def torch_dtype(cfg) -> torch.dtype:
    return torch.bfloat16 if cfg.act_dtype == "bf16" else torch.float32


def quantize_layer(cfg, lat, check: bool = True):
    """Ternarise one layer on the GPU and in the oracle; (gpu weight dict, oracle weight dict)."""
    gw, ow = {}, {}
    for name in cfg.proj_shapes:
        w = lat["W_" + name]
        if cfg.is_fp(name):  # full-precision projection: the weights as stored in the act dtype
            wv = bf16_values(w) if cfg.act_dtype == "bf16" else w
            gw["fw_" + name] = to_dev(wv, torch_dtype(cfg))
            ow["f_" + name] = wv
            continue
        packed, scale, zc = tws.ssm_ternary_quantize_weights(to_dev(w), cfg.group_size)
        codes, oscale, ozeros = oracle.quantize_weights(w, cfg.group_size)
        if check:
            assert np.array_equal(host(packed), oracle.pack(codes)), name
            assert np.array_equal(host(scale).ravel(), np.asarray(oscale).ravel()), name
            assert int(host(zc)[0]) == ozeros, name
        gw["w_" + name], gw["s_" + name] = packed, scale
        ow["c_" + name], ow["s_" + name] = codes, oscale
    for key in ("A", "D", "dt_bias", "conv_w", "conv_b"):
        if key in lat:
            gw[key] = to_dev(lat[key])
            ow[key] = lat[key]
    return gw, ow


def gpu_config(cfg):
    return tws.mixer_config(cfg.kind, cfg.d_model, cfg.d_inner, cfg.d_state, dt_rank=cfg.dt_rank,
                            nheads=cfg.nheads, headdim=cfg.headdim, act_bits=cfg.act_bits,
                            group_size=cfg.group_size, act_dtype=torch_dtype(cfg), norm_eps=cfg.norm_eps,
                            gated=cfg.gated, d_conv=cfg.d_conv, fp_proj=cfg.fp_proj)


def oracle_config(cfg):
    return dict(kind=cfg.kind, d_model=cfg.d_model, d_inner=cfg.d_inner, d_state=cfg.d_state, dt_rank=cfg.dt_rank,
                nheads=cfg.nheads, headdim=cfg.headdim, group_size=cfg.group_size, act_bits=cfg.act_bits,
                act_dtype=oracle.BF16 if cfg.act_dtype == "bf16" else oracle.F32, norm_eps=cfg.norm_eps,
                gated=cfg.gated, d_conv=cfg.d_conv, fp_proj=cfg.fp_proj)


def run_gpu_stack(cfg, gws, u_host, workspace=None):
    """out = u + mixer_l(u), layer after layer, in the act dtype; returns the device tensor."""
    c = gpu_config(cfg)
    h = to_dev(u_host, torch_dtype(cfg))
    nb = tws.ssm_mixer_workspace_bytes(c, h.shape[0], h.shape[1])
    ws = workspace if workspace is not None else torch.empty(nb, dtype=torch.uint8, device=DEV)
    mws = [tws.mixer_weights(g) for g in gws]
    for mw in mws:
        h = tws.ssm_mixer_fwd(c, mw, h, add_residual=True, out=h, workspace=ws)
    return h
