#!/usr/bin/env python3
"""Throughput of the ternary selective-SSM mixer forward on one MI355X.

A step is one forward pass of the whole hot path over one batch: for the default
workload, the TriSSM-shaped stack of 12 BitSSM mixer layers (d_model 256, d_inner 512,
d_state 16, dt_rank 16, batch 64 x L 256, fp32 activations, int8 activations into the
ternary projections), out = u + mixer(u) per layer.  Inputs are seeded synthetic data,
resident in HBM before the timed region.  Prints one JSON line.

Also measured, in a second timed loop that runs the same kernels through the stage entry
points with HIP events around each stage: the average duration of every kernel stage, and
the roofline of the dominant one.  The CPU oracle is timed on a bounded sample of the same
workload on the host cores (a reported baseline, not the target).

Also measured: token-by-token decoding of the same stack (one ssm_mixer_step per layer, the
recurrent state carried in HBM), at the workload's batch and at batch 1; and the training side
of one ternary projection (straight-through-estimator backward, one QAT step).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import ternary_weight_selective_amd as tws  # noqa: E402
import workloads as wl  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (FMA = 2 FLOP per lane)
INT8_MFMA_PEAK_TOPS = 5000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_MATRIX_PEAK_TFLOPS = 157.3  # MI355X fp32 on the matrix cores (the full-precision baselines)
# One VALU lane-instruction slot counts as 2 FLOP-equivalents (an FMA); a transcendental
# (v_exp_f32) occupies 4 slots (quarter rate).  The Mamba-1 recurrence needs, per
# (token, channel, state): dt*A, exp2, (dt*x)*B, fma for h, fma for y = 4 slots + 4 slots.
SCAN_M1_SLOTS_PER_STATE_STEP = 8

KERNEL_SOURCES = {  # source files whose text defines each timed kernel (for stale-counter checks)
    "scan_m1": ["scan.hip", "common.hpp", "launch.hpp"],
    "ssd": ["ssd.hip", "common.hpp", "launch.hpp"],
    "bitlinear": ["norm.hip", "bitlinear.hip", "common.hpp", "launch.hpp"],
    "conv": ["conv.hip", "common.hpp", "launch.hpp"],
    "dense": ["dense.cpp", "launch.hpp"],
}


def kernel_src_hash(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "ternary_weight_selective_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="trissm", choices=list(wl.CONFIGS))
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work of the oracle sample")
    ap.add_argument("--stages-only", action="store_true", help="skip the headline loop (profiling runs)")
    ap.add_argument("--no-decode", action="store_true", help="skip the token-by-token decode measurement")
    ap.add_argument("--decode-only", action="store_true", help="only the decode measurement (profiling runs)")
    ap.add_argument("--no-train", action="store_true", help="skip the BitLinear backward / QAT step measurement")
    ap.add_argument("--train-only", action="store_true", help="only the BitLinear backward / QAT step (profiling runs)")
    ap.add_argument("--mixer-bwd-only", action="store_true", help="only the mixer layer backward (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run 3 plain device copies of 1 GiB (reference for HBM byte counters)")
    return ap.parse_args()


# ------------------------------------------------------------------ set-up

class Problem:
    """Device-resident weights, input and buffers of one workload."""

    def __init__(self, cfg: wl.MixerConfig, seed: int, dev):
        self.cfg = cfg
        self.dev = dev
        lat, u = wl.mixer_problem(cfg, seed=seed)
        self.u_host = u
        self.lat0 = lat[0]  # the first layer's latent weights (host), for the training-side timings
        self.act = torch.bfloat16 if cfg.act_dtype == "bf16" else torch.float32
        self.layers = []  # dicts of device tensors
        for lw in lat:
            d = {}
            for name in cfg.proj_shapes:
                if cfg.is_fp(name):  # full-precision projection: dense weights in the act dtype
                    d["fw_" + name] = torch.from_numpy(lw["W_" + name]).to(dev).to(self.act)
                    continue
                packed, scale, _ = tws.ssm_ternary_quantize_weights(
                    torch.from_numpy(lw["W_" + name]).to(dev), cfg.group_size)
                d["w_" + name], d["s_" + name] = packed, scale
            for key in ("A", "D", "dt_bias", "conv_w", "conv_b"):
                if key in lw:
                    d[key] = torch.from_numpy(lw[key]).to(dev)
            self.layers.append(d)
        self.c = tws.mixer_config(cfg.kind, cfg.d_model, cfg.d_inner, cfg.d_state, dt_rank=cfg.dt_rank,
                                  nheads=cfg.nheads, headdim=cfg.headdim, act_bits=cfg.act_bits,
                                  group_size=cfg.group_size, act_dtype=self.act, norm_eps=cfg.norm_eps,
                                  gated=cfg.gated, d_conv=cfg.d_conv, fp_proj=cfg.fp_proj)
        self.mws = [tws.mixer_weights(d) for d in self.layers]
        self.u = torch.from_numpy(u).to(dev).to(self.act)
        self.bufs = [torch.empty_like(self.u), torch.empty_like(self.u)]
        self.ws_bytes = tws.ssm_mixer_workspace_bytes(self.c, cfg.batch, cfg.seqlen)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def step(self, stream_handle):
        """One pass of the stack: out = u + mixer_l(u) layer after layer (ping-pong buffers)."""
        L = tws.lib()
        h = self.u
        cb = ctypes.byref(self.c)
        for i, mw in enumerate(self.mws):
            out = self.bufs[i % 2]
            st = L.ssm_mixer_fwd(cb, ctypes.byref(mw), h.data_ptr(), out.data_ptr(), self.cfg.batch,
                                 self.cfg.seqlen, 1, self.ws.data_ptr(), self.ws_bytes, stream_handle)
            if st != 0:
                raise tws.SsmError(st, L.ssm_last_error().decode())
            h = out
        return h


class StagePlan:
    """The same layer as ssm_mixer_fwd, issued stage by stage through the public entry points
    (identical kernels and arguments), so that HIP events can bracket each stage."""

    def __init__(self, prob: Problem):
        cfg = prob.cfg
        dev = prob.dev
        M = cfg.tokens
        es = 2 if prob.act == torch.bfloat16 else 4
        dt = tws._DTYPES[prob.act]
        self.prob = prob
        self.stages = []  # per layer: list of (name, fn, args ctypes object)
        ZG = cfg.d_inner if cfg.gated else 0  # gate branch columns of the in_proj output
        Cc = cfg.conv_channels
        if cfg.kind == wl.MAMBA1:
            PW = cfg.dt_rank + 2 * cfg.d_state
            XW = cfg.d_inner + ZG
            self.xz = torch.empty((M, XW), dtype=prob.act, device=dev)
            self.x = torch.empty((M, cfg.d_inner), dtype=prob.act, device=dev) if cfg.gated else self.xz
            self.p = torch.empty((M, PW), dtype=prob.act, device=dev)
            self.dl = torch.empty((M, cfg.d_inner), dtype=prob.act, device=dev) if cfg.fp_proj == 2 else None
            self.y = torch.empty((M, cfg.d_inner), dtype=prob.act, device=dev)
        else:
            VW0 = cfg.d_inner + 2 * cfg.d_state + cfg.nheads
            VW = VW0 + ZG
            self.v = torch.empty((M, VW), dtype=prob.act, device=dev)
            self.xbc = torch.empty((M, Cc), dtype=prob.act, device=dev) if cfg.gated else None
            self.y = torch.empty((M, cfg.d_inner), dtype=prob.act, device=dev)
        self.bl_ws = torch.empty(prob.ws_bytes, dtype=torch.uint8, device=dev)
        L = tws.lib()

        def bl(x_ptr, k, ldx, w, s, n, y_ptr, ldy, res_ptr):
            a = tws.BitlinearArgs()
            a.x, a.x_dtype, a.act_bits, a.m, a.k, a.ldx = x_ptr, dt, cfg.act_bits, M, k, ldx
            a.norm_eps = cfg.norm_eps
            a.w_packed, a.w_scale, a.n_out, a.group_size = w.data_ptr(), s.data_ptr(), n, cfg.group_size
            a.residual, a.ld_res = res_ptr, cfg.d_model
            a.y, a.y_dtype, a.ldy = y_ptr, dt, ldy
            assert L.ssm_bitlinear_workspace_bytes(ctypes.byref(a)) <= prob.ws_bytes
            return a

        def dense(x_ptr, k, ldx, w, n, y_ptr, ldy, res_ptr):  # arguments of ssm_dense_fwd
            return (x_ptr, dt, M, k, ldx, w.data_ptr(), n, res_ptr, cfg.d_model if res_ptr else 0, y_ptr, ldy)

        def proj(name, x_ptr, k, ldx, d, n, y_ptr, ldy, res_ptr):
            """(stage name, args) of one projection, ternary or full precision."""
            if cfg.is_fp(name):
                return ("dense_" + name, dense(x_ptr, k, ldx, d["fw_" + name], n, y_ptr, ldy, res_ptr))
            return ("bitlinear_" + name, bl(x_ptr, k, ldx, d["w_" + name], d["s_" + name], n, y_ptr, ldy, res_ptr))

        def conv(x_ptr, ldx, d, out_ptr):  # arguments of ssm_conv1d_silu_fwd (stream appended at run)
            return (x_ptr, dt, cfg.batch, cfg.seqlen, Cc, ldx, d["conv_w"].data_ptr(), cfg.d_conv,
                    d["conv_b"].data_ptr(), None, None, out_ptr, Cc)

        for li, d in enumerate(prob.layers):
            src = prob.u if li == 0 else prob.bufs[(li - 1) % 2]
            dst = prob.bufs[li % 2]
            st = []
            if cfg.kind == wl.MAMBA1:
                R, N = cfg.dt_rank, cfg.d_state
                st.append(proj("in", src.data_ptr(), cfg.d_model, cfg.d_model, d, XW, self.xz.data_ptr(), XW, None))
                if cfg.gated:
                    st.append(("conv", conv(self.xz.data_ptr(), XW, d, self.x.data_ptr())))
                st.append(proj("x", self.x.data_ptr(), cfg.d_inner, cfg.d_inner, d, PW, self.p.data_ptr(), PW, None))
                if cfg.fp_proj == 2:
                    st.append(proj("dt", self.p.data_ptr(), R, PW, d, cfg.d_inner, self.dl.data_ptr(), cfg.d_inner,
                                   None))
                a = tws.ScanArgs()
                a.batch, a.seqlen, a.nheads, a.headdim, a.d_state = cfg.batch, cfg.seqlen, cfg.d_inner, 1, N
                a.a_per_state, a.act_dtype = 1, dt
                a.x, a.ld_x = self.x.data_ptr(), cfg.d_inner
                a.delta_bias, a.delta_softplus = d["dt_bias"].data_ptr(), 1
                a.A = d["A"].data_ptr()
                a.Bm, a.ld_B = self.p.data_ptr() + R * es, PW
                a.Cm, a.ld_C = self.p.data_ptr() + (R + N) * es, PW
                a.D = d["D"].data_ptr()
                a.y, a.ld_y = self.y.data_ptr(), cfg.d_inner
                if cfg.fp_proj == 2:
                    a.delta, a.ld_delta = self.dl.data_ptr(), cfg.d_inner
                else:
                    a.dt_in, a.ld_dt_in, a.dt_rank = self.p.data_ptr(), PW, R
                    a.w_dt, a.s_dt, a.dt_eps = d["w_dt"].data_ptr(), d["s_dt"].data_ptr(), cfg.norm_eps
                if cfg.gated:
                    a.gate, a.ld_gate = self.xz.data_ptr() + cfg.d_inner * es, XW
                st.append(("scan", a))
                st.append(proj("out", self.y.data_ptr(), cfg.d_inner, cfg.d_inner, d, cfg.d_model, dst.data_ptr(),
                               cfg.d_model, src.data_ptr()))
            else:
                H, P, N = cfg.nheads, cfg.headdim, cfg.d_state
                st.append(proj("in", src.data_ptr(), cfg.d_model, cfg.d_model, d, VW, self.v.data_ptr(), VW, None))
                base = self.v.data_ptr()
                xb, ldb = base, VW
                if cfg.gated:
                    st.append(("conv", conv(base, VW, d, self.xbc.data_ptr())))
                    xb, ldb = self.xbc.data_ptr(), Cc
                a = tws.ScanArgs()
                a.batch, a.seqlen, a.nheads, a.headdim, a.d_state = cfg.batch, cfg.seqlen, H, P, N
                a.a_per_state, a.act_dtype = 0, dt
                a.x, a.ld_x = xb, ldb
                a.Bm, a.ld_B = xb + cfg.d_inner * es, ldb
                a.Cm, a.ld_C = xb + (cfg.d_inner + N) * es, ldb
                a.delta, a.ld_delta = base + (cfg.d_inner + 2 * N) * es, VW
                if cfg.gated:
                    a.gate, a.ld_gate = base + VW0 * es, VW
                a.delta_bias, a.delta_softplus = d["dt_bias"].data_ptr(), 1
                a.A, a.D = d["A"].data_ptr(), d["D"].data_ptr()
                a.y, a.ld_y = self.y.data_ptr(), cfg.d_inner
                st.append(("scan", a))
                st.append(proj("out", self.y.data_ptr(), cfg.d_inner, cfg.d_inner, d, cfg.d_model, dst.data_ptr(),
                               cfg.d_model, src.data_ptr()))
            self.stages.append(st)
        self.scan_ws_bytes = max(1, L.ssm_selective_scan_workspace_bytes(ctypes.byref(self.stages[0][-2][1])))
        self.scan_ws = torch.empty(self.scan_ws_bytes, dtype=torch.uint8, device=dev)

    def run(self, stream_handle, events=None):
        """events: name -> (iterator of pre-created start events, iterator of end events)."""
        L = tws.lib()
        for st in self.stages:
            for name, a in st:
                if events is not None:
                    next(events[name][0]).record()
                if name == "scan":
                    rc = L.ssm_selective_scan_fwd(ctypes.byref(a), self.scan_ws.data_ptr(), self.scan_ws_bytes,
                                                  stream_handle)
                elif name == "conv":
                    rc = L.ssm_conv1d_silu_fwd(*a, stream_handle)
                elif name.startswith("dense"):
                    rc = L.ssm_dense_fwd(*a, stream_handle)
                else:
                    rc = L.ssm_bitlinear_fwd(ctypes.byref(a), self.bl_ws.data_ptr(), self.prob.ws_bytes,
                                             stream_handle)
                if rc != 0:
                    raise tws.SsmError(rc, L.ssm_last_error().decode())
                if events is not None:
                    next(events[name][1]).record()


# ------------------------------------------------------------------ algorithmic cost per launch

def stage_cost(cfg: wl.MixerConfig, name: str) -> dict:
    """Algorithmic HBM bytes and work of one launch of a stage over the whole batch."""
    M = cfg.tokens
    es = 2 if cfg.act_dtype == "bf16" else 4
    shapes = cfg.proj_shapes
    if name.startswith("dense"):  # full-precision projection: dense weights in the act dtype
        n, k = shapes[name.split("_")[1]]
        byts = M * (k + n) * es + n * k * es + (M * n * es if name == "dense_out" else 0)
        return {"bytes": byts, "ops": 2 * M * n * k, "ops_unit": "bf16-FLOP" if es == 2 else "fp32-FLOP"}
    if name.startswith("bitlinear"):
        n, k = shapes[name.split("_")[1]]
        wbytes = n * 4 * ((k + 15) // 16)
        byts = M * (k + n) * es + wbytes + (M * n * es if name == "bitlinear_out" else 0)
        return {"bytes": byts, "ops": 2 * M * n * k, "ops_unit": "int8-OP" if cfg.act_bits == 8 else "bf16-FLOP"}
    if name == "conv":  # read and write each convolved channel once
        return {"bytes": 2 * M * cfg.conv_channels * es, "ops": None, "ops_unit": None}
    gate = M * cfg.d_inner * es if cfg.gated else 0
    if cfg.kind == wl.MAMBA1:
        PW = cfg.dt_rank + 2 * cfg.d_state
        byts = M * (cfg.d_inner + PW + cfg.d_inner) * es + gate
        slots = M * cfg.d_inner * cfg.d_state * SCAN_M1_SLOTS_PER_STATE_STEP
        return {"bytes": byts, "ops": 2 * slots, "ops_unit": "fp32-FLOP-eq"}
    VW = cfg.d_inner + 2 * cfg.d_state + cfg.nheads
    byts = M * (VW + cfg.d_inner) * es + gate
    return {"bytes": byts, "ops": None, "ops_unit": None}


def read_traffic(kind: str, name: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None when absent or
    taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{name}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                vals[k.strip()] = v.strip()
    if vals.get("kernel_src_sha") != kernel_src_hash(kind):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ CPU baseline

def decode_bench(prob: Problem, steps: int, warmup: int, batches) -> dict:
    """Token-by-token decoding through the whole stack (ssm_mixer_step per layer, one token per
    sequence, the recurrent state of every layer carried in HBM), one token step captured as a
    HIP graph and replayed.  Algorithmic bytes per token step: the packed ternary weights and
    scales of every layer, the fp32 state read and written, and the token's input and output."""
    cfg = prob.cfg
    L = tws.lib()
    cb = ctypes.byref(prob.c)
    es = 2 if prob.act == torch.bfloat16 else 4
    wbytes = sum(t.numel() * t.element_size() for d in prob.layers for k, t in d.items())
    out = {}
    for B in batches:
        nb = tws.ssm_mixer_workspace_bytes(prob.c, B, 1)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=prob.dev)
        shape = (B, cfg.d_inner, cfg.d_state) if cfg.kind == wl.MAMBA1 else (B, cfg.nheads, cfg.headdim, cfg.d_state)
        states = [torch.zeros(shape, dtype=torch.float32, device=prob.dev) for _ in prob.mws]
        cshape = (B, cfg.d_conv - 1, cfg.conv_channels)
        cstates = [torch.zeros(cshape, dtype=torch.float32, device=prob.dev) if cfg.gated and cfg.d_conv > 1 else None
                   for _ in prob.mws]
        u = prob.u[:B, 0].contiguous()
        bufs = [torch.empty_like(u), torch.empty_like(u)]

        def token_step(sh):
            h = u
            for i, mw in enumerate(prob.mws):
                o = bufs[i % 2]
                cs = None if cstates[i] is None else cstates[i].data_ptr()
                st = L.ssm_mixer_step(cb, ctypes.byref(mw), h.data_ptr(), o.data_ptr(), B, states[i].data_ptr(), cs, 1,
                                      ws.data_ptr(), nb, sh)
                if st != 0:
                    raise tws.SsmError(st, L.ssm_last_error().decode())
                h = o

        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            token_step(s2.cuda_stream)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s2):
                token_step(s2.cuda_stream)
        torch.cuda.synchronize()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        sbytes = 2 * sum(t.numel() * 4 for t in states + [c for c in cstates if c is not None])
        byts = wbytes + sbytes + 2 * B * cfg.d_model * es
        out[f"batch_{B}"] = {"us_per_token_step": us, "tokens_per_s": B / (us * 1e-6), "layers": len(prob.mws),
                             "bytes_per_step": byts, "GBps": byts / (us * 1e-6) / 1e9,
                             "finite": bool(all(torch.isfinite(t).all() for t in states))}
        del g
    return out


def train_bench(prob: Problem, steps: int, warmup: int, parts=("projection", "scan", "mixer")) -> dict:
    """The training side of one ternary projection at the workload's shape (its out_proj: the
    largest k): straight-through-estimator backward (dx through RMSNorm, dW, the scale
    gradient) and one QAT step (SGD on latent weights and scales, re-ternarised under the
    learned scales), each timed with HIP events over `steps` calls; then the scan's backward and
    the whole mixer layer's backward (parts selects which)."""
    out = {}
    if "projection" in parts:
        out.update(_train_projection(prob, steps, warmup))
    if "scan" in parts:
        out.update(_train_scan(prob, steps, warmup))
    if "mixer" in parts:
        out.update(_train_mixer(prob, steps, warmup))
    return out


def _train_projection(prob: Problem, steps: int, warmup: int) -> dict:
    cfg = prob.cfg
    if "out" not in cfg.proj_shapes or cfg.is_fp("out") or cfg.act_bits != 8:
        return {}
    n, k = cfg.proj_shapes["out"]
    M = cfg.tokens
    g = wl.rng(7)
    dev = prob.dev
    w = torch.from_numpy(wl.normal(g, (n, k), 0.0, 0.02)).to(dev)
    packed, scale, _ = tws.ssm_ternary_quantize_weights(w, cfg.group_size)
    x = torch.from_numpy(wl.normal(g, (M, k))).to(dev).to(prob.act)
    dy = torch.from_numpy(wl.normal(g, (M, n))).to(dev)
    L = tws.lib()
    a = tws.BitlinearBwdArgs()
    dx = torch.empty((M, k), dtype=torch.float32, device=dev)
    dw = torch.empty((n, k), dtype=torch.float32, device=dev)
    ds = torch.empty(scale.numel(), dtype=torch.float32, device=dev)
    a.x, a.x_dtype, a.m, a.k, a.ldx = x.data_ptr(), tws._DTYPES[prob.act], M, k, k
    a.norm_eps = cfg.norm_eps
    a.w_packed, a.w_scale, a.n_out, a.group_size = packed.data_ptr(), scale.data_ptr(), n, cfg.group_size
    a.w_latent, a.dy, a.ld_dy, a.dx, a.ld_dx = w.data_ptr(), dy.data_ptr(), n, dx.data_ptr(), k
    a.dw, a.d_scale = dw.data_ptr(), ds.data_ptr()
    nb = L.ssm_bitlinear_bwd_workspace_bytes(ctypes.byref(a))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    sh = torch.cuda.current_stream().cuda_stream
    zc = torch.zeros(1, dtype=torch.int64, device=dev)

    def bwd():
        st = L.ssm_bitlinear_bwd(ctypes.byref(a), ws.data_ptr(), nb, sh)
        if st != 0:
            raise tws.SsmError(st, L.ssm_last_error().decode())

    def qat():
        st = L.ssm_qat_sgd_step(w.data_ptr(), scale.data_ptr(), dw.data_ptr(), ds.data_ptr(), n, k, cfg.group_size,
                                1e-6, 0.0, packed.data_ptr(), zc.data_ptr(), None, 0, sh)
        if st != 0:
            raise tws.SsmError(st, L.ssm_last_error().decode())

    out = {"projection": "out_proj", "m": M, "n": n, "k": k}
    for name, fn in (("bwd", bwd), ("qat_step", qat)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_us"] = e0.elapsed_time(e1) * 1e3 / steps
    flops = 2 * (2.0 * M * n * k)  # the two dense contractions
    out["bwd_TFLOP/s"] = flops / (out["bwd_us"] * 1e-6) / 1e12
    out["zero_ratio"] = float(zc.item()) / (n * k)
    return out


def _train_scan(prob: Problem, steps: int, warmup: int) -> dict:
    cfg, dev, out = prob.cfg, prob.dev, {}
    g = wl.rng(8)
    if cfg.kind == wl.MAMBA1:  # the scan's backward at the workload's shape
        H, N = cfg.d_inner, cfg.d_state
        p = wl.scan_problem(cfg.batch, cfg.seqlen, H, 1, N, True, seed=5)
        t = {k: torch.from_numpy(v).to(dev) for k, v in p.items()}
        for k in ("x", "delta", "Bm", "Cm"):
            t[k] = t[k].to(prob.act)
        dys = torch.from_numpy(wl.normal(g, (cfg.batch, cfg.seqlen, H))).to(dev)

        def sbwd():
            tws.ssm_selective_scan_bwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], dys, D=t["D"],
                                       delta_bias=t["dt_bias"], stream=torch.cuda.current_stream())

        for _ in range(max(1, warmup // 2)):
            sbwd()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(2, steps // 4)
        e0.record()
        for _ in range(reps):
            sbwd()
        e1.record()
        torch.cuda.synchronize()
        out["scan_bwd_us"] = e0.elapsed_time(e1) * 1e3 / reps
        # algorithmic bytes: read x, delta, B, C, dy; write dx, ddelta, dB, dC (fp32 grads)
        es = 2 if prob.act == torch.bfloat16 else 4
        Mt = cfg.tokens
        byts = Mt * (2 * H + 2 * N) * es + Mt * H * 4 + Mt * (2 * H + 2 * N) * 4
        out["scan_bwd_GBps"] = byts / (out["scan_bwd_us"] * 1e-6) / 1e9
    return out


def _train_mixer(prob: Problem, steps: int, warmup: int) -> dict:
    cfg, dev, out = prob.cfg, prob.dev, {}
    g = wl.rng(9)
    if cfg.kind == wl.MAMBA1 and not cfg.gated and cfg.fp_proj == 0 and prob.act == torch.float32:
        # the whole layer's backward (forward again, then the chain) for the stack's first layer
        lats = {"lat_" + p: torch.from_numpy(prob.lat0["W_" + p]).to(dev) for p in cfg.proj_shapes}
        dout = torch.from_numpy(wl.normal(g, (cfg.batch, cfg.seqlen, cfg.d_model))).to(dev)
        mws = torch.empty(tws.ssm_mixer_bwd_workspace_bytes(prob.c, cfg.batch, cfg.seqlen), dtype=torch.uint8,
                          device=dev)

        def mbwd():
            return tws.ssm_mixer_bwd(prob.c, prob.mws[0], prob.u, dout, latents=lats, workspace=mws,
                                     stream=torch.cuda.current_stream())

        for _ in range(max(1, warmup // 2)):
            mbwd()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(2, steps // 4)
        e0.record()
        for _ in range(reps):
            mbwd()
        e1.record()
        torch.cuda.synchronize()
        out["mixer_bwd_us"] = e0.elapsed_time(e1) * 1e3 / reps
        out["mixer_bwd_tokens_per_s"] = cfg.tokens / (out["mixer_bwd_us"] * 1e-6)
    return out


def cpu_baseline(cfg: wl.MixerConfig, seed: int, target_s: float) -> dict:
    import oracle
    from oracle import mixer_stack
    lat, u = wl.mixer_problem(cfg, seed=seed)
    if cfg.act_dtype == "bf16":
        u = torch.from_numpy(u).to(torch.bfloat16).float().numpy()
    layers = []
    for lw in lat:
        w = {k: lw[k] for k in ("A", "D", "dt_bias", "conv_w", "conv_b") if k in lw}
        for name in cfg.proj_shapes:
            if cfg.is_fp(name):
                wv = lw["W_" + name]
                w["f_" + name] = torch.from_numpy(wv).to(torch.bfloat16).float().numpy() if cfg.act_dtype == "bf16" else wv
                continue
            c, s, _ = oracle.quantize_weights(lw["W_" + name], cfg.group_size)
            w["c_" + name], w["s_" + name] = c, s
        layers.append(w)
    oc = dict(kind=cfg.kind, d_model=cfg.d_model, d_inner=cfg.d_inner, d_state=cfg.d_state, dt_rank=cfg.dt_rank,
              nheads=cfg.nheads, headdim=cfg.headdim, group_size=cfg.group_size, act_bits=cfg.act_bits,
              act_dtype=oracle.BF16 if cfg.act_dtype == "bf16" else oracle.F32, norm_eps=cfg.norm_eps,
              gated=cfg.gated, d_conv=cfg.d_conv, fp_proj=cfg.fp_proj)
    # calibrate on one sequence, then run enough whole sequences (the whole batch repeated, when
    # one pass over it is shorter than the target) to fill the target time
    t0 = time.perf_counter()
    mixer_stack(oc, layers, u[:1])
    t1 = time.perf_counter() - t0
    nseq = int(max(1, min(cfg.batch, round(target_s / max(t1, 1e-3)))))
    reps, el = 0, 0.0
    while reps < 16 and (reps == 0 or el < 0.8 * target_s):
        t0 = time.perf_counter()
        mixer_stack(oc, layers, u[:nseq])
        el += time.perf_counter() - t0
        reps += 1
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": reps * nseq * cfg.seqlen / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x {nseq} of {cfg.batch} sequences x {cfg.seqlen} tokens through all {cfg.layers} "
                      f"layers ({el:.1f} s, fp64 oracle with OpenMP)"}


# ------------------------------------------------------------------ main

def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (sequences are independent, "
              "so a data-parallel run would shard the batch with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    cfg = wl.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    prob = Problem(cfg, args.seed, dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    if args.mixer_bwd_only:
        print(json.dumps({"train": train_bench(prob, args.steps, args.warmup, parts=("mixer",))}))
        return

    if args.train_only:
        print(json.dumps({"train_bitlinear": train_bench(prob, args.steps, args.warmup)}))
        return

    if args.decode_only:
        print(json.dumps({"decode": decode_bench(prob, args.steps, args.warmup, (cfg.batch, 1))}))
        return

    result = {}
    if not args.stages_only:
        for _ in range(args.warmup):
            prob.step(sh)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record()
        for _ in range(args.steps):
            prob.step(sh)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        eager_ms = e0.elapsed_time(e1) / args.steps
        result["eager_ms_per_step"] = eager_ms
        result["eager_wall_ms_per_step"] = wall * 1e3 / args.steps
        step_ms = eager_ms
        if not args.no_graph:
            g = torch.cuda.CUDAGraph()
            s2 = torch.cuda.Stream()
            s2.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s2):
                prob.step(s2.cuda_stream)  # warm the capture stream
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=s2):
                    prob.step(s2.cuda_stream)
            torch.cuda.synchronize()
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.steps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            graph_ms = e0.elapsed_time(e1) / args.steps
            result["graph_ms_per_step"] = graph_ms
            step_ms = min(step_ms, graph_ms)
        result["ms_per_step"] = step_ms

    # per-stage durations (same kernels, issued stage by stage with events in between)
    plan = StagePlan(prob)
    for _ in range(max(1, args.warmup)):
        plan.run(sh)
    torch.cuda.synchronize()
    names = [n for n, _ in plan.stages[0]]
    nper = args.steps * len(plan.stages)
    ev = {n: ([torch.cuda.Event(enable_timing=True) for _ in range(nper)],
              [torch.cuda.Event(enable_timing=True) for _ in range(nper)]) for n in names}
    events = {n: (iter(ev[n][0]), iter(ev[n][1])) for n in names}
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)  # let the host queue the instrumented launches ahead of the GPU
    s0.record()
    for _ in range(args.steps):
        plan.run(sh, events)
    s1.record()
    torch.cuda.synchronize()
    stage_total_ms = s0.elapsed_time(s1) / args.steps
    stages = {}
    for n in names:
        durs = [a.elapsed_time(b) for a, b in zip(*ev[n])]
        cost = stage_cost(cfg, n)
        avg_s = float(np.mean(durs)) * 1e-3
        stages[n] = {"avg_us": avg_s * 1e6, "launches": len(durs), "GBps": cost["bytes"] / avg_s / 1e9,
                     "bytes": cost["bytes"]}
        if cost["ops"]:
            stages[n]["T" + cost["ops_unit"] + "/s"] = cost["ops"] / avg_s / 1e12
    dominant = max(names, key=lambda n: stages[n]["avg_us"] * stages[n]["launches"])

    # whole mixer layers (ssm_mixer_fwd, as in the headline step), bracketed per layer: for the
    # Mamba-1 kind the mixer runs in_proj, x_proj and the dt-input quantisation as one fused
    # kernel, whose time is the layer time minus the scan and out_proj stages
    L = tws.lib()
    nl = len(prob.mws)
    lev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps * nl)]
    torch.cuda._sleep(20_000_000)
    k = 0
    for _ in range(args.steps):
        h = prob.u
        for i, mw in enumerate(prob.mws):
            out = prob.bufs[i % 2]
            lev[k][0].record()
            st = L.ssm_mixer_fwd(ctypes.byref(prob.c), ctypes.byref(mw), h.data_ptr(), out.data_ptr(), cfg.batch,
                                 cfg.seqlen, 1, prob.ws.data_ptr(), prob.ws_bytes, sh)
            lev[k][1].record()
            if st != 0:
                raise tws.SsmError(st, L.ssm_last_error().decode())
            h = out
            k += 1
    torch.cuda.synchronize()
    layer_us = float(np.mean([a.elapsed_time(b) for a, b in lev])) * 1e3
    layer = {"avg_us": layer_us, "launches": len(lev)}
    if cfg.kind == wl.MAMBA1 and L.ssm_mixer_fuses_front(ctypes.byref(prob.c)):
        front_us = layer_us - stages["scan"]["avg_us"] - stages["bitlinear_out"]["avg_us"]
        byts = cfg.tokens * (cfg.d_model + cfg.d_inner + cfg.dt_rank + 2 * cfg.d_state) * (2 if cfg.act_dtype == "bf16" else 4)
        layer["front_fused_us_derived"] = front_us
        layer["front_fused_GBps_derived"] = byts / (front_us * 1e-6) / 1e9

    cost = stage_cost(cfg, dominant)
    avg_s = stages[dominant]["avg_us"] * 1e-6
    if dominant == "scan" and cfg.kind == wl.MAMBA1:
        kind = "scan_m1"
        alu_t = cost["ops"] / (FP32_VECTOR_PEAK_TFLOPS * 1e12)
        hbm_t = cost["bytes"] / (HBM_PEAK_GBPS * 1e9)
        bound = "alu" if alu_t >= hbm_t else "hbm"
    elif dominant == "scan":
        kind, bound = "ssd", "hbm"
    elif dominant == "conv":
        kind, bound = "conv", "hbm"
    elif dominant.startswith("dense"):  # full-precision projection on rocBLAS (fp32 or bf16 matrix cores)
        kind = "dense"
        pk = FP32_MATRIX_PEAK_TFLOPS if cfg.act_dtype == "f32" else BF16_MFMA_PEAK_TFLOPS
        bound = "mfma" if cost["ops"] / cost["bytes"] >= pk * 1e12 / (HBM_PEAK_GBPS * 1e9) else "hbm"
    else:
        kind = "bitlinear"
        ai = cost["ops"] / cost["bytes"]
        ridge = (INT8_MFMA_PEAK_TOPS if cfg.act_bits == 8 else BF16_MFMA_PEAK_TFLOPS) * 1e12 / (HBM_PEAK_GBPS * 1e9)
        bound = "mfma" if ai >= ridge else "hbm"
    if bound == "alu":
        roof = {"bound": "alu", "achieved": cost["ops"] / avg_s / 1e12, "peak": FP32_VECTOR_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    elif bound == "mfma":
        if kind == "dense":
            pk = FP32_MATRIX_PEAK_TFLOPS if cfg.act_dtype == "f32" else BF16_MFMA_PEAK_TFLOPS
        else:
            pk = INT8_MFMA_PEAK_TOPS if cfg.act_bits == 8 else BF16_MFMA_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": cost["ops"] / avg_s / 1e12, "peak": pk, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": cost["bytes"] / avg_s / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = read_traffic(kind, dominant, args.workload)
    roof["kernel"] = dominant
    roof["avg_launch_us"] = stages[dominant]["avg_us"]
    roof["hbm_frac"] = cost["bytes"] / avg_s / 1e9 / HBM_PEAK_GBPS

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.stages_only:
        print(json.dumps({"stages": stages, "stage_ms_per_step": stage_total_ms, "layer": layer, "roofline": roof}))
        return

    tokens = cfg.tokens
    blk = "gated block (conv + SiLU gate around the mixer)" if cfg.gated else "mixer"
    line = {
        "metric": "mixer tokens/s at TriSSM shape" if args.workload == "trissm" else f"mixer tokens/s ({cfg.name})",
        "value": tokens / (result["ms_per_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": result["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.act_dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.layers}-layer ternary selective-SSM {blk} stack" if cfg.layers > 1
                   else f"{cfg.name}: one ternary selective-SSM {blk} layer",
                   "kind": "mamba1" if cfg.kind == wl.MAMBA1 else "ssd", "layers": cfg.layers,
                   "d_model": cfg.d_model, "d_inner": cfg.d_inner, "d_state": cfg.d_state, "dt_rank": cfg.dt_rank,
                   "nheads": cfg.nheads, "headdim": cfg.headdim, "batch": cfg.batch, "seq_len": cfg.seqlen,
                   "tokens_per_step": tokens, "act_bits": cfg.act_bits, "group_size": cfg.group_size,
                   "contraction": "int8 x ternary -> int32 (MFMA)" if cfg.act_bits == 8 else
                   "bf16 x ternary -> fp32 (MFMA)", "scan_state": "fp32", "gated": cfg.gated, "d_conv": cfg.d_conv},
        "timing": {k: v for k, v in result.items() if k != "ms_per_step"},
        "weight_bytes": sum(t.numel() * t.element_size() for d in prob.layers for t in d.values()),
        "stages": stages,
        "stage_ms_per_step": stage_total_ms,
        "layer": layer,
        "roofline": roof,
    }
    if not args.no_decode:
        line["decode"] = decode_bench(prob, max(args.steps, 50), args.warmup, (cfg.batch, 1))
    if not args.no_train:
        line["train_bitlinear"] = train_bench(prob, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.seed, args.cpu_seconds)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
