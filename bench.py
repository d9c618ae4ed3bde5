#!/usr/bin/env python3
"""Throughput of the ternary selective-SSM mixer forward on one MI355X.

A step is one forward pass of the whole hot path over one batch: for the default
workload, the TriSSM-shaped stack of 12 BitSSM mixer layers (d_model 256, d_inner 512,
d_state 16, dt_rank 16, batch 64 x L 256, fp32 activations, int8 activations into the
ternary projections), out = u + mixer(u) per layer.  Inputs are seeded synthetic data,
resident in HBM before the timed region.  Prints one JSON line.

Also measured (each with HIP events on the stream the kernels run on):
  * every stage of the same layers issued through the stage entry points (in_proj, x_proj,
    the dt input's codes, the scan kernel alone, out_proj): average, median, p10 and p90 per
    launch, back to back (warm: each stage reads what the previous one just wrote) and with a
    512 MB write between launches (cold: inputs from HBM);
  * the roofline of the scan: the method's bytes per token (x, Delta, B, C read, y written)
    over the scan kernel's launch time, against the 8 TB/s HBM peak;
  * the int8 matrix-core contraction at the Mamba-2 1.3B shapes (8192 x 4416 x 2048 and
    8192 x 2048 x 4096) against the 5.0 POP/s int8 peak, and the chunked SSD scan at that shape;
  * the TriSSM model's own precision split (in/out projections full precision, Delta, B, C
    ternary) on the same stack;
  * token-by-token decoding; the training side of one projection, the scan and the layer;
  * the CPU oracle on a bounded sample on the host cores, single-threaded and on every core.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import ternary_weight_selective_amd as tws  # noqa: E402
import workloads as wl  # noqa: E402

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, packed (FMA = 2 FLOP per lane, two lanes per slot)
FP32_VECTOR_NONPACKED_TFLOPS = 78.6  # the same without packed fp32 instructions (not used by these kernels)
INT8_MFMA_PEAK_TOPS = 5000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_MATRIX_PEAK_TFLOPS = 157.3  # MI355X fp32 on the matrix cores (the full-precision baselines)
# Issue-slot model of the Mamba-1 recurrence (a secondary figure): per (token, channel, state)
# dt*A, exp2, (dt*x)*B, fma for h, fma for y = 4 slots + 4 slots for the quarter-rate exp2; a
# slot counts as 2 FLOP-equivalents.
SCAN_M1_SLOTS_PER_STATE_STEP = 8
FLUSH_BYTES = 512 << 20          # written between launches for the cold figures (> 256 MB MALL)

KERNEL_SOURCES = {  # source files whose text defines each timed kernel (for stale-counter checks)
    "scan_m1": ["scan.hip", "common.hpp", "launch.hpp"],
    "ssd": ["ssd.hip", "common.hpp", "launch.hpp"],
    "bitlinear": ["norm.hip", "bitlinear.hip", "common.hpp", "launch.hpp"],
    "conv": ["conv.hip", "common.hpp", "launch.hpp"],
    "dense": ["dense.hip", "launch.hpp"],
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
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU work of each oracle sample")
    ap.add_argument("--stages-only", action="store_true", help="skip the headline loop (profiling runs)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the Mamba-2-shape contraction / SSD scan and the full-precision split")
    ap.add_argument("--extra-only", action="store_true", help="only the Mamba-2-shape contraction and SSD scan")
    ap.add_argument("--no-decode", action="store_true", help="skip the token-by-token decode measurement")
    ap.add_argument("--decode-only", action="store_true", help="only the decode measurement (profiling runs)")
    ap.add_argument("--no-train", action="store_true", help="skip the BitLinear backward / QAT step measurement")
    ap.add_argument("--train-only", action="store_true", help="only the BitLinear backward / QAT step (profiling runs)")
    ap.add_argument("--mixer-bwd-only", action="store_true", help="only the mixer layer backward (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run 3 plain device copies of 1 GiB (reference for HBM byte counters)")
    return ap.parse_args()


def dist(us) -> dict:
    a = np.asarray(us, dtype=np.float64)
    return {"avg_us": float(a.mean()), "median_us": float(np.median(a)), "p10_us": float(np.percentile(a, 10)),
            "p90_us": float(np.percentile(a, 90)), "launches": int(a.size)}


def timed(fn, n: int, stream_handle, flush: torch.Tensor | None = None) -> list:
    """Per-call durations (us) of fn() with HIP events on the current stream; with `flush`, a
    512 MB write runs before every call, outside the events."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in evs:
        if flush is not None:
            flush.zero_()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def status(rc: int):
    if rc != 0:
        L = tws.lib()
        raise tws.SsmError(rc, L.ssm_last_error().decode())


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

    def weight_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for d in self.layers for t in d.values())

    def step(self, stream_handle):
        """One pass of the stack: out = u + mixer_l(u) layer after layer (ping-pong buffers)."""
        L = tws.lib()
        h = self.u
        cb = ctypes.byref(self.c)
        for i, mw in enumerate(self.mws):
            out = self.bufs[i % 2]
            status(L.ssm_mixer_fwd(cb, ctypes.byref(mw), h.data_ptr(), out.data_ptr(), self.cfg.batch,
                                   self.cfg.seqlen, 1, self.ws.data_ptr(), self.ws_bytes, stream_handle))
            h = out
        return h


def headline(prob: Problem, args, sh, flush) -> dict:
    """The timed stack: W untimed warm-up steps, then exactly K steps back to back between two
    synchronisations (eager launches; then the same step replayed as a captured graph).  Also
    the per-step distribution of the graph replay, back to back and with a 512 MB write before
    every step (cold)."""
    out = {}
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
    out["eager_wall_ms_per_step"] = (time.perf_counter() - w0) * 1e3 / args.steps
    out["eager_ms_per_step"] = e0.elapsed_time(e1) / args.steps
    out["ms_per_step"] = out["eager_ms_per_step"]
    if args.no_graph:
        return out
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
    out["graph_ms_per_step"] = e0.elapsed_time(e1) / args.steps
    out["ms_per_step"] = min(out["ms_per_step"], out["graph_ms_per_step"])
    warm = timed(g.replay, args.steps, sh)
    cold = timed(g.replay, args.steps, sh, flush)
    for key, us in (("graph_step_warm", warm), ("graph_step_cold", cold)):
        d = dist(us)
        out[key] = {"median_ms": d["median_us"] / 1e3, "p10_ms": d["p10_us"] / 1e3, "p90_ms": d["p90_us"] / 1e3}
    del g
    return out


class StagePlan:
    """The same layers as ssm_mixer_fwd, issued stage by stage through the public entry points
    (identical kernels and arguments), so that HIP events can bracket each stage.  For the
    Mamba-1 kind the dt input's codes are their own stage (ssm_dt_input_quantize), so that the
    scan stage is the scan kernel alone."""

    def __init__(self, prob: Problem):
        cfg = prob.cfg
        dev = prob.dev
        M = cfg.tokens
        es = 2 if prob.act == torch.bfloat16 else 4
        dt = tws._DTYPES[prob.act]
        self.prob = prob
        self.stages = []  # per layer: list of (name, callable)
        ZG = cfg.d_inner if cfg.gated else 0  # gate branch columns of the in_proj output
        Cc = cfg.conv_channels
        L = tws.lib()
        self.keep = []
        if cfg.kind == wl.MAMBA1:
            PW = cfg.dt_rank + 2 * cfg.d_state
            XW = cfg.d_inner + ZG
            self.xz = torch.empty((M, XW), dtype=prob.act, device=dev)
            self.x = torch.empty((M, cfg.d_inner), dtype=prob.act, device=dev) if cfg.gated else self.xz
            self.p = torch.empty((M, PW), dtype=prob.act, device=dev)
            self.dl = torch.empty((M, cfg.d_inner), dtype=prob.act, device=dev) if cfg.fp_proj == 2 else None
            self.y = torch.empty((M, cfg.d_inner), dtype=prob.act, device=dev)
            cw = 16 * ((cfg.dt_rank + 15) // 16)
            self.codes = torch.empty((M, cw), dtype=torch.int8, device=dev)
            self.deq = torch.empty(M, dtype=torch.float64, device=dev)
        else:
            VW0 = cfg.d_inner + 2 * cfg.d_state + cfg.nheads
            VW = VW0 + ZG
            self.v = torch.empty((M, VW), dtype=prob.act, device=dev)
            self.xbc = torch.empty((M, Cc), dtype=prob.act, device=dev) if cfg.gated else None
            self.y = torch.empty((M, cfg.d_inner), dtype=prob.act, device=dev)
        self.bl_ws = torch.empty(prob.ws_bytes, dtype=torch.uint8, device=dev)
        self.scan_ws = None

        def bl(x_ptr, k, ldx, w, s, n, y_ptr, ldy, res_ptr):
            a = tws.BitlinearArgs()
            a.x, a.x_dtype, a.act_bits, a.m, a.k, a.ldx = x_ptr, dt, cfg.act_bits, M, k, ldx
            a.norm_eps = cfg.norm_eps
            a.w_packed, a.w_scale, a.n_out, a.group_size = w.data_ptr(), s.data_ptr(), n, cfg.group_size
            a.residual, a.ld_res = res_ptr, cfg.d_model
            a.y, a.y_dtype, a.ldy = y_ptr, dt, ldy
            assert L.ssm_bitlinear_workspace_bytes(ctypes.byref(a)) <= prob.ws_bytes
            self.keep.append(a)
            return lambda sh: status(L.ssm_bitlinear_fwd(ctypes.byref(a), self.bl_ws.data_ptr(), prob.ws_bytes, sh))

        def dense(x_ptr, k, ldx, w, n, y_ptr, ldy, res_ptr):
            return lambda sh: status(L.ssm_dense_fwd(x_ptr, dt, M, k, ldx, w.data_ptr(), n, res_ptr,
                                                     cfg.d_model if res_ptr else 0, y_ptr, ldy, sh))

        def proj(name, x_ptr, k, ldx, d, n, y_ptr, ldy, res_ptr):
            if cfg.is_fp(name):
                return ("dense_" + name, dense(x_ptr, k, ldx, d["fw_" + name], n, y_ptr, ldy, res_ptr))
            return ("bitlinear_" + name, bl(x_ptr, k, ldx, d["w_" + name], d["s_" + name], n, y_ptr, ldy, res_ptr))

        def conv(x_ptr, ldx, d, out_ptr):
            return ("conv", lambda sh: status(L.ssm_conv1d_silu_fwd(
                x_ptr, dt, cfg.batch, cfg.seqlen, Cc, ldx, d["conv_w"].data_ptr(), cfg.d_conv,
                d["conv_b"].data_ptr(), None, None, out_ptr, Cc, sh)))

        def scan(a):
            self.keep.append(a)
            nb = max(1, L.ssm_selective_scan_workspace_bytes(ctypes.byref(a)))
            if self.scan_ws is None or self.scan_ws.numel() < nb:
                self.scan_ws = torch.empty(nb, dtype=torch.uint8, device=dev)
            return ("scan", lambda sh: status(L.ssm_selective_scan_fwd(ctypes.byref(a), self.scan_ws.data_ptr(),
                                                                       self.scan_ws.numel(), sh)))

        for li, d in enumerate(prob.layers):
            src = prob.u if li == 0 else prob.bufs[(li - 1) % 2]
            dst = prob.bufs[li % 2]
            st = []
            if cfg.kind == wl.MAMBA1:
                R, N = cfg.dt_rank, cfg.d_state
                st.append(proj("in", src.data_ptr(), cfg.d_model, cfg.d_model, d, XW, self.xz.data_ptr(), XW, None))
                if cfg.gated:
                    st.append(conv(self.xz.data_ptr(), XW, d, self.x.data_ptr()))
                st.append(proj("x", self.x.data_ptr(), cfg.d_inner, cfg.d_inner, d, PW, self.p.data_ptr(), PW, None))
                if cfg.fp_proj == 2:
                    st.append(proj("dt", self.p.data_ptr(), R, PW, d, cfg.d_inner, self.dl.data_ptr(), cfg.d_inner,
                                   None))
                else:
                    p_ptr, c_ptr, q_ptr = self.p.data_ptr(), self.codes.data_ptr(), self.deq.data_ptr()
                    st.append(("dt_codes", lambda sh, p_ptr=p_ptr, c_ptr=c_ptr, q_ptr=q_ptr: status(
                        L.ssm_dt_input_quantize(p_ptr, dt, M, R, PW, None, cfg.norm_eps, c_ptr, q_ptr, sh))))
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
                    a.dt_codes, a.dt_deq = self.codes.data_ptr(), self.deq.data_ptr()
                if cfg.gated:
                    a.gate, a.ld_gate = self.xz.data_ptr() + cfg.d_inner * es, XW
                st.append(scan(a))
                st.append(proj("out", self.y.data_ptr(), cfg.d_inner, cfg.d_inner, d, cfg.d_model, dst.data_ptr(),
                               cfg.d_model, src.data_ptr()))
            else:
                H, P, N = cfg.nheads, cfg.headdim, cfg.d_state
                st.append(proj("in", src.data_ptr(), cfg.d_model, cfg.d_model, d, VW, self.v.data_ptr(), VW, None))
                base = self.v.data_ptr()
                xb, ldb = base, VW
                if cfg.gated:
                    st.append(conv(base, VW, d, self.xbc.data_ptr()))
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
                st.append(scan(a))
                st.append(proj("out", self.y.data_ptr(), cfg.d_inner, cfg.d_inner, d, cfg.d_model, dst.data_ptr(),
                               cfg.d_model, src.data_ptr()))
            self.stages.append(st)
        self.names = [n for n, _ in self.stages[0]]

    def run(self, sh, events=None):
        """events: name -> (iterator of start events, iterator of end events) or None."""
        for st in self.stages:
            for name, fn in st:
                if events is not None:
                    next(events[name][0]).record()
                fn(sh)
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
    if name == "dt_codes":  # dt input rows read, codes and factors written
        return {"bytes": M * (cfg.dt_rank * es + 16 * ((cfg.dt_rank + 15) // 16) + 8), "ops": None, "ops_unit": None}
    gate = M * cfg.d_inner * es if cfg.gated else 0
    if cfg.kind == wl.MAMBA1:
        # the method's bytes: x, Delta (pre-activation, d_inner per token), B, C read; y written
        byts = M * (3 * cfg.d_inner + 2 * cfg.d_state) * es + gate
        slots = M * cfg.d_inner * cfg.d_state * SCAN_M1_SLOTS_PER_STATE_STEP
        return {"bytes": byts, "ops": 2 * slots, "ops_unit": "fp32-FLOP-eq"}
    # SSD: x, B, C, dt read; y written
    byts = M * (2 * cfg.d_inner + 2 * cfg.d_state + cfg.nheads) * es + gate
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


def stage_bench(prob: Problem, args, sh, flush) -> tuple[dict, dict]:
    """Per-stage durations: the stage loop K times back to back (warm), then every stage of
    the first layer K times with a 512 MB write before each launch (cold)."""
    cfg = prob.cfg
    plan = StagePlan(prob)
    for _ in range(max(1, args.warmup)):
        plan.run(sh)
    torch.cuda.synchronize()
    names = plan.names
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
    stages = {}
    for n in names:
        durs = [a.elapsed_time(b) * 1e3 for a, b in zip(*ev[n])]
        cost = stage_cost(cfg, n)
        d = dist(durs)
        d["bytes"] = cost["bytes"]
        d["GBps"] = cost["bytes"] / (d["avg_us"] * 1e-6) / 1e9
        if cost["ops"]:
            d["T" + cost["ops_unit"] + "/s"] = cost["ops"] / (d["avg_us"] * 1e-6) / 1e12
        fn = dict(plan.stages[0])[n]
        cold = dist(timed(lambda: fn(sh), max(5, args.steps), sh, flush))
        d["cold_median_us"] = cold["median_us"]
        d["cold_GBps"] = cost["bytes"] / (cold["median_us"] * 1e-6) / 1e9
        stages[n] = d
    return stages, {"stage_ms_per_step": s0.elapsed_time(s1) / args.steps}


def layer_bench(prob: Problem, args, sh, stages: dict) -> dict:
    """Whole mixer layers (ssm_mixer_fwd, as in the headline step), bracketed per layer.  The
    Mamba-1 kind mixer runs in_proj, x_proj and the dt input's codes as one fused kernel at the
    shapes it supports: its time is the layer time minus the scan kernel and out_proj stages."""
    cfg = prob.cfg
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
            status(L.ssm_mixer_fwd(ctypes.byref(prob.c), ctypes.byref(mw), h.data_ptr(), out.data_ptr(), cfg.batch,
                                   cfg.seqlen, 1, prob.ws.data_ptr(), prob.ws_bytes, sh))
            lev[k][1].record()
            h = out
            k += 1
    torch.cuda.synchronize()
    layer = dist([a.elapsed_time(b) * 1e3 for a, b in lev])
    if cfg.kind == wl.MAMBA1 and L.ssm_mixer_fuses_front(ctypes.byref(prob.c)):
        front_us = layer["avg_us"] - stages["scan"]["avg_us"] - stages["bitlinear_out"]["avg_us"]
        byts = cfg.tokens * ((cfg.d_model + cfg.d_inner + cfg.dt_rank + 2 * cfg.d_state) *
                             (2 if cfg.act_dtype == "bf16" else 4) + 16 * ((cfg.dt_rank + 15) // 16) + 8)
        layer["front_fused_us_derived"] = front_us
        layer["front_fused_GBps_derived"] = byts / (front_us * 1e-6) / 1e9
    return layer


def scan_roofline(cfg: wl.MixerConfig, stages: dict, workload: str) -> dict:
    """%-of-HBM-peak of the scan kernel on the method's bytes (x, Delta, B, C read, y written),
    over its average launch duration in the stage loop (HIP events); the issue-slot model of the
    recurrence as a secondary figure."""
    st = stages["scan"]
    cost = stage_cost(cfg, "scan")
    avg_s = st["avg_us"] * 1e-6
    kind = "scan_m1" if cfg.kind == wl.MAMBA1 else "ssd"
    roof = {"bound": "hbm", "achieved": cost["bytes"] / avg_s / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = read_traffic(kind, "scan", workload)
    roof["kernel"] = (("k_scan_m1_g8" if cfg.d_state == 16 else "k_scan_m1") if cfg.kind == wl.MAMBA1
                      else "k_ssd_seg (+ k_ssd_combine)")
    roof["bytes_per_launch"] = cost["bytes"]
    roof["bytes_per_token"] = cost["bytes"] / cfg.tokens
    roof["avg_launch_us"] = st["avg_us"]
    roof["median_launch_us"] = st["median_us"]
    roof["p10_launch_us"], roof["p90_launch_us"] = st["p10_us"], st["p90_us"]
    roof["cold_median_launch_us"] = st["cold_median_us"]
    roof["cold_frac"] = cost["bytes"] / (st["cold_median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS
    if cost["ops"]:
        alu = cost["ops"] / avg_s / 1e12
        roof["alu_model"] = {"achieved_TFLOPeq_per_s": alu, "frac_of_157.3": alu / FP32_VECTOR_PEAK_TFLOPS,
                             "frac_of_78.6_nonpacked": alu / FP32_VECTOR_NONPACKED_TFLOPS,
                             "slots_per_state_step": SCAN_M1_SLOTS_PER_STATE_STEP}
    return roof


# ------------------------------------------------------------------ Mamba-2-shape contractions and SSD scan

def mamba2_extra(args, sh, flush, dev) -> dict:
    """The int8 x ternary contraction at the Mamba-2 1.3B layer's shapes (in_proj 8192 x 4416 x
    2048, out_proj 8192 x 2048 x 4096; int8 codes given, so only the matrix-core kernel runs),
    against the 5.0 POP/s int8 peak; and the chunked SSD scan of that layer (bf16, 64 heads x
    64, d_state 128) against the HBM peak."""
    cfg = wl.CONFIGS["mamba2_a8"]
    M = cfg.tokens
    g = wl.rng(11)
    out = {}
    for name in ("in", "out"):
        n, k = cfg.proj_shapes[name]
        w = torch.from_numpy(wl.normal(g, (n, k), 0.0, 0.02)).to(dev)
        packed, scale, _ = tws.ssm_ternary_quantize_weights(w)
        xq = torch.randint(-127, 128, (M, k), dtype=torch.int8, device=dev, generator=torch.Generator(dev).manual_seed(3))
        am = torch.full((M,), 3.0, dtype=torch.float32, device=dev)
        y = torch.empty((M, n), dtype=torch.bfloat16, device=dev)

        def call():
            tws.ssm_bitlinear_fwd(xq, packed, scale, n, x_absmax=am, y_dtype=torch.bfloat16, out=y)

        for _ in range(3):
            call()
        d = dist(timed(call, max(10, args.steps), sh))
        cold = dist(timed(call, max(5, args.steps // 2), sh, flush))
        ops = 2.0 * M * n * k
        d.update({"m": M, "n": n, "k": k, "kernel": "k_gemm_i8_big", "ops": ops,
                  "TOPS": ops / (d["avg_us"] * 1e-6) / 1e12, "cold_median_us": cold["median_us"]})
        d["frac"] = d["TOPS"] / INT8_MFMA_PEAK_TOPS
        out[name + "_proj"] = d
    # the SSD scan of the Mamba-2 layer (bf16 activations, fp32 state)
    sc = wl.CONFIGS["mamba2_ssd"]
    H, P, N = sc.nheads, sc.headdim, sc.d_state
    VW = sc.d_inner + 2 * N + H
    v = torch.randn((M, VW), dtype=torch.float32, device=dev, generator=torch.Generator(dev).manual_seed(4))
    v[:, sc.d_inner + 2 * N:] -= 2.0  # dt pre-activations ~ N(-2, 1)
    v = v.to(torch.bfloat16)
    A = torch.from_numpy(wl.a_log_uniform(g, (H,))).to(dev)
    D = torch.ones(H, device=dev)
    bias = torch.zeros(H, device=dev)
    yv = torch.empty((M, sc.d_inner), dtype=torch.bfloat16, device=dev)
    vv = v.view(sc.batch, sc.seqlen, VW)
    x_, B_, C_, dt_ = (vv[..., :sc.d_inner], vv[..., sc.d_inner:sc.d_inner + N],
                       vv[..., sc.d_inner + N:sc.d_inner + 2 * N], vv[..., sc.d_inner + 2 * N:])
    def ssd():
        tws.ssm_selective_scan_fwd(x_, dt_, A, B_, C_, D, bias, True, out=yv.view(sc.batch, sc.seqlen, -1))

    for _ in range(3):
        ssd()
    d = dist(timed(ssd, max(10, args.steps), sh))
    cold = dist(timed(ssd, max(5, args.steps // 2), sh, flush))
    byts = stage_cost(sc, "scan")["bytes"]
    d.update({"bytes": byts, "GBps": byts / (d["avg_us"] * 1e-6) / 1e9, "frac": byts / (d["avg_us"] * 1e-6) / 1e9 /
              HBM_PEAK_GBPS, "cold_median_us": cold["median_us"],
              "kernels": "k_ssd_seg state pass, k_ssd_combine, k_ssd_seg output pass"})
    out["ssd_scan"] = d
    return out


def fp_inout_bench(args, sh, dev) -> dict:
    """The TriSSM model's own precision split on the same stack: in/out projections full
    precision, Delta, B, C ternary (trissm_fp_inout), timed like the headline."""
    cfg = wl.CONFIGS["trissm_fp_inout"]
    prob = Problem(cfg, args.seed, dev)
    for _ in range(max(2, args.warmup)):
        prob.step(sh)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        prob.step(sh)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    res = {"workload": cfg.name, "ms_per_step": ms, "tokens_per_s": cfg.tokens / (ms * 1e-3),
           "weight_bytes": prob.weight_bytes()}
    del prob
    return res


# ------------------------------------------------------------------ decode and training side

def decode_bench(prob: Problem, steps: int, warmup: int, batches) -> dict:
    """Token-by-token decoding through the whole stack (ssm_mixer_stack_step: one token per
    sequence through every layer, the recurrent state of every layer carried in HBM; beside it
    the same step as ssm_mixer_step per layer), one token step captured as a HIP graph and
    replayed.  Algorithmic bytes per token step: the packed ternary weights and scales of every
    layer, the fp32 state read and written, and the token's input and output."""
    cfg = prob.cfg
    L = tws.lib()
    cb = ctypes.byref(prob.c)
    es = 2 if prob.act == torch.bfloat16 else 4
    wbytes = prob.weight_bytes()
    out = {}
    for B in batches:
        nb = tws.ssm_mixer_workspace_bytes(prob.c, B, 1)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=prob.dev)
        nbs = tws.ssm_mixer_stack_workspace_bytes(prob.c, B)
        wss = torch.empty(max(nbs, 256), dtype=torch.uint8, device=prob.dev)
        nl = len(prob.mws)
        wp = (ctypes.POINTER(tws.MixerWeights) * nl)(*[ctypes.pointer(m) for m in prob.mws])
        shape = (B, cfg.d_inner, cfg.d_state) if cfg.kind == wl.MAMBA1 else (B, cfg.nheads, cfg.headdim, cfg.d_state)
        states = [torch.zeros(shape, dtype=torch.float32, device=prob.dev) for _ in prob.mws]
        cshape = (B, cfg.d_conv - 1, cfg.conv_channels)
        cstates = [torch.zeros(cshape, dtype=torch.float32, device=prob.dev) if cfg.gated and cfg.d_conv > 1 else None
                   for _ in prob.mws]
        u = prob.u[:B, 0].contiguous()
        bufs = [torch.empty_like(u), torch.empty_like(u)]

        sp = (ctypes.c_void_p * nl)(*[t.data_ptr() for t in states])
        cp = None if cstates[0] is None else (ctypes.c_void_p * nl)(*[t.data_ptr() for t in cstates])

        def layer_steps(sh):
            h = u
            for i, mw in enumerate(prob.mws):
                o = bufs[i % 2]
                cs = None if cstates[i] is None else cstates[i].data_ptr()
                status(L.ssm_mixer_step(cb, ctypes.byref(mw), h.data_ptr(), o.data_ptr(), B, states[i].data_ptr(), cs,
                                        1, ws.data_ptr(), nb, sh))
                h = o

        def stack_step(sh):
            status(L.ssm_mixer_stack_step(cb, wp, nl, u.data_ptr(), bufs[0].data_ptr(), B, sp, cp, 1, wss.data_ptr(),
                                          nbs, sh))

        def timed(token_step):
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
            del g
            return e0.elapsed_time(e1) * 1e3 / steps

        us = timed(stack_step)
        us_layers = timed(layer_steps)
        sbytes = 2 * sum(t.numel() * 4 for t in states + [c for c in cstates if c is not None])
        byts = wbytes + sbytes + 2 * B * cfg.d_model * es
        out[f"batch_{B}"] = {"us_per_token_step": us, "tokens_per_s": B / (us * 1e-6), "layers": nl,
                             "bytes_per_step": byts, "GBps": byts / (us * 1e-6) / 1e9,
                             "us_per_token_step_layer_by_layer": us_layers,
                             "finite": bool(all(torch.isfinite(t).all() for t in states))}
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


def _avg_us(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


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
    out = {"projection": "out_proj", "m": M, "n": n, "k": k}
    out["bwd_us"] = _avg_us(lambda: status(L.ssm_bitlinear_bwd(ctypes.byref(a), ws.data_ptr(), nb, sh)), steps, warmup)
    out["qat_step_us"] = _avg_us(lambda: status(L.ssm_qat_sgd_step(
        w.data_ptr(), scale.data_ptr(), dw.data_ptr(), ds.data_ptr(), n, k, cfg.group_size, 1e-6, 0.0,
        packed.data_ptr(), zc.data_ptr(), None, 0, sh)), steps, warmup)
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

        out["scan_bwd_us"] = _avg_us(sbwd, max(2, steps // 4), max(1, warmup // 2))
        es = 2 if prob.act == torch.bfloat16 else 4
        Mt = cfg.tokens
        byts = Mt * (2 * H + 2 * N) * es + Mt * H * 4 + Mt * (2 * H + 2 * N) * 4
        out["scan_bwd_GBps"] = byts / (out["scan_bwd_us"] * 1e-6) / 1e9
    return out


def _train_mixer(prob: Problem, steps: int, warmup: int) -> dict:
    cfg, dev, out = prob.cfg, prob.dev, {}
    g = wl.rng(9)
    if cfg.kind == wl.MAMBA1 and not cfg.gated and cfg.fp_proj == 0 and prob.act == torch.float32:
        lats = {"lat_" + p: torch.from_numpy(prob.lat0["W_" + p]).to(dev) for p in cfg.proj_shapes}
        dout = torch.from_numpy(wl.normal(g, (cfg.batch, cfg.seqlen, cfg.d_model))).to(dev)
        mws = torch.empty(tws.ssm_mixer_bwd_workspace_bytes(prob.c, cfg.batch, cfg.seqlen), dtype=torch.uint8,
                          device=dev)

        def mbwd():
            return tws.ssm_mixer_bwd(prob.c, prob.mws[0], prob.u, dout, latents=lats, workspace=mws,
                                     stream=torch.cuda.current_stream())

        out["mixer_bwd_us"] = _avg_us(mbwd, max(2, steps // 4), max(1, warmup // 2))
        out["mixer_bwd_tokens_per_s"] = cfg.tokens / (out["mixer_bwd_us"] * 1e-6)
    return out


# ------------------------------------------------------------------ CPU baseline

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(cfg: wl.MixerConfig, seed: int, target_s: float) -> dict:
    """The oracle (plain C, fp64 scan, int64 contraction) on whole sequences of the same
    workload: on every host core (OpenMP over independent rows and channels) and on one thread,
    each on a sample sized to about target_s seconds."""
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

    def run(threads: int) -> tuple[float, str]:
        oracle.set_threads(threads)
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
        return reps * nseq * cfg.seqlen / el, (f"{reps} x {nseq} of {cfg.batch} sequences x {cfg.seqlen} tokens "
                                               f"through all {cfg.layers} layers ({el:.1f} s)")

    env = os.environ.get("OMP_NUM_THREADS")
    threads = int(env) if env and env.isdigit() else (os.cpu_count() or 1)
    multi, smp = run(threads)
    single, smp1 = run(1)
    oracle.set_threads(threads)
    return {"value": multi, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{smp}, fp64 oracle with OpenMP on {threads} threads",
            "single_thread_value": single, "single_thread_sample": smp1, "cpu_model": cpu_model(),
            "nproc": os.cpu_count()}


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
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    if args.extra_only:
        print(json.dumps({"mamba2_extra": mamba2_extra(args, sh, flush, dev)}))
        return

    prob = Problem(cfg, args.seed, dev)

    if args.mixer_bwd_only:
        print(json.dumps({"train": train_bench(prob, args.steps, args.warmup, parts=("mixer",))}))
        return
    if args.train_only:
        print(json.dumps({"train_bitlinear": train_bench(prob, args.steps, args.warmup)}))
        return
    if args.decode_only:
        print(json.dumps({"decode": decode_bench(prob, args.steps, args.warmup, (cfg.batch, 1))}))
        return

    timing = {} if args.stages_only else headline(prob, args, sh, flush)
    stages, st_total = stage_bench(prob, args, sh, flush)
    layer = layer_bench(prob, args, sh, stages)
    roof = scan_roofline(cfg, stages, args.workload)

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.stages_only:
        print(json.dumps({"stages": stages, **st_total, "layer": layer, "roofline": roof}))
        return

    tokens = cfg.tokens
    blk = "gated block (conv + SiLU gate around the mixer)" if cfg.gated else "mixer"
    line = {
        "metric": "mixer tokens/s at TriSSM shape" if args.workload == "trissm" else f"mixer tokens/s ({cfg.name})",
        "value": tokens / (timing["ms_per_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": timing["ms_per_step"],
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
                   "bf16 x ternary -> fp32 (MFMA)", "scan_state": "fp32", "gated": cfg.gated, "d_conv": cfg.d_conv,
                   "timed_region": "K steps back to back; every buffer reused across steps (warm); "
                                   "graph_step_cold in timing: a 512 MB write before each step"},
        "timing": {k: v for k, v in timing.items() if k != "ms_per_step"},
        "weight_bytes": prob.weight_bytes(),
        "stages": stages,
        **st_total,
        "layer": layer,
        "roofline": roof,
    }
    if not args.no_extra:
        line["mamba2_extra"] = mamba2_extra(args, sh, flush, dev)
        if cfg.name == "trissm":
            fp = fp_inout_bench(args, sh, dev)
            fp["ternary_speedup"] = line["value"] / fp["tokens_per_s"]
            fp["ternary_weight_ratio"] = fp["weight_bytes"] / line["weight_bytes"]
            line["fp_inout"] = fp
    if not args.no_decode:
        line["decode"] = decode_bench(prob, max(args.steps, 50), args.warmup, (cfg.batch, 1))
    if not args.no_train:
        line["train_bitlinear"] = train_bench(prob, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.seed, args.cpu_seconds)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
