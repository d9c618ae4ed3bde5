"""Seeded synthetic inputs for the ternary selective-SSM mixer (shared by tests and bench).

This module only draws random numbers and describes shapes; it holds none of
the mixer's arithmetic.  Both the HIP path and the CPU oracle receive exactly
the arrays drawn here.

The workloads follow the model shapes of the pages:
  * bitssm_tiny   one BitSSM mixer layer, fp32 (a small case the oracle finishes quickly)
  * trissm        the TriSSM stack of the TriSSM README ("selective SSM, 12 layers,
                  d=256", trained on 64 x 256-token batches), fp32 activations
  * long_scan     one layer at L = 8192, exercising the carried inter-chunk state
  * ternaryssm50m an ~50M-scale stack (the TernarySSM abstract's 50M scale), bf16
                  activations with an fp32 scan state, 8 layers
  * mamba2_ssd    a Mamba-2 1.3B-shaped W1.58A16 SSD mixer (the Ternary Mamba
                  abstract): per-group (128) ternary scales, bf16 activations
  * mamba2_a8     the same SSD mixer shape with int8 absmax activations and one scale
                  per tensor: the A8 contraction at its largest shapes, (8192, 4416, 2048)
                  and (8192, 2048, 4096), where it is bound by the int8 matrix cores
  * trissm_fp_inout, trissm_fp, mamba2_ssd_fp: full-precision projections (the TriSSM
                  model's in/out projections; all of them for the fp_ssm baseline), weights
                  ~ N(0, 1/k) for those
  * trissm_gated, mamba2_ssd_gated: the same shapes as the gated block (a short causal
                  convolution of width 4 with SiLU on the SSM input, a SiLU gate from a
                  second in_proj branch)
Distributions: activations u ~ N(0,1); latent weights ~ N(0, 0.02); A = -exp(U[ln 1,
ln 16]) per (channel, state) (per head for SSD); D ~ N(1, 0.1); dt_bias ~ N(-2, 1);
convolution weights and biases ~ U(-1/sqrt(width), 1/sqrt(width)); RMSNorm gains are ones.  No dataset is read: these stand in for the activations of
TinyStories / WikiText-103 / zero-shot-suite runs, which are not available here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

MAMBA1, SSD = 0, 1


@dataclass(frozen=True)
class MixerConfig:
    name: str
    kind: int
    d_model: int
    d_inner: int
    d_state: int
    batch: int
    seqlen: int
    layers: int = 1
    dt_rank: int = 0
    nheads: int = 0
    headdim: int = 0
    act_dtype: str = "f32"      # storage dtype of every activation tensor
    act_bits: int = 8           # 8: int8 absmax activations (A8); 16: unquantised (A16)
    group_size: int = 0         # 0: one absmean scale per tensor; >0: per (row, group)
    norm_eps: float = 1e-5
    gated: int = 0              # 1: the gated block (short causal convolution + SiLU gate)
    d_conv: int = 0             # width of that convolution
    fp_proj: int = 0            # 0 all projections ternary; 1 in/out full precision; 2 all full precision

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    @property
    def proj_shapes(self) -> dict:
        """(n_out, k) of each ternary projection."""
        zg = self.d_inner if self.gated else 0  # gate branch rows of in_proj
        if self.kind == MAMBA1:
            return {"in": (self.d_inner + zg, self.d_model),
                    "x": (self.dt_rank + 2 * self.d_state, self.d_inner),
                    "dt": (self.d_inner, self.dt_rank),
                    "out": (self.d_model, self.d_inner)}
        vw = self.nheads * self.headdim + 2 * self.d_state + self.nheads
        return {"in": (vw + zg, self.d_model), "out": (self.d_model, self.d_inner)}

    def is_fp(self, name: str) -> bool:
        """Whether projection `name` is full precision (dense weights) rather than ternary."""
        if self.fp_proj >= 2:
            return True
        return self.fp_proj == 1 and name in ("in", "out")

    @property
    def conv_channels(self) -> int:
        """Channels through the short convolution: x (Mamba-1), or x, B and C (SSD)."""
        return self.d_inner if self.kind == MAMBA1 else self.d_inner + 2 * self.d_state

    def with_(self, **kw) -> "MixerConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return MixerConfig(**d)


CONFIGS = {
    "bitssm_tiny": MixerConfig("bitssm_tiny", MAMBA1, 64, 128, 16, batch=2, seqlen=64, dt_rank=8),
    "trissm": MixerConfig("trissm", MAMBA1, 256, 512, 16, batch=64, seqlen=256, layers=12, dt_rank=16),
    "long_scan": MixerConfig("long_scan", MAMBA1, 256, 512, 16, batch=8, seqlen=8192, dt_rank=16),
    "ternaryssm50m": MixerConfig("ternaryssm50m", MAMBA1, 512, 1024, 16, batch=16, seqlen=1024, layers=8,
                                 dt_rank=32, act_dtype="bf16"),
    "mamba2_ssd": MixerConfig("mamba2_ssd", SSD, 2048, 4096, 128, batch=4, seqlen=2048, nheads=64, headdim=64,
                              act_dtype="bf16", act_bits=16, group_size=128),
    "mamba2_a8": MixerConfig("mamba2_a8", SSD, 2048, 4096, 128, batch=4, seqlen=2048, nheads=64, headdim=64,
                             act_dtype="bf16", act_bits=8, group_size=0),
}
# the gated block around the mixer (short causal convolution of width 4 with SiLU on the SSM
# input, SiLU gate from a second in_proj branch), at the TriSSM and Mamba-2 shapes
CONFIGS["trissm_gated"] = CONFIGS["trissm"].with_(name="trissm_gated", gated=1, d_conv=4)
CONFIGS["mamba2_ssd_gated"] = CONFIGS["mamba2_ssd"].with_(name="mamba2_ssd_gated", gated=1, d_conv=4)
# full-precision projections: the TriSSM model's own split (in/out full precision, Delta, B, C
# ternary) and its fp_ssm baseline (no ternary projection); the Mamba-2 layer in bf16
CONFIGS["trissm_fp_inout"] = CONFIGS["trissm"].with_(name="trissm_fp_inout", fp_proj=1)
CONFIGS["trissm_fp"] = CONFIGS["trissm"].with_(name="trissm_fp", fp_proj=2)
CONFIGS["mamba2_ssd_fp"] = CONFIGS["mamba2_ssd"].with_(name="mamba2_ssd_fp", fp_proj=2)
CONFIG_ORDER = ["bitssm_tiny", "trissm", "long_scan", "ternaryssm50m", "mamba2_ssd", "mamba2_a8", "trissm_gated",
                "mamba2_ssd_gated", "trissm_fp_inout", "trissm_fp", "mamba2_ssd_fp"]


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal(g: np.random.Generator, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    return (g.standard_normal(shape) * std + mean).astype(np.float32)


def a_log_uniform(g: np.random.Generator, shape) -> np.ndarray:
    """A = -exp(U[ln 1, ln 16])."""
    return (-np.exp(g.uniform(0.0, math.log(16.0), shape))).astype(np.float32)


def layer_latent(cfg: MixerConfig, g: np.random.Generator) -> dict:
    """Latent fp32 weights of one layer, drawn in a fixed order: projections, A, D, dt_bias."""
    out = {}
    for name, (n, k) in cfg.proj_shapes.items():
        # full-precision projections have no RMSNorm in front: unit-variance outputs (std 1/sqrt(k))
        out["W_" + name] = normal(g, (n, k), 0.0, 1.0 / math.sqrt(k) if cfg.is_fp(name) else 0.02)
    h = cfg.d_inner if cfg.kind == MAMBA1 else cfg.nheads
    out["A"] = a_log_uniform(g, (h, cfg.d_state) if cfg.kind == MAMBA1 else (h,))
    out["D"] = normal(g, (h,), 1.0, 0.1)
    out["dt_bias"] = normal(g, (h,), -2.0, 1.0)
    if cfg.gated:  # depthwise convolution, uniform on +-1/sqrt(width) (fan-in of one channel)
        bnd = 1.0 / math.sqrt(cfg.d_conv)
        out["conv_w"] = g.uniform(-bnd, bnd, (cfg.conv_channels, cfg.d_conv)).astype(np.float32)
        out["conv_b"] = g.uniform(-bnd, bnd, (cfg.conv_channels,)).astype(np.float32)
    return out


def mixer_problem(cfg: MixerConfig, seed: int = 42, layers: int | None = None, batch: int | None = None):
    """(list of latent layer weights, u [B, L, d_model] fp32)."""
    g = rng(seed)
    nl = cfg.layers if layers is None else layers
    lw = [layer_latent(cfg, g) for _ in range(nl)]
    b = cfg.batch if batch is None else batch
    u = normal(g, (b, cfg.seqlen, cfg.d_model))
    return lw, u


def scan_problem(batch: int, seqlen: int, nheads: int, headdim: int, d_state: int, a_per_state: bool,
                 seed: int = 42):
    """Scan-only inputs: x, B, C ~ N(0,1); A, D as above; the softplus argument delta + dt_bias
    ~ N(-2, 1), so that softplus(delta + bias) spans slow and fast decay: delta ~ N(0, 0.75)
    per token and dt_bias ~ N(-2, 0.25) per channel (the variances add up to 1)."""
    g = rng(seed)
    x = normal(g, (batch, seqlen, nheads * headdim))
    delta = normal(g, (batch, seqlen, nheads), 0.0, math.sqrt(0.75))
    Bm = normal(g, (batch, seqlen, d_state))
    Cm = normal(g, (batch, seqlen, d_state))
    A = a_log_uniform(g, (nheads, d_state) if a_per_state else (nheads,))
    D = normal(g, (nheads,), 1.0, 0.1)
    dt_bias = normal(g, (nheads,), -2.0, 0.5)
    return dict(x=x, delta=delta, Bm=Bm, Cm=Cm, A=A, D=D, dt_bias=dt_bias)
