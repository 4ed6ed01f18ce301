"""Seeded synthetic inputs for the Agent Attention forward.

This module only draws random numbers and converts number formats.  It holds
none of the attention arithmetic, so the CPU oracle and the GPU path can both
consume exactly the same operands without sharing any method code.

Workloads (shapes named after the models the Agent Attention pages evaluate:
DeiT-S at 224^2, PVT stage 1, the Stable-Diffusion v1.5 UNet latent, and a
high-resolution latent; see "Agent Attention: On the Integration of Softmax and
Linear Attention", §4 Agent Transformer and §5 Experiments).  Trained weights
and datasets are not used: Q, K, V (and caller-supplied agents) are i.i.d.
normal draws of the stated standard deviation, generated in float32 with
numpy's PCG64 in the order Q, K, V, A and then rounded to bfloat16 with
round-to-nearest-even for the bf16 workloads.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    h: int          # token-grid rows
    w: int          # token-grid columns
    d: int          # head dimension
    s: int          # agent grid side: k = s*s agents
    dtype: str      # "f32", "bf16" or "f16"
    sigma: float    # std of the i.i.d. normal Q, K, V draws
    supplied_agents: bool = False   # caller passes A instead of pooling Q
    agent_sigma: float = 1.0

    @property
    def N(self) -> int:
        return self.h * self.w

    @property
    def k(self) -> int:
        return self.s * self.s

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def es(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 1, 1, 14, 14, 64, 7, "f32", 1.0),
        Workload("deit_s", 64, 6, 14, 14, 64, 7, "bf16", 1.0),
        Workload("pvt_stage1", 16, 1, 56, 56, 64, 7, "bf16", 0.5),
        Workload("sd_unet", 2, 8, 64, 64, 40, 8, "bf16", 1.0),
        Workload("sd_unet_agents", 2, 8, 64, 64, 40, 8, "bf16", 1.0,
                 supplied_agents=True, agent_sigma=1.0),
        Workload("latent_hr", 1, 8, 128, 128, 64, 16, "bf16", 1.0),
    ]
}


def custom(name="custom", *, B, H, h, w, d, s, dtype="bf16", sigma=1.0,
           supplied_agents=False, agent_sigma=1.0) -> Workload:
    return Workload(name, B, H, h, w, d, s, dtype, sigma, supplied_agents,
                    agent_sigma)


# ---------------------------------------------------------------------------
# number formats

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Finite inputs only (the generators never produce inf/nan)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def f16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns (uint16), round to nearest even
    (numpy's float16 conversion)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_from_f16_bits(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


@dataclasses.dataclass
class Operand:
    """One tensor in its storage format plus its exact value in float64."""
    storage: np.ndarray   # float32 array, or uint16 bfloat16 / float16 bit patterns
    exact: np.ndarray     # the same values, widened exactly to float64
    dtype: str


def _pack(x32: np.ndarray, dtype: str) -> Operand:
    if dtype == "f32":
        x32 = np.ascontiguousarray(x32, dtype=np.float32)
        return Operand(x32, x32.astype(np.float64), dtype)
    if dtype == "f16":
        bits = f16_bits_from_f32(x32)
        return Operand(bits, f32_from_f16_bits(bits).astype(np.float64), dtype)
    bits = bf16_bits_from_f32(x32)
    return Operand(bits, f32_from_bf16_bits(bits).astype(np.float64), dtype)


@dataclasses.dataclass
class Inputs:
    wl: Workload
    Q: Operand
    K: Operand
    V: Operand
    A: Operand | None     # caller-supplied agents, or None (pool Q)


def make_inputs(wl: Workload, seed: int, kind: str = "iid") -> Inputs:
    """Draw Q, K, V (and A when the workload supplies agents).

    kind="iid":  i.i.d. N(0, sigma^2) as the workload states.
    kind="discriminating":  inputs for which |O| is of order one and both
    softmaxes are far from uniform, so that a wrong output cannot hide inside
    the absolute tolerance:
      * Q is a smooth random field over the h x w grid (three low-frequency
        cosines per channel plus a little noise), so that window means of Q
        stay far from zero;
      * K ~ N(0, 1.8^2);
      * V has per-channel means spread over [-2, 2] plus N(0, 1) noise;
      * supplied agents ~ N(0, 1).
    Amplitudes are chosen so that the logits of both softmaxes have a
    standard deviation of roughly 1.5-2.5.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shp = (wl.B, wl.H, wl.N, wl.d)
    ashp = (wl.B, wl.H, wl.k, wl.d)
    if kind == "iid":
        q = rng.standard_normal(shp, dtype=np.float32) * np.float32(wl.sigma)
        k = rng.standard_normal(shp, dtype=np.float32) * np.float32(wl.sigma)
        v = rng.standard_normal(shp, dtype=np.float32) * np.float32(wl.sigma)
        a = (rng.standard_normal(ashp, dtype=np.float32)
             * np.float32(wl.agent_sigma)) if wl.supplied_agents else None
    elif kind == "discriminating":
        rr = np.arange(wl.h, dtype=np.float64)[:, None] / wl.h
        cc = np.arange(wl.w, dtype=np.float64)[None, :] / wl.w
        field = np.zeros((wl.B, wl.H, wl.h, wl.w, wl.d))
        for _ in range(3):
            fr = rng.uniform(0.0, 2.0, size=(wl.B, wl.H, 1, 1, wl.d))
            fc = rng.uniform(0.0, 2.0, size=(wl.B, wl.H, 1, 1, wl.d))
            ph = rng.uniform(0.0, 2 * np.pi, size=(wl.B, wl.H, 1, 1, wl.d))
            field += np.cos(2 * np.pi * (fr * rr[..., None] + fc * cc[..., None]) + ph)
        q = (0.7 * field.reshape(shp)
             + 0.3 * rng.standard_normal(shp)).astype(np.float32)
        k = (1.8 * rng.standard_normal(shp)).astype(np.float32)
        mu = np.linspace(-2.0, 2.0, wl.d)
        v = (mu + rng.standard_normal(shp)).astype(np.float32)
        a = rng.standard_normal(ashp).astype(np.float32) if wl.supplied_agents else None
    else:
        raise ValueError(f"unknown input kind {kind!r}")
    return Inputs(wl, _pack(q, wl.dtype), _pack(k, wl.dtype), _pack(v, wl.dtype),
                  _pack(a, wl.dtype) if a is not None else None)


def make_module_terms(wl: Workload, seed: int, terms=("bias_agg", "bias_bcast", "dwc")) -> dict:
    """Seeded float32 parameters of the module terms for workload `wl`:
    agent biases B1 [H, k, N] and B2 [H, N, k] ~ N(0, 1) (the size of the
    logits they are added to), depth-wise convolution weights [H*d, 3, 3] ~
    N(0, 1/9) (so that the term is about as large as V) and its bias [H*d] ~
    N(0, 0.25).  Keys: bias_agg, bias_bcast, dwc_weight, dwc_bias (None for
    terms not asked for).  Drawn in that order from PCG64(seed + 7919)."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    H, k, N, d = wl.H, wl.k, wl.N, wl.d
    b1 = rng.standard_normal((H, k, N)).astype(np.float32)
    b2 = rng.standard_normal((H, N, k)).astype(np.float32)
    w = (rng.standard_normal((H * d, 3, 3)) / 3.0).astype(np.float32)
    b = (0.5 * rng.standard_normal(H * d)).astype(np.float32)
    return {"bias_agg": b1 if "bias_agg" in terms else None,
            "bias_bcast": b2 if "bias_bcast" in terms else None,
            "dwc_weight": w if "dwc" in terms else None,
            "dwc_bias": b if "dwc" in terms else None}


@dataclasses.dataclass
class ModuleInputs:
    """Token features and projection parameters of the attention module."""
    X: Operand            # [B, N, C], C = H d
    W_qkv: Operand        # [3C, C] (Linear layout [out, in])
    b_qkv: np.ndarray     # float32 [3C]
    W_out: Operand        # [C, C]
    b_out: np.ndarray     # float32 [C]


def make_module_inputs(wl: Workload, seed: int) -> ModuleInputs:
    """X ~ N(0, 1); weights ~ N(0, 1/C) (so that q, k, v and y are of order
    one); biases ~ N(0, 0.1^2).  Drawn in the order X, W_qkv, b_qkv, W_out,
    b_out from PCG64(seed + 104729), in float32, then rounded to the
    workload's format (biases stay float32)."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    C = wl.H * wl.d
    x = rng.standard_normal((wl.B, wl.N, C), dtype=np.float32)
    sd = np.float32(1.0 / math.sqrt(C))
    wqkv = rng.standard_normal((3 * C, C), dtype=np.float32) * sd
    bqkv = rng.standard_normal(3 * C, dtype=np.float32) * np.float32(0.1)
    wout = rng.standard_normal((C, C), dtype=np.float32) * sd
    bout = rng.standard_normal(C, dtype=np.float32) * np.float32(0.1)
    return ModuleInputs(_pack(x, wl.dtype), _pack(wqkv, wl.dtype), bqkv, _pack(wout, wl.dtype),
                        bout)
