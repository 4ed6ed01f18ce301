"""Backward pass on the GPU against the float64 oracle's gradients.

Gradients are compared by max |error| / max |reference| over each tensor
(dq, dk, dv and, for supplied agents, dagents): 1e-4 for float32 tensors
(float32 arithmetic throughout), 1e-2 for bfloat16 and 5e-3 for float16
tensors (inputs exact in their format, float32 arithmetic, gradients
rounded to the format once).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import efficient_attention_vision_amd as eav
from efficient_attention_vision_amd import inputs
from tests import parity
from tests.gpu_util import say, to_device, to_host_f64

pytestmark = pytest.mark.gpu

RTOL = {"f32": 1e-4, "bf16": 1e-2, "f16": 5e-3}


def run_backward(wl, seed, kind="discriminating"):
    say(f"[backward] {wl.name} B={wl.B} H={wl.H} grid={wl.h}x{wl.w} d={wl.d} s={wl.s} "
        f"{wl.dtype} seed={seed} {kind} supplied={wl.supplied_agents}")
    inp = inputs.make_inputs(wl, seed, kind)
    # the output gradient: same recipe and format as the inputs
    g = inputs.make_inputs(dataclasses.replace(wl, supplied_agents=False), seed + 1000, "iid").Q
    q, k, v, a, dout = (to_device(x) for x in (inp.Q, inp.K, inp.V, inp.A, g))
    dq, dk, dv, da = eav.agent_attn_backward(q, k, v, dout, (wl.h, wl.w), wl.s, wl.scale, agents=a)
    torch.cuda.synchronize()
    ref = oracle.backward(inp.Q.exact, inp.K.exact, inp.V.exact, g.exact, wl.h, wl.w, wl.s,
                          wl.scale, A=None if inp.A is None else inp.A.exact)
    got = (dq, dk, dv, da)
    for name, t, r in zip(("dq", "dk", "dv", "dagents"), got, ref):
        if r is None:
            assert t is None
            continue
        a_err, r_err = parity.errors(to_host_f64(t), r)
        say(f"       {name}: max-abs {a_err:.3e}  relative {r_err:.3e}  max|ref| "
            f"{np.abs(r).max():.3e}")
        assert r_err <= RTOL[wl.dtype], (wl.name, name, r_err)


def _as(wl, dtype, name=None):
    return dataclasses.replace(wl, dtype=dtype, name=name or f"{wl.name}_{dtype}")


CASES = [
    inputs.WORKLOADS["tiny_fp32"],
    inputs.WORKLOADS["pvt_stage1"],
    inputs.WORKLOADS["sd_unet"],
    inputs.WORKLOADS["sd_unet_agents"],
    _as(inputs.WORKLOADS["deit_s"], "f16"),
    inputs.custom("bwd_ragged_13x11_s3", B=2, H=3, h=13, w=11, d=64, s=3),
    inputs.custom("bwd_ragged_f32", B=1, H=2, h=9, w=7, d=40, s=3, dtype="f32"),
    inputs.custom("bwd_d128_f32", B=1, H=2, h=12, w=16, d=128, s=4, dtype="f32"),
    inputs.custom("bwd_d128", B=1, H=2, h=24, w=24, d=128, s=8),
    inputs.custom("bwd_d32_256", B=1, H=2, h=32, w=32, d=32, s=16),
    inputs.custom("bwd_supplied_f32", B=2, H=2, h=10, w=10, d=64, s=3, dtype="f32",
                  supplied_agents=True),
    inputs.custom("bwd_supplied_f16", B=1, H=3, h=12, w=12, d=64, s=4, dtype="f16",
                  supplied_agents=True),
    inputs.custom("bwd_one_agent", B=2, H=1, h=6, w=5, d=64, s=1),
    # matrix-core path: head dims below one 32-channel slab and between slabs,
    # many token workgroups per head (two batches of partials per wave in the
    # reductions), supplied bf16 agents at 64 agents
    inputs.custom("bwd_d32_k49", B=2, H=2, h=14, w=14, d=32, s=7),
    inputs.custom("bwd_d24_f16", B=1, H=2, h=12, w=10, d=24, s=3, dtype="f16"),
    inputs.custom("bwd_d96_k36", B=1, H=2, h=16, w=16, d=96, s=6),
    inputs.custom("bwd_one_head_4096", B=1, H=1, h=64, w=64, d=64, s=8),
    inputs.custom("bwd_supplied_k64", B=2, H=2, h=16, w=16, d=64, s=8, supplied_agents=True),
    # more than 64 agents: chunks of 64 with a ragged last chunk (81 = 64 + 17,
    # 144 = 2 x 64 + 16), supplied agents over 196 = 3 x 64 + 4, and 512 heads
    # of 81 tokens, where each pass holds a whole head in one workgroup
    inputs.custom("bwd_chunk_k81", B=2, H=2, h=27, w=27, d=64, s=9),
    inputs.custom("bwd_chunk_k144_d128_f16", B=1, H=2, h=48, w=40, d=128, s=12, dtype="f16"),
    inputs.custom("bwd_chunk_supplied_k196", B=1, H=2, h=28, w=28, d=48, s=14,
                  supplied_agents=True),
    inputs.custom("bwd_chunk_512_heads", B=64, H=8, h=9, w=9, d=16, s=9),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_backward(wl):
    run_backward(wl, 50)


def test_backward_iid_latent_sample():
    """The latent workload's shape (16384 tokens, 256 agents) on one head."""
    wl = dataclasses.replace(inputs.WORKLOADS["latent_hr"], H=1, name="latent_1head")
    run_backward(wl, 51, "iid")
