"""The full module's forward (agent biases in both attentions, depth-wise
3 x 3 convolution of V) on the GPU against the float64 oracle.

Cases span the kernel paths: groups of workgroups per head with up to 64
agents (early broadcast probabilities) and with 256 agents, one workgroup
per head, every head-dim class, ragged grids (convolution borders), each
term alone, float32 / bfloat16 / float16 tensors.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import efficient_attention_vision_amd as eav
from efficient_attention_vision_amd import inputs
from tests import parity
from tests.gpu_util import f64_to_device, say, to_device, to_host_f64

pytestmark = pytest.mark.gpu


def run_module(wl, seed, terms=("bias_agg", "bias_bcast", "dwc"), kind="discriminating"):
    say(f"[module] {wl.name} B={wl.B} H={wl.H} grid={wl.h}x{wl.w} d={wl.d} s={wl.s} "
        f"{wl.dtype} seed={seed} {kind} terms={','.join(terms)}")
    inp = inputs.make_inputs(wl, seed, kind)
    mt = inputs.make_module_terms(wl, seed, terms)
    q, k, v, a = (to_device(x) for x in (inp.Q, inp.K, inp.V, inp.A))
    dev = {n: (None if x is None else f64_to_device(x)) for n, x in mt.items()}
    out = eav.agent_attn_forward_module(q, k, v, (wl.h, wl.w), wl.s, wl.scale, agents=a, **dev)
    torch.cuda.synchronize()
    assert eav.agent_attn_read_faults() == 0
    O, _, _ = oracle.forward(inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w, wl.s, wl.scale,
                             A=None if inp.A is None else inp.A.exact,
                             bias_agg=mt["bias_agg"], bias_bcast=mt["bias_bcast"],
                             dwc_weight=mt["dwc_weight"], dwc_bias=mt["dwc_bias"])
    got = to_host_f64(out)
    a_err, r_err = parity.errors(got, O)
    say(f"       max-abs {a_err:.3e}  relative {r_err:.3e}  max|O| {np.abs(O).max():.2f}")
    parity.assert_close(got, O, wl.dtype, wl.name, kind="discriminating")


def _f16(wl):
    return dataclasses.replace(wl, name=wl.name + "_f16", dtype="f16")


CASES = [
    inputs.WORKLOADS["pvt_stage1"],
    inputs.WORKLOADS["sd_unet"],
    inputs.WORKLOADS["deit_s"],
    inputs.WORKLOADS["latent_hr"],
    inputs.WORKLOADS["sd_unet_agents"],
    _f16(inputs.WORKLOADS["pvt_stage1"]),
    inputs.custom("mod_ragged_13x11_s3", B=2, H=3, h=13, w=11, d=64, s=3),
    inputs.custom("mod_d128_s8", B=1, H=2, h=24, w=24, d=128, s=8),
    inputs.custom("mod_d32_s10_p1", B=33, H=8, h=20, w=20, d=32, s=10),
    inputs.custom("mod_d96_s10_f16", B=1, H=2, h=40, w=30, d=96, s=10, dtype="f16"),
    inputs.custom("mod_f32_ragged", B=2, H=2, h=9, w=7, d=40, s=3, dtype="f32"),
    inputs.custom("mod_f32_d128", B=1, H=2, h=16, w=12, d=128, s=4, dtype="f32"),
    inputs.custom("mod_thin_2x300", B=1, H=2, h=2, w=300, d=64, s=2),
    # more heads than CUs, up to 64 agents: four-wave workgroups, two per CU,
    # the convolution's V rows staged in the plan's free LDS
    inputs.custom("mod_w4_d32", B=40, H=8, h=12, w=12, d=32, s=4),
    inputs.custom("mod_w4_f16_ragged", B=70, H=4, h=15, w=13, d=64, s=7, dtype="f16"),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_module_forward(wl):
    run_module(wl, 40)


@pytest.mark.parametrize("terms", [("bias_agg",), ("bias_bcast",), ("dwc",)],
                         ids=lambda t: t[0])
@pytest.mark.parametrize("wl", [inputs.WORKLOADS["pvt_stage1"],
                                inputs.custom("mod_small_f32", B=1, H=2, h=10, w=10, d=64, s=5,
                                              dtype="f32"),
                                inputs.custom("mod_256", B=1, H=2, h=64, w=48, d=64, s=16)],
                         ids=lambda w: w.name)
def test_module_terms_alone(wl, terms):
    run_module(wl, 41, terms)


def test_module_without_terms_is_the_plain_forward():
    """With every term absent the module entry point gives the plain
    forward's output, bit for bit (same kernels)."""
    wl = inputs.WORKLOADS["pvt_stage1"]
    inp = inputs.make_inputs(wl, 42, "discriminating")
    q, k, v = (to_device(x) for x in (inp.Q, inp.K, inp.V))
    a = eav.agent_attn_forward(q, k, v, (wl.h, wl.w), wl.s, wl.scale)
    b = eav.agent_attn_forward_module(q, k, v, (wl.h, wl.w), wl.s, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
