"""Seeded random shapes through every GPU entry point against the oracle.

Forty configurations drawn once from a fixed seed: batch 1-3, heads 1-4,
token grids up to 64 x 64 (ragged and tiny ones included), agent grids up to
16 x 16, head dims 8-128, float32 / bfloat16 / float16, pooled or supplied
agents.  Each runs the forward (dense and [B, N, H, d] strided views), the
module forward with a random subset of its terms, the module on token
features (projections) and the backward, on the discriminating inputs, with
the parity criteria of the dedicated tests.
"""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

import oracle
import efficient_attention_vision_amd as eav
from efficient_attention_vision_amd import inputs
from tests import parity
from tests.gpu_util import f64_to_device, say, to_device, to_host_f64

pytestmark = pytest.mark.gpu

BWD_RTOL = {"f32": 1e-4, "bf16": 1e-2, "f16": 5e-3}


def _configs(n=40, seed=2024):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(n):
        h, w = (int(x) for x in rng.integers(1, 65, size=2))
        s = int(rng.integers(1, min(h, w, 16) + 1))
        d = int(rng.choice([8, 16, 24, 32, 40, 48, 64, 72, 96, 128]))
        dtype = str(rng.choice(["f32", "bf16", "f16"]))
        out.append(inputs.custom(f"rand{i}_{dtype}_{h}x{w}_s{s}_d{d}", B=int(rng.integers(1, 4)),
                                 H=int(rng.integers(1, 5)), h=h, w=w, d=d, s=s, dtype=dtype,
                                 supplied_agents=bool(rng.random() < 0.25)))
    return out


CONFIGS = _configs()


def _agents(inp):
    return None if inp.A is None else inp.A.exact


@pytest.mark.parametrize("wl", CONFIGS, ids=lambda w: w.name)
def test_random_forward(wl):
    say(f"[random fwd] {wl.name} B={wl.B} H={wl.H} supplied={wl.supplied_agents}")
    inp = inputs.make_inputs(wl, 3, "discriminating")
    q, k, v, a = (to_device(x) for x in (inp.Q, inp.K, inp.V, inp.A))
    O, _, _ = oracle.forward(inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w, wl.s, wl.scale,
                             A=_agents(inp))
    out = eav.agent_attn_forward(q, k, v, (wl.h, wl.w), wl.s, wl.scale, agents=a)
    torch.cuda.synchronize()
    parity.assert_close(to_host_f64(out), O, wl.dtype, wl.name, kind="discriminating")
    # the same values in [B, N, H, d] storage
    qs, ks, vs = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    outs = eav.agent_attn_forward(qs, ks, vs, (wl.h, wl.w), wl.s, wl.scale, agents=a)
    torch.cuda.synchronize()
    assert eav.agent_attn_read_faults() == 0
    parity.assert_close(to_host_f64(outs.contiguous()), O, wl.dtype, wl.name + " strided",
                        kind="discriminating")


@pytest.mark.parametrize("wl", CONFIGS, ids=lambda w: w.name)
def test_random_module(wl):
    rng = np.random.Generator(np.random.PCG64(zlib.crc32(wl.name.encode())))
    terms = tuple(t for t in ("bias_agg", "bias_bcast", "dwc") if rng.random() < 0.6) or ("dwc",)
    say(f"[random module] {wl.name} terms={','.join(terms)}")
    inp = inputs.make_inputs(wl, 4, "discriminating")
    mt = inputs.make_module_terms(wl, 4, terms)
    q, k, v, a = (to_device(x) for x in (inp.Q, inp.K, inp.V, inp.A))
    dev = {n: (None if x is None else f64_to_device(x)) for n, x in mt.items()}
    out = eav.agent_attn_forward_module(q, k, v, (wl.h, wl.w), wl.s, wl.scale, agents=a, **dev)
    torch.cuda.synchronize()
    assert eav.agent_attn_read_faults() == 0
    O, _, _ = oracle.forward(inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w, wl.s, wl.scale,
                             A=_agents(inp), **mt)
    parity.assert_close(to_host_f64(out), O, wl.dtype, wl.name, kind="discriminating")


@pytest.mark.parametrize("wl", CONFIGS, ids=lambda w: w.name)
def test_random_projections(wl):
    say(f"[random proj] {wl.name} C={wl.H * wl.d}")
    mi = inputs.make_module_inputs(wl, 5)
    mt = inputs.make_module_terms(wl, 5)
    agents = inputs.make_inputs(wl, 5).A if wl.supplied_agents else None
    x, wqkv, wout = (to_device(t) for t in (mi.X, mi.W_qkv, mi.W_out))
    dev = {n: f64_to_device(t) for n, t in mt.items()}
    y = eav.agent_attn_module_forward(x, wqkv, (wl.h, wl.w), wl.s, wl.H, wl.scale,
                                      b_qkv=f64_to_device(mi.b_qkv), w_out=wout,
                                      b_out=f64_to_device(mi.b_out),
                                      agents=None if agents is None else to_device(agents),
                                      **dev)
    torch.cuda.synchronize()
    assert eav.agent_attn_read_faults() == 0
    ref = oracle.module_forward(mi.X.exact, mi.W_qkv.exact, mi.b_qkv, mi.W_out.exact, mi.b_out,
                                wl.H, wl.h, wl.w, wl.s, wl.scale, wl.dtype,
                                A=None if agents is None else agents.exact, **mt)
    parity.assert_close(to_host_f64(y), ref, wl.dtype, wl.name, kind="discriminating")


@pytest.mark.parametrize("wl", CONFIGS, ids=lambda w: w.name)
def test_random_backward(wl):
    say(f"[random bwd] {wl.name}")
    inp = inputs.make_inputs(wl, 6, "discriminating")
    g = inputs.make_inputs(dataclasses.replace(wl, supplied_agents=False), 1006, "iid").Q
    q, k, v, a, dout = (to_device(x) for x in (inp.Q, inp.K, inp.V, inp.A, g))
    got = eav.agent_attn_backward(q, k, v, dout, (wl.h, wl.w), wl.s, wl.scale, agents=a)
    torch.cuda.synchronize()
    ref = oracle.backward(inp.Q.exact, inp.K.exact, inp.V.exact, g.exact, wl.h, wl.w, wl.s,
                          wl.scale, A=_agents(inp))
    for name, t, r in zip(("dq", "dk", "dv", "dagents"), got, ref):
        if r is None:
            assert t is None
            continue
        _, r_err = parity.errors(to_host_f64(t), r)
        assert r_err <= BWD_RTOL[wl.dtype], (wl.name, name, r_err)
