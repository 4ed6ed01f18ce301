"""GPU path vs the float64 CPU oracle, element by element, on seeded inputs.

Every workload runs at its full size (the oracle finishes each in seconds),
on the i.i.d. inputs of its definition and on the discriminating inputs,
through the same C ABI entry point and launch configuration that the
benchmark times.  Edge cases cover ragged grids (windows that overlap by one
row or column), head dims 8..128, 1..256 agents, a single token, empty
batches and caller-supplied agents.
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


def run_case(wl, seed, kind, cached=False):
    say(f"[case] {wl.name} B={wl.B} H={wl.H} grid={wl.h}x{wl.w} d={wl.d} s={wl.s} "
        f"{wl.dtype} seed={seed} {kind} supplied={wl.supplied_agents} cached={cached}")
    inp = inputs.make_inputs(wl, seed, kind)
    q, k, v, a = (to_device(x) for x in (inp.Q, inp.K, inp.V, inp.A))
    fwd = eav.agent_attn_forward_cached if cached else eav.agent_attn_forward
    out = fwd(q, k, v, (wl.h, wl.w), wl.s, wl.scale, agents=a)
    torch.cuda.synchronize()
    O, _, _ = oracle.forward(inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w, wl.s, wl.scale,
                             A=None if inp.A is None else inp.A.exact)
    got = to_host_f64(out)
    assert eav.agent_attn_read_faults() == 0
    a_err, r_err = parity.errors(got, O)
    say(f"       max-abs {a_err:.3e}  relative {r_err:.3e}")
    parity.assert_close(got, O, wl.dtype, wl.name, kind=kind)
    return got, O


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_workload_iid(name, seed):
    run_case(inputs.WORKLOADS[name], seed, "iid")


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_discriminating(name):
    run_case(inputs.WORKLOADS[name], 0, "discriminating")


EDGE = [
    # ragged grids: h, w not multiples of s (windows share a row/column)
    inputs.custom("ragged_13x11_s3", B=2, H=3, h=13, w=11, d=64, s=3),
    inputs.custom("ragged_30x17_s5_f32", B=1, H=2, h=30, w=17, d=32, s=5, dtype="f32"),
    inputs.custom("ragged_57x55_s7", B=1, H=2, h=57, w=55, d=64, s=7),
    # head dims
    inputs.custom("d8", B=2, H=2, h=16, w=16, d=8, s=4),
    inputs.custom("d40_f32", B=1, H=3, h=12, w=12, d=40, s=4, dtype="f32"),
    inputs.custom("d128", B=1, H=2, h=24, w=24, d=128, s=8),
    inputs.custom("d128_f32", B=1, H=1, h=16, w=16, d=128, s=4, dtype="f32"),
    inputs.custom("d96", B=1, H=2, h=20, w=20, d=96, s=5),
    # agent counts: one agent, one agent per token, the maximum
    inputs.custom("one_agent", B=2, H=2, h=9, w=7, d=64, s=1),
    inputs.custom("agent_per_token", B=1, H=2, h=6, w=6, d=64, s=6),
    inputs.custom("max_agents_d128", B=1, H=2, h=64, w=48, d=128, s=16),
    inputs.custom("max_agents_f32", B=1, H=1, h=32, w=32, d=64, s=16, dtype="f32"),
    # a single token
    inputs.custom("single_token", B=3, H=1, h=1, w=1, d=64, s=1),
    # long thin grid and a long sequence
    inputs.custom("thin_2x300", B=1, H=2, h=2, w=300, d=64, s=2),
    inputs.custom("long_96x96", B=1, H=2, h=96, w=96, d=64, s=12),
    # grouping regimes: two workgroups per head on one XCD (B*H = 128), two
    # per head across XCDs (B*H = 100), one per head just above the CU count
    inputs.custom("bh128_p2", B=16, H=8, h=24, w=24, d=64, s=6),
    inputs.custom("bh100_p2", B=25, H=4, h=20, w=20, d=32, s=5),
    inputs.custom("bh260_p1", B=26, H=10, h=8, w=8, d=64, s=4),
    # more heads than CUs with up to 64 agents: one head per four-wave
    # workgroup, two per CU (head dims 32, 48, 64; several key/value rounds
    # of 256 tokens; ragged windows in fp16; supplied agents), and d = 128,
    # whose LDS keeps one eight-wave workgroup per CU
    inputs.custom("bh320_w4_d32", B=40, H=8, h=12, w=12, d=32, s=4),
    inputs.custom("bh300_w4_n576", B=300, H=1, h=24, w=24, d=64, s=6),
    inputs.custom("bh280_w4_f16_ragged", B=70, H=4, h=15, w=13, d=64, s=7, dtype="f16"),
    inputs.custom("bh264_w4_supplied", B=33, H=8, h=10, w=10, d=48, s=3, supplied_agents=True),
    inputs.custom("bh300_d128_p1", B=100, H=3, h=8, w=8, d=128, s=4),
    # a long sequence: 256 x 256 grid, 256 agents
    inputs.custom("long_256x256", B=1, H=2, h=256, w=256, d=64, s=16),
    # one workgroup per head with 100 agents (grouped broadcast, partial
    # groups of query tiles, padding agents in the last chunk)
    inputs.custom("p1_100_agents", B=40, H=8, h=20, w=20, d=64, s=10),
    inputs.custom("p1_100_agents_d32", B=33, H=8, h=20, w=20, d=32, s=10),
    # caller-supplied agents with ragged counts
    inputs.custom("supplied_s3", B=2, H=2, h=10, w=10, d=64, s=3, supplied_agents=True),
    inputs.custom("supplied_f32", B=1, H=2, h=10, w=12, d=48, s=2, dtype="f32",
                  supplied_agents=True),
]


@pytest.mark.parametrize("wl", EDGE, ids=lambda w: w.name)
def test_edge_cases(wl):
    run_case(wl, 5, "iid")
    run_case(wl, 6, "discriminating")


def test_cached_workspace_path():
    run_case(inputs.WORKLOADS["pvt_stage1"], 0, "iid", cached=True)
    run_case(inputs.custom("cached_small", B=1, H=1, h=8, w=8, d=64, s=2), 1, "iid", cached=True)
    eav.agent_attn_release()
    run_case(inputs.WORKLOADS["sd_unet"], 0, "iid", cached=True)


def test_empty_batch():
    q = torch.empty((0, 4, 64, 64), dtype=torch.bfloat16, device="cuda")
    out = eav.agent_attn_forward(q, q.clone(), q.clone(), (8, 8), 4)
    assert out.shape == q.shape


def test_repeated_calls_are_deterministic():
    wl = inputs.WORKLOADS["latent_hr"]
    inp = inputs.make_inputs(wl, 0, "iid")
    q, k, v = (to_device(x) for x in (inp.Q, inp.K, inp.V))
    o1 = eav.agent_attn_forward(q, k, v, (wl.h, wl.w), wl.s, wl.scale)
    o2 = eav.agent_attn_forward(q, k, v, (wl.h, wl.w), wl.s, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_validation_errors_raise_on_gpu():
    q = torch.zeros((1, 1, 64, 12), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        eav.agent_attn_forward(q, q.clone(), q.clone(), (8, 8), 2)
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        eav.agent_attn_forward(q, q.clone(), q.clone(), (8, 8), 9)


# ------------------------------------------------------------ single steps

STEP_CASES = [
    inputs.WORKLOADS["tiny_fp32"], inputs.WORKLOADS["pvt_stage1"], inputs.WORKLOADS["sd_unet"],
    inputs.WORKLOADS["latent_hr"], EDGE[0], EDGE[1], EDGE[5],
]


@pytest.mark.parametrize("wl", STEP_CASES, ids=lambda w: w.name)
def test_pool_step(wl):
    say(f"[pool] {wl.name}")
    inp = inputs.make_inputs(wl, 3, "discriminating")
    A = eav.agent_attn_pool(to_device(inp.Q), (wl.h, wl.w), wl.s)
    ref = oracle.pool_agents(inp.Q.exact, wl.h, wl.w, wl.s)
    err = np.abs(to_host_f64(A) - ref).max()
    assert err <= 1e-5 * max(1.0, np.abs(ref).max()), err


@pytest.mark.parametrize("wl", STEP_CASES, ids=lambda w: w.name)
def test_aggregate_step(wl):
    say(f"[aggregate] {wl.name}")
    inp = inputs.make_inputs(wl, 4, "discriminating")
    A32 = oracle.pool_agents(inp.Q.exact, wl.h, wl.w, wl.s).astype(np.float32)
    VA = eav.agent_attn_aggregate(f64_to_device(A32), to_device(inp.K), to_device(inp.V),
                                  wl.scale)
    ref = oracle.aggregate(A32.astype(np.float64), inp.K.exact, inp.V.exact, wl.scale)
    parity.assert_close(to_host_f64(VA), ref, wl.dtype, "aggregate " + wl.name,
                        kind="discriminating")


@pytest.mark.parametrize("wl", STEP_CASES, ids=lambda w: w.name)
def test_broadcast_step(wl):
    say(f"[broadcast] {wl.name}")
    inp = inputs.make_inputs(wl, 5, "discriminating")
    A32 = oracle.pool_agents(inp.Q.exact, wl.h, wl.w, wl.s).astype(np.float32)
    VA32 = oracle.aggregate(A32.astype(np.float64), inp.K.exact, inp.V.exact,
                            wl.scale).astype(np.float32)
    out = eav.agent_attn_broadcast(to_device(inp.Q), f64_to_device(A32), f64_to_device(VA32),
                                   wl.scale)
    ref = oracle.broadcast(inp.Q.exact, A32.astype(np.float64), VA32.astype(np.float64),
                           wl.scale)
    parity.assert_close(to_host_f64(out), ref, wl.dtype, "broadcast " + wl.name,
                        kind="discriminating")


def test_fused_counters_return_to_zero():
    """Many fused launches on one caller workspace, alternating shapes: every
    result matches the oracle and the group counters end at zero."""
    from efficient_attention_vision_amd import _binding
    wls = [inputs.WORKLOADS["pvt_stage1"], inputs.WORKLOADS["sd_unet"],
           inputs.custom("p3", B=3, H=5, h=20, w=18, d=64, s=4)]
    need = max(_binding.agent_attn_workspace_bytes(w.B, w.H, w.h, w.w, w.d, w.s, 1)
               for w in wls)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    cases = []
    for i, wl in enumerate(wls):
        inp = inputs.make_inputs(wl, 10 + i, "discriminating")
        O, _, _ = oracle.forward(inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w, wl.s,
                                 wl.scale)
        cases.append((wl, [to_device(x) for x in (inp.Q, inp.K, inp.V)], O))
    for rep in range(12):
        wl, (q, k, v), O = cases[rep % len(cases)]
        say(f"[fused repeat] {rep} {wl.name}")
        out = eav.agent_attn_forward(q, k, v, (wl.h, wl.w), wl.s, wl.scale, workspace=ws)
        torch.cuda.synchronize()
        parity.assert_close(to_host_f64(out), O, "bf16", wl.name, kind="discriminating")
    torch.cuda.synchronize()
    assert int(ws[: 512 * 512].count_nonzero()) == 0     # counters
    assert eav.agent_attn_read_faults(ws) == 0


def test_shared_workspace_across_shapes():
    """A small-B*H call between two large ones on the binding's cached
    workspace must not disturb the large calls' barrier counters."""
    seq = [inputs.WORKLOADS["deit_s"], inputs.custom("one_head", B=1, H=1, h=16, w=16, d=64, s=4),
           inputs.WORKLOADS["pvt_stage1"], inputs.custom("bh2", B=2, H=1, h=30, w=30, d=64, s=5),
           inputs.WORKLOADS["sd_unet"], inputs.WORKLOADS["pvt_stage1"]]
    for i, wl in enumerate(seq):
        run_case(wl, 20 + i, "discriminating")


def test_barrier_timeout_is_reported_and_recovers():
    """With the barrier wait limit forced to zero from the host, a grouped
    forward gives up at a barrier, ends normally and reports
    AGENT_ATTN_FAULT_BARRIER; the next forward with the default limit is
    correct again (the group state was cleared)."""
    from efficient_attention_vision_amd import _binding
    wl = inputs.WORKLOADS["pvt_stage1"]
    inp = inputs.make_inputs(wl, 7, "discriminating")
    q, k, v = (to_device(x) for x in (inp.Q, inp.K, inp.V))
    assert eav.agent_attn_read_faults() == 0
    prev = eav.agent_attn_set_wait_limit(0)
    try:
        say("[timeout] forward with a zero wait limit")
        eav.agent_attn_forward(q, k, v, (wl.h, wl.w), wl.s, wl.scale)
        faults = eav.agent_attn_read_faults()
    finally:
        eav.agent_attn_set_wait_limit(prev)
    assert faults & _binding.FAULT_BARRIER, faults
    assert eav.agent_attn_set_wait_limit(-1) == prev
    say("[timeout] forward with the default limit")
    out = eav.agent_attn_forward(q, k, v, (wl.h, wl.w), wl.s, wl.scale)
    assert eav.agent_attn_read_faults() == 0
    O, _, _ = oracle.forward(inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w, wl.s, wl.scale)
    parity.assert_close(to_host_f64(out), O, wl.dtype, "after timeout", kind="discriminating")


# ------------------------------------------------------ strided layouts

def _bnhd(t):
    """The same [B, H, N, d] values stored as [B, N, H, d] (a head-split
    projection output), returned as the [B, H, N, d] view of that storage."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def _packed_qkv(q, k, v):
    """q, k, v stored interleaved in one [B, N, 3, H, d] tensor."""
    x = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous()
    return tuple(x[:, :, i].transpose(1, 2) for i in range(3))


STRIDED = [
    (inputs.WORKLOADS["sd_unet"], "bnhd"),
    (inputs.WORKLOADS["deit_s"], "bnhd"),
    (inputs.custom("packed_d64", B=2, H=4, h=20, w=20, d=64, s=5), "packed"),
    (inputs.custom("bnhd_f32", B=2, H=3, h=12, w=12, d=32, s=4, dtype="f32"), "bnhd"),
    (inputs.custom("packed_f32", B=1, H=2, h=10, w=10, d=64, s=2, dtype="f32"), "packed"),
    (inputs.custom("bnhd_ragged", B=2, H=3, h=13, w=11, d=48, s=3), "bnhd"),
]


@pytest.mark.parametrize("wl,layout", STRIDED, ids=lambda x: x if isinstance(x, str) else x.name)
def test_strided_layouts(wl, layout):
    """q, k, v (and out) as strided views: head-split [B, N, H, d] storage and
    a packed [B, N, 3, H, d] projection output.  The strided entry point must
    give the oracle's result, in out's own strides."""
    say(f"[strided] {wl.name} {layout}")
    inp = inputs.make_inputs(wl, 8, "discriminating")
    q, k, v = (to_device(x) for x in (inp.Q, inp.K, inp.V))
    if layout == "bnhd":
        qs, ks, vs = _bnhd(q), _bnhd(k), _bnhd(v)
    else:
        qs, ks, vs = _packed_qkv(q, k, v)
    assert not qs.is_contiguous() or wl.H == 1
    out = eav.agent_attn_forward(qs, ks, vs, (wl.h, wl.w), wl.s, wl.scale)
    assert out.stride() == qs.stride()
    torch.cuda.synchronize()
    assert eav.agent_attn_read_faults() == 0
    O, _, _ = oracle.forward(inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w, wl.s, wl.scale)
    parity.assert_close(to_host_f64(out.contiguous()), O, wl.dtype, wl.name + " " + layout,
                        kind="discriminating")


# ------------------------------------------------------ float16 tensors

def _as_f16(wl, name=None):
    return dataclasses.replace(wl, name=name or wl.name + "_f16", dtype="f16")


F16_CASES = [_as_f16(inputs.WORKLOADS[n]) for n in
             ("deit_s", "pvt_stage1", "sd_unet", "sd_unet_agents", "latent_hr")] + [
    # every head-dim class (d <= 32, 64, 128) and agent-tile count (<= 64,
    # 128, 256 agents), ragged windows and a single token
    inputs.custom("f16_d8_s4", B=2, H=2, h=16, w=16, d=8, s=4, dtype="f16"),
    inputs.custom("f16_ragged_57x55_s7", B=1, H=2, h=57, w=55, d=64, s=7, dtype="f16"),
    inputs.custom("f16_d96_s10", B=1, H=2, h=40, w=30, d=96, s=10, dtype="f16"),
    inputs.custom("f16_max_agents_d128", B=1, H=2, h=64, w=48, d=128, s=16, dtype="f16"),
    inputs.custom("f16_bh100_p2", B=25, H=4, h=20, w=20, d=32, s=5, dtype="f16"),
    inputs.custom("f16_single_token", B=3, H=1, h=1, w=1, d=64, s=1, dtype="f16"),
    inputs.custom("f16_supplied_s3", B=2, H=2, h=10, w=10, d=64, s=3, dtype="f16",
                  supplied_agents=True),
]


@pytest.mark.parametrize("wl", F16_CASES, ids=lambda w: w.name)
def test_f16_forward(wl):
    run_case(wl, 30, "iid")
    run_case(wl, 31, "discriminating")


@pytest.mark.parametrize("wl", [F16_CASES[1], F16_CASES[4]], ids=lambda w: w.name)
def test_f16_steps(wl):
    """Pool, aggregation and broadcast steps called one by one on float16
    tensors."""
    say(f"[f16 steps] {wl.name}")
    inp = inputs.make_inputs(wl, 32, "discriminating")
    A = eav.agent_attn_pool(to_device(inp.Q), (wl.h, wl.w), wl.s)
    refA = oracle.pool_agents(inp.Q.exact, wl.h, wl.w, wl.s)
    assert np.abs(to_host_f64(A) - refA).max() <= 1e-5 * max(1.0, np.abs(refA).max())
    A32 = refA.astype(np.float32)
    VA = eav.agent_attn_aggregate(f64_to_device(A32), to_device(inp.K), to_device(inp.V),
                                  wl.scale)
    refVA = oracle.aggregate(A32.astype(np.float64), inp.K.exact, inp.V.exact, wl.scale)
    parity.assert_close(to_host_f64(VA), refVA, "f16", "aggregate " + wl.name,
                        kind="discriminating")
    VA32 = refVA.astype(np.float32)
    out = eav.agent_attn_broadcast(to_device(inp.Q), f64_to_device(A32), f64_to_device(VA32),
                                   wl.scale)
    ref = oracle.broadcast(inp.Q.exact, A32.astype(np.float64), VA32.astype(np.float64),
                           wl.scale)
    parity.assert_close(to_host_f64(out), ref, "f16", "broadcast " + wl.name,
                        kind="discriminating")


def test_f16_strided():
    wl = inputs.custom("f16_bnhd", B=2, H=8, h=32, w=32, d=40, s=8, dtype="f16")
    say(f"[f16 strided] {wl.name}")
    inp = inputs.make_inputs(wl, 33, "discriminating")
    q, k, v = (_bnhd(to_device(x)) for x in (inp.Q, inp.K, inp.V))
    out = eav.agent_attn_forward(q, k, v, (wl.h, wl.w), wl.s, wl.scale)
    assert out.dtype == torch.float16 and out.stride() == q.stride()
    torch.cuda.synchronize()
    assert eav.agent_attn_read_faults() == 0
    O, _, _ = oracle.forward(inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w, wl.s, wl.scale)
    parity.assert_close(to_host_f64(out.contiguous()), O, "f16", wl.name, kind="discriminating")

