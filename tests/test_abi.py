"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from efficient_attention_vision_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "agent_attn.h")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_UNSUP, ERR_SCALE, ERR_ALIAS, ERR_ALIGN, ERR_WS = (
    0, -1, -2, -3, -4, -5, -6, -7, -8)

# fake, never dereferenced device addresses: validation fails before any use
P = [ctypes.c_void_p(0x7f0000000000 + i * (1 << 32)) for i in range(8)]
WS = ctypes.c_void_p(0x7f1000000000)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(agent_attn_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _binding.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_binding.EXPORTED)


def fwd(L, *, q=P[0], k=P[1], v=P[2], out=P[3], agents=None, B=2, H=3, h=8, w=8, d=64, s=4,
        scale=0.125, dtype=1, ws=WS, ws_bytes=1 << 40):
    return L.agent_attn_forward_ws(q, k, v, out, agents, B, H, h, w, d, s, scale, dtype, ws,
                                   ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), ERR_NULL),
    (dict(out=None), ERR_NULL),
    (dict(B=-1), ERR_SHAPE),
    (dict(h=0), ERR_SHAPE),
    (dict(s=0), ERR_SHAPE),
    (dict(s=9), ERR_SHAPE),                  # s > h
    (dict(h=40, w=40, s=17), ERR_UNSUP),     # 289 agents
    (dict(d=12), ERR_UNSUP),
    (dict(d=136), ERR_UNSUP),
    (dict(d=0), ERR_SHAPE),
    (dict(dtype=7), ERR_DTYPE),
    (dict(dtype=3), ERR_DTYPE),
    (dict(dtype=-1), ERR_DTYPE),
    (dict(scale=0.0), ERR_SCALE),
    (dict(scale=float("nan")), ERR_SCALE),
    (dict(scale=float("inf")), ERR_SCALE),
    (dict(scale=-1.0), ERR_SCALE),
    (dict(out=P[0]), ERR_ALIAS),
    (dict(out=ctypes.c_void_p(P[1].value + 64)), ERR_ALIAS),
    (dict(q=ctypes.c_void_p(P[0].value + 8)), ERR_ALIGN),
    (dict(ws=None), ERR_WS),
    (dict(ws_bytes=100), ERR_WS),
    (dict(ws=ctypes.c_void_p(WS.value + 16)), ERR_ALIGN),
    (dict(ws=P[1]), ERR_ALIAS),
    (dict(B=1 << 20, H=16), ERR_SHAPE),       # B*H >= 2^23
])
def test_forward_validation(L, kw, code):
    assert fwd(L, **kw) == code
    assert L.agent_attn_last_error().decode() != ""


def test_empty_batch_is_a_no_op(L):
    assert fwd(L, B=0) == OK
    assert fwd(L, H=0, ws=None, ws_bytes=0) == OK
    assert L.agent_attn_workspace_bytes(0, 4, 8, 8, 64, 4, 1) == 0


def test_workspace_bytes(L):
    assert L.agent_attn_workspace_bytes(16, 1, 56, 56, 64, 7, 1) > 0
    assert L.agent_attn_workspace_bytes(16, 1, 56, 56, 12, 7, 1) == 0     # invalid d
    assert L.agent_attn_workspace_bytes(16, 1, 56, 56, 64, 7, 9) == 0     # invalid dtype


def test_float16_is_a_16_bit_dtype(L):
    """float16 plans like bfloat16: the same matrix-core workspace, and the
    same validation (the dtype itself is accepted)."""
    assert L.agent_attn_workspace_bytes(16, 1, 56, 56, 64, 7, 2) == \
        L.agent_attn_workspace_bytes(16, 1, 56, 56, 64, 7, 1)
    assert fwd(L, dtype=2, d=12) == ERR_UNSUP
    assert fwd(L, dtype=2, out=P[0]) == ERR_ALIAS


def test_step_entry_points_validate(L):
    assert L.agent_attn_pool(P[0], None, 1, 1, 8, 8, 64, 2, 1, None) == ERR_NULL
    assert L.agent_attn_pool(P[0], P[1], 1, 1, 8, 8, 64, 9, 1, None) == ERR_SHAPE
    assert L.agent_attn_pool(P[0], P[0], 1, 1, 8, 8, 64, 2, 1, None) == ERR_ALIAS
    assert L.agent_attn_aggregate(P[0], P[1], P[2], P[3], 1, 1, 64, 64, 300, 0.1, 1, WS, 1 << 30,
                                  None) == ERR_UNSUP
    assert L.agent_attn_aggregate(P[0], P[1], P[2], P[3], 1, 1, 64, 64, 16, 0.1, 1, WS, 10,
                                  None) == ERR_WS
    assert L.agent_attn_aggregate(P[0], P[1], P[2], P[1], 1, 1, 64, 64, 16, 0.1, 1, WS, 1 << 30,
                                  None) == ERR_ALIAS
    assert L.agent_attn_broadcast(P[0], P[1], P[2], P[0], 1, 1, 64, 64, 16, 0.1, 1,
                                  None) == ERR_ALIAS
    assert L.agent_attn_broadcast(P[0], P[1], P[2], P[3], 1, 1, 0, 64, 16, 0.1, 1,
                                  None) == ERR_SHAPE
    assert L.agent_attn_broadcast(P[0], P[1], P[2], P[3], 1, 1, 64, 64, 16, 0.0, 1,
                                  None) == ERR_SCALE
    assert L.agent_attn_aggregate_workspace_bytes(2, 2, 1000, 64, 49, 1) > 0


def test_status_strings(L):
    for code in range(-9, 1):
        assert L.agent_attn_status_string(code).decode() not in ("", "unknown status")
    assert L.agent_attn_status_string(-100).decode() == "unknown status"


def test_python_binding_rejects_cpu_tensors():
    import torch
    import efficient_attention_vision_amd as eav
    q = torch.zeros(1, 1, 4, 8)
    with pytest.raises(ValueError):
        eav.agent_attn_forward(q, q, q, (2, 2), 1)


def test_read_faults_needs_an_output(L):
    assert L.agent_attn_read_faults(WS, None, None) == ERR_NULL


def test_wait_limit_query_and_set(L):
    prev = L.agent_attn_set_wait_limit(-1)
    assert prev > 0
    assert L.agent_attn_set_wait_limit(123) == prev
    assert L.agent_attn_set_wait_limit(prev) == 123
    assert L.agent_attn_set_wait_limit(-1) == prev


def strided(L, sb, sh, sn, *, B=2, H=3, h=8, w=8, d=64, s=4, dtype=1):
    return L.agent_attn_forward_strided(P[0], P[1], P[2], P[3], None, B, H, h, w, d, s, sb, sh,
                                        sn, 0.125, dtype, WS, 1 << 40, None)


@pytest.mark.parametrize("sb,sh,sn,code", [
    (64 * 3 * 64, 64, 3 * 64 + 4, ERR_ALIGN),     # token stride not a multiple of 8
    (64 * 3 * 64, 12, 3 * 64, ERR_ALIGN),          # head stride not a multiple of 8
    (64 * 3 * 64, 64, 32, ERR_SHAPE),               # token stride below d
    (64 * 3 * 64, 64, 64, ERR_SHAPE),               # heads and tokens share elements
    (64 * 64, 64 * 64, 64, ERR_SHAPE),              # batches and heads share elements
    (0, 64, 3 * 64, ERR_SHAPE),                     # zero stride
    (-8, 64, 3 * 64, ERR_SHAPE),                    # negative stride
])
def test_strided_validation(L, sb, sh, sn, code):
    assert strided(L, sb, sh, sn) == code


def test_strided_huge_head_span_rejected(L):
    # one head spanning more than 2^31 bytes of bf16
    assert strided(L, 1 << 34, 1 << 33, 1 << 26, B=1, H=1, h=64, w=64) == ERR_SHAPE


# ---------------------------------------------------------- module forward

def modfwd(L, *, b1=None, b2=None, w=None, wb=None, out=P[3], ws=WS, ws_bytes=1 << 40, dtype=1,
           d=64):
    return L.agent_attn_forward_module(P[0], P[1], P[2], out, None, b1, b2, w, wb, 2, 3, 8, 8,
                                       d, 4, 0.125, dtype, ws, ws_bytes, None)


def test_module_forward_validates_its_parameters(L):
    """Misaligned, overlapping or oversized bias / convolution buffers are
    rejected on the host, after the checks of the plain forward."""
    good = ctypes.c_void_p(P[5].value)
    assert modfwd(L, b1=ctypes.c_void_p(good.value + 2)) == ERR_ALIGN
    assert modfwd(L, w=ctypes.c_void_p(good.value + 1)) == ERR_ALIGN
    # out covers [P3, P3 + 2*3*64*64*2): a bias starting inside it aliases
    assert modfwd(L, b2=ctypes.c_void_p(P[3].value + 4096)) == ERR_ALIAS
    assert modfwd(L, wb=ctypes.c_void_p(P[3].value + 64), w=good) == ERR_ALIAS
    # the workspace may not overlap them either
    assert modfwd(L, b1=ctypes.c_void_p(WS.value + 256)) == ERR_ALIAS
    # plain-forward checks still apply
    assert modfwd(L, b1=good, d=12) == ERR_UNSUP
    assert modfwd(L, b1=good, dtype=5) == ERR_DTYPE
    assert modfwd(L, b1=good, ws=None) == ERR_WS
    # a DWC bias without weights is ignored (no alias check against it)
    assert modfwd(L, wb=ctypes.c_void_p(P[3].value + 64), ws_bytes=10) == ERR_WS


# ------------------------------------------------ module with projections

def projfwd(L, *, x=P[0], wqkv=P[1], bqkv=None, wout=None, bout=None, y=P[3], B=2, H=2, h=8,
            w=8, d=32, s=4, scale=0.125, dtype=1, ws=WS, ws_bytes=1 << 40):
    return L.agent_attn_module_forward(x, wqkv, bqkv, wout, bout, None, None, None, None, None,
                                       y, B, H, h, w, d, s, scale, dtype, ws, ws_bytes, None)


def test_projection_module_validation(L):
    """The module with projections checks its own tensors on the host:
    x [B, N, C] and y [B, N, C] with C = H d, weights, float32 biases."""
    assert L.agent_attn_module_workspace_bytes(2, 2, 8, 8, 32, 4, 1) > 0
    assert L.agent_attn_module_workspace_bytes(2, 2, 8, 8, 12, 4, 1) == 0
    assert projfwd(L, x=None) == ERR_NULL
    assert projfwd(L, wqkv=None) == ERR_NULL
    assert projfwd(L, y=None) == ERR_NULL
    assert projfwd(L, x=ctypes.c_void_p(P[0].value + 8)) == ERR_ALIGN
    assert projfwd(L, wout=ctypes.c_void_p(P[2].value + 4)) == ERR_ALIGN
    assert projfwd(L, bqkv=ctypes.c_void_p(P[5].value + 2)) == ERR_ALIGN
    # y [2, 64, 64] bf16 covers 16 KiB from P3: an input starting inside it aliases
    assert projfwd(L, x=ctypes.c_void_p(P[3].value + 4096)) == ERR_ALIAS
    assert projfwd(L, bout=ctypes.c_void_p(P[3].value + 64)) == ERR_ALIAS
    assert projfwd(L, ws=ctypes.c_void_p(P[3].value + 256)) == ERR_ALIAS
    assert projfwd(L, ws=None) == ERR_WS
    assert projfwd(L, ws_bytes=100) == ERR_WS
    assert projfwd(L, d=12) == ERR_UNSUP
    assert projfwd(L, scale=-1.0) == ERR_SCALE
    assert projfwd(L, dtype=9) == ERR_DTYPE
    # 3 C^2 * 4 bytes of weights past 2^31 (C = 16 * 128 * 8)
    assert projfwd(L, H=16 * 8, d=128) == ERR_UNSUP


# ---------------------------------------------------------------- backward

def bwd(L, *, q=P[0], k=P[1], v=P[2], dout=P[3], agents=None, dq=P[4], dk=P[5], dv=P[6],
        da=None, B=2, H=3, h=8, w=8, d=64, s=4, scale=0.125, dtype=1, ws=WS, ws_bytes=1 << 40):
    return L.agent_attn_backward(q, k, v, dout, agents, dq, dk, dv, da, B, H, h, w, d, s, scale,
                                 dtype, ws, ws_bytes, None)


def test_backward_validation(L):
    assert L.agent_attn_backward_workspace_bytes(2, 3, 8, 8, 64, 4, 1) > 0
    assert L.agent_attn_backward_workspace_bytes(2, 3, 8, 8, 12, 4, 1) == 0
    assert bwd(L, dq=None) == ERR_NULL
    assert bwd(L, agents=P[7]) == ERR_NULL                       # agents without dagents
    assert bwd(L, dk=ctypes.c_void_p(P[4].value + 64)) == ERR_ALIAS   # dk inside dq
    assert bwd(L, dv=P[0]) == ERR_ALIAS                          # dv on q
    assert bwd(L, dq=ctypes.c_void_p(P[4].value + 8)) == ERR_ALIGN
    assert bwd(L, d=12) == ERR_UNSUP
    assert bwd(L, scale=0.0) == ERR_SCALE
    assert bwd(L, dtype=4) == ERR_DTYPE
    assert bwd(L, ws=None) == ERR_WS
    assert bwd(L, ws_bytes=16) == ERR_WS
    assert bwd(L, ws=ctypes.c_void_p(P[3].value)) == ERR_ALIAS
    assert bwd(L, B=0) == OK
