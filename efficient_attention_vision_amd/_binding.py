"""ctypes binding of libagent_attn.so (argument marshalling only).

Every step of the forward runs in the library's HIP kernels; this module
only turns torch tensors into pointers and sizes, picks torch's current
stream, allocates the workspace through torch's caching allocator and maps
status codes to exceptions.  There is no fallback: without the built library
every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libagent_attn.so")

F32, BF16, F16 = 0, 1, 2   # agent_attn_dtype_t
OK = 0
_VALIDATION = {-1, -2, -3, -4, -5, -6, -7, -8}

_c_int, _c_size, _c_float, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p

_SIGNATURES = {
    "agent_attn_workspace_bytes": (_c_size, [_c_int] * 7),
    "agent_attn_forward": (_c_int, [_vp] * 5 + [_c_int] * 6 + [_c_float, _c_int, _vp]),
    "agent_attn_forward_ws": (_c_int, [_vp] * 5 + [_c_int] * 6 + [_c_float, _c_int, _vp, _c_size,
                                                                  _vp]),
    "agent_attn_forward_strided": (_c_int, [_vp] * 5 + [_c_int] * 6 + [ctypes.c_longlong] * 3 +
                                   [_c_float, _c_int, _vp, _c_size, _vp]),
    "agent_attn_forward_module": (_c_int, [_vp] * 9 + [_c_int] * 6 + [_c_float, _c_int, _vp,
                                                                       _c_size, _vp]),
    "agent_attn_module_workspace_bytes": (_c_size, [_c_int] * 7),
    "agent_attn_module_forward": (_c_int, [_vp] * 11 + [_c_int] * 6 + [_c_float, _c_int, _vp,
                                                                        _c_size, _vp]),
    "agent_attn_backward_workspace_bytes": (_c_size, [_c_int] * 7),
    "agent_attn_backward": (_c_int, [_vp] * 9 + [_c_int] * 6 + [_c_float, _c_int, _vp, _c_size,
                                                                 _vp]),
    "agent_attn_pool": (_c_int, [_vp, _vp] + [_c_int] * 7 + [_vp]),
    "agent_attn_aggregate_workspace_bytes": (_c_size, [_c_int] * 6),
    "agent_attn_aggregate": (_c_int, [_vp] * 4 + [_c_int] * 5 + [_c_float, _c_int, _vp, _c_size,
                                                                 _vp]),
    "agent_attn_broadcast": (_c_int, [_vp] * 4 + [_c_int] * 5 + [_c_float, _c_int, _vp]),
    "agent_attn_read_faults": (_c_int, [_vp, _vp, ctypes.POINTER(_c_int)]),
    "agent_attn_set_wait_limit": (ctypes.c_long, [ctypes.c_long]),
    "agent_attn_release": (None, []),
    "agent_attn_status_string": (ctypes.c_char_p, [_c_int]),
    "agent_attn_last_error": (ctypes.c_char_p, []),
}

EXPORTED = tuple(_SIGNATURES)

_lib = None


class AgentAttnError(RuntimeError):
    """A HIP failure reported by the library."""


def lib() -> ctypes.CDLL:
    """Load the shared library once (after torch, so that both use the same
    HIP runtime).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m efficient_attention_vision_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc == OK:
        return
    L = lib()
    msg = f"{L.agent_attn_status_string(rc).decode()}: {L.agent_attn_last_error().decode()}"
    if rc in _VALIDATION:
        raise ValueError(msg)
    raise AgentAttnError(msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return F16
    raise ValueError(f"unsupported dtype {t.dtype}; use float32, bfloat16 or float16")


def _dev_tensor(t, name, ndim=4):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _same(ref, t, name, shape=None, dtype=None):
    if t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, expected {ref.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


_ws_cache: dict = {}


def cached_workspace(device, nbytes: int) -> torch.Tensor:
    """A zero-initialised workspace of at least `nbytes` for torch's current
    stream on `device`, reused across calls on that stream (the library
    leaves its synchronisation counters at zero after every call)."""
    device = torch.device(device)
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    t = _ws_cache.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = t
    return t


def agent_attn_workspace_bytes(B, H, h, w, d, s, dtype_code) -> int:
    return int(lib().agent_attn_workspace_bytes(B, H, h, w, d, s, dtype_code))


def agent_attn_backward_workspace_bytes(B, H, h, w, d, s, dtype_code) -> int:
    return int(lib().agent_attn_backward_workspace_bytes(B, H, h, w, d, s, dtype_code))


def _strided_view(t, name):
    """A [B, H, N, d] GPU tensor whose channels are contiguous (any strides
    for the other three dimensions, e.g. a [B, N, H, d] tensor transposed)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != 4:
        raise ValueError(f"{name} must have 4 dimensions, got shape {tuple(t.shape)}")
    if t.stride(3) != 1 and t.shape[3] > 1:
        raise ValueError(f"{name} must have contiguous channels (stride 1 in the last dimension)")
    return t


def agent_attn_forward(q, k, v, grid_hw, s, scale=None, agents=None, out=None, workspace=None):
    """O = softmax(scale Q A^T) softmax(scale A K^T) V with A = 2-D average
    pool of Q to s x s agents (or `agents` [B, H, s*s, d]).

    q, k, v: [B, H, h*w, d] float32, bfloat16 or float16 GPU tensors;
    grid_hw = (h, w).
    Dense tensors use agent_attn_forward_ws; views with contiguous channels
    and the same strides for q, k, v (for example x.view(B, N, H, d)
    .transpose(1, 2)) use agent_attn_forward_strided, with `out` given those
    strides too.  Runs on torch's current stream; returns `out`.
    """
    L = lib()
    _strided_view(q, "q")
    B, H, N, d = q.shape
    h, w = (int(x) for x in grid_hw)
    if h * w != N:
        raise ValueError(f"grid {h}x{w} does not match N={N}")
    dense = q.is_contiguous()
    for name, t in (("k", k), ("v", v)):
        _strided_view(t, name)
        _same(q, t, name, q.shape, q.dtype)
        if dense != t.is_contiguous() or (not dense and t.stride() != q.stride()):
            raise ValueError(f"{name} must have q's strides {q.stride()}, got {t.stride()}")
    if agents is not None:
        _dev_tensor(agents, "agents")
        _same(q, agents, "agents", (B, H, int(s) * int(s), d), q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q) if dense else torch.empty_strided(
            q.shape, q.stride(), dtype=q.dtype, device=q.device)
    else:
        _strided_view(out, "out")
        _same(q, out, "out", q.shape, q.dtype)
        if dense != out.is_contiguous() or (not dense and out.stride() != q.stride()):
            raise ValueError(f"out must have q's strides {q.stride()}, got {out.stride()}")
    code = _dtype_code(q)
    with torch.cuda.device(q.device):
        need = L.agent_attn_workspace_bytes(B, H, h, w, d, int(s), code)
        ws_ptr, ws_size = None, 0
        if need > 0:      # 0: invalid sizes (reported by the call) or an empty batch
            if workspace is None:
                workspace = cached_workspace(q.device, need)
            ws_ptr, ws_size = _ptr(workspace), workspace.numel() * workspace.element_size()
        if dense:
            rc = L.agent_attn_forward_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(agents), B, H,
                                         h, w, d, int(s), float(scale), code, ws_ptr, ws_size,
                                         _stream(q.device))
        else:
            sb, sh, sn, _ = q.stride()
            rc = L.agent_attn_forward_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(agents),
                                              B, H, h, w, d, int(s), sb, sh, sn, float(scale),
                                              code, ws_ptr, ws_size, _stream(q.device))
    _check(rc)
    return out


def agent_attn_forward_module(q, k, v, grid_hw, s, scale=None, agents=None, bias_agg=None,
                              bias_bcast=None, dwc_weight=None, dwc_bias=None, out=None,
                              workspace=None):
    """The full module's forward: softmax(scale Q A^T + B2) softmax(scale A
    K^T + B1) V + DWC(V) ("Agent Attention: On the Integration of Softmax
    and Linear Attention", §4 Module Enhancements).

    q, k, v: dense [B, H, h*w, d] GPU tensors (float32, bfloat16 or float16).
    bias_agg B1 [H, s*s, N], bias_bcast B2 [H, N, s*s], dwc_weight
    [H*d, 3, 3] and dwc_bias [H*d]: float32 GPU tensors or None.
    Runs on torch's current stream; returns `out`.
    """
    L = lib()
    _dev_tensor(q, "q")
    B, H, N, d = q.shape
    h, w = (int(x) for x in grid_hw)
    if h * w != N:
        raise ValueError(f"grid {h}x{w} does not match N={N}")
    k_ag = int(s) * int(s)
    for name, t in (("k", k), ("v", v)):
        _dev_tensor(t, name)
        _same(q, t, name, q.shape, q.dtype)
    if agents is not None:
        _dev_tensor(agents, "agents")
        _same(q, agents, "agents", (B, H, k_ag, d), q.dtype)
    shapes = {"bias_agg": (H, k_ag, N), "bias_bcast": (H, N, k_ag),
              "dwc_weight": (H * d, 3, 3), "dwc_bias": (H * d,)}
    params = {"bias_agg": bias_agg, "bias_bcast": bias_bcast, "dwc_weight": dwc_weight,
              "dwc_bias": dwc_bias}
    for name, t in params.items():
        if t is None:
            continue
        _dev_tensor(t, name, ndim=len(shapes[name]))
        _same(q, t, name, shapes[name], torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev_tensor(out, "out")
        _same(q, out, "out", q.shape, q.dtype)
    code = _dtype_code(q)
    with torch.cuda.device(q.device):
        need = L.agent_attn_workspace_bytes(B, H, h, w, d, int(s), code)
        ws_ptr, ws_size = None, 0
        if need > 0:
            if workspace is None:
                workspace = cached_workspace(q.device, need)
            ws_ptr, ws_size = _ptr(workspace), workspace.numel() * workspace.element_size()
        rc = L.agent_attn_forward_module(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(agents),
                                         _ptr(bias_agg), _ptr(bias_bcast), _ptr(dwc_weight),
                                         _ptr(dwc_bias), B, H, h, w, d, int(s), float(scale),
                                         code, ws_ptr, ws_size, _stream(q.device))
    _check(rc)
    return out


def agent_attn_module_forward(x, w_qkv, grid_hw, s, num_heads, scale=None, b_qkv=None,
                              w_out=None, b_out=None, agents=None, bias_agg=None,
                              bias_bcast=None, dwc_weight=None, dwc_bias=None, out=None,
                              workspace=None):
    """The attention module on token features x [B, h*w, C]: q, k, v = x
    w_qkv^T + b_qkv (order q, k, v; H = num_heads heads of d = C / H
    channels), agent attention with the optional module terms, y = o w_out^T
    + b_out (y = o, heads side by side, without w_out).  Weights in the
    Linear layout [out, in] and x's dtype; biases float32.  Returns y
    [B, h*w, C]; runs on torch's current stream."""
    L = lib()
    _dev_tensor(x, "x", ndim=3)
    B, N, C = x.shape
    H = int(num_heads)
    if H < 1 or C % H:
        raise ValueError(f"C={C} is not a multiple of num_heads={H}")
    d = C // H
    h, w = (int(t) for t in grid_hw)
    if h * w != N:
        raise ValueError(f"grid {h}x{w} does not match N={N}")
    k_ag = int(s) * int(s)
    _dev_tensor(w_qkv, "w_qkv", ndim=2)
    _same(x, w_qkv, "w_qkv", (3 * C, C), x.dtype)
    if w_out is not None:
        _dev_tensor(w_out, "w_out", ndim=2)
        _same(x, w_out, "w_out", (C, C), x.dtype)
    if agents is not None:
        _dev_tensor(agents, "agents")
        _same(x, agents, "agents", (B, H, k_ag, d), x.dtype)
    shapes = {"b_qkv": (3 * C,), "b_out": (C,), "bias_agg": (H, k_ag, N),
              "bias_bcast": (H, N, k_ag), "dwc_weight": (H * d, 3, 3), "dwc_bias": (H * d,)}
    params = {"b_qkv": b_qkv, "b_out": b_out, "bias_agg": bias_agg, "bias_bcast": bias_bcast,
              "dwc_weight": dwc_weight, "dwc_bias": dwc_bias}
    for name, t in params.items():
        if t is None:
            continue
        _dev_tensor(t, name, ndim=len(shapes[name]))
        _same(x, t, name, shapes[name], torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(x)
    else:
        _dev_tensor(out, "out", ndim=3)
        _same(x, out, "out", x.shape, x.dtype)
    code = _dtype_code(x)
    with torch.cuda.device(x.device):
        need = L.agent_attn_module_workspace_bytes(B, H, h, w, d, int(s), code)
        if workspace is None:   # leading synchronisation bytes zero, as the call leaves them
            workspace = cached_workspace(x.device, max(1, need))
        ws_size = workspace.numel() * workspace.element_size()
        rc = L.agent_attn_module_forward(
            _ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(w_out), _ptr(b_out), _ptr(agents),
            _ptr(bias_agg), _ptr(bias_bcast), _ptr(dwc_weight), _ptr(dwc_bias), _ptr(out),
            B, H, h, w, d, int(s), float(scale), code, _ptr(workspace), ws_size,
            _stream(x.device))
    _check(rc)
    return out


def agent_attn_backward(q, k, v, dout, grid_hw, s, scale=None, agents=None, workspace=None):
    """Gradients (dq, dk, dv, dagents) of the forward agent_attn_forward(q, k,
    v, grid_hw, s, scale, agents) for the output gradient dout.  dagents is
    None for pooled agents (their gradient is part of dq).  Dense
    [B, H, h*w, d] GPU tensors of one dtype; runs on torch's current stream."""
    L = lib()
    _dev_tensor(q, "q")
    B, H, N, d = q.shape
    h, w = (int(x) for x in grid_hw)
    if h * w != N:
        raise ValueError(f"grid {h}x{w} does not match N={N}")
    for name, t in (("k", k), ("v", v), ("dout", dout)):
        _dev_tensor(t, name)
        _same(q, t, name, q.shape, q.dtype)
    if agents is not None:
        _dev_tensor(agents, "agents")
        _same(q, agents, "agents", (B, H, int(s) * int(s), d), q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    da = torch.empty_like(agents) if agents is not None else None
    code = _dtype_code(q)
    with torch.cuda.device(q.device):
        need = L.agent_attn_backward_workspace_bytes(B, H, h, w, d, int(s), code)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        rc = L.agent_attn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(agents), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(da), B, H, h, w, d, int(s),
                                   float(scale), code, _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _stream(q.device))
    _check(rc)
    return dq, dk, dv, da


def agent_attn_forward_cached(q, k, v, grid_hw, s, scale=None, agents=None, out=None):
    """agent_attn_forward through the library's own cached workspace."""
    L = lib()
    _dev_tensor(q, "q")
    B, H, N, d = q.shape
    h, w = (int(x) for x in grid_hw)
    if h * w != N:
        raise ValueError(f"grid {h}x{w} does not match N={N}")
    for name, t in (("k", k), ("v", v)):
        _dev_tensor(t, name)
        _same(q, t, name, q.shape, q.dtype)
    if agents is not None:
        _dev_tensor(agents, "agents")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    with torch.cuda.device(q.device):
        rc = L.agent_attn_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(agents), B, H, h, w,
                                  d, int(s), float(scale), _dtype_code(q), _stream(q.device))
    _check(rc)
    return out


def agent_attn_pool(q, grid_hw, s, out=None):
    """float32 agents [B, H, s*s, d] = 2-D average pool of q over its h x w grid."""
    L = lib()
    _dev_tensor(q, "q")
    B, H, N, d = q.shape
    h, w = (int(x) for x in grid_hw)
    if h * w != N:
        raise ValueError(f"grid {h}x{w} does not match N={N}")
    if out is None:
        out = torch.empty((B, H, int(s) * int(s), d), dtype=torch.float32, device=q.device)
    else:
        _dev_tensor(out, "out")
        _same(q, out, "out", (B, H, int(s) * int(s), d), torch.float32)
    with torch.cuda.device(q.device):
        rc = L.agent_attn_pool(_ptr(q), _ptr(out), B, H, h, w, d, int(s), _dtype_code(q),
                               _stream(q.device))
    _check(rc)
    return out


def agent_attn_aggregate(agents_f32, k, v, scale, out=None):
    """float32 V_A [B, H, n_agents, d] = softmax(scale agents k^T) v."""
    L = lib()
    _dev_tensor(k, "k")
    B, H, N, d = k.shape
    _dev_tensor(v, "v")
    _same(k, v, "v", k.shape, k.dtype)
    _dev_tensor(agents_f32, "agents_f32")
    if agents_f32.shape[:2] != (B, H) or agents_f32.shape[3] != d:
        raise ValueError(f"agents_f32 shape {tuple(agents_f32.shape)} does not match k")
    _same(k, agents_f32, "agents_f32", dtype=torch.float32)
    nag = agents_f32.shape[2]
    if out is None:
        out = torch.empty_like(agents_f32)
    else:
        _dev_tensor(out, "out")
        _same(k, out, "out", agents_f32.shape, torch.float32)
    code = _dtype_code(k)
    with torch.cuda.device(k.device):
        need = L.agent_attn_aggregate_workspace_bytes(B, H, N, d, nag, code)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=k.device)
        rc = L.agent_attn_aggregate(_ptr(agents_f32), _ptr(k), _ptr(v), _ptr(out), B, H, N, d,
                                    nag, float(scale), code, _ptr(ws), ws.numel(),
                                    _stream(k.device))
    _check(rc)
    return out


def agent_attn_broadcast(q, agents_f32, agent_values_f32, scale, out=None):
    """out [B, H, N, d] (q's dtype) = softmax(scale q agents^T) agent_values."""
    L = lib()
    _dev_tensor(q, "q")
    B, H, N, d = q.shape
    for name, t in (("agents_f32", agents_f32), ("agent_values_f32", agent_values_f32)):
        _dev_tensor(t, name)
        _same(q, t, name, dtype=torch.float32)
    nag = agents_f32.shape[2]
    if tuple(agents_f32.shape) != (B, H, nag, d) or agent_values_f32.shape != agents_f32.shape:
        raise ValueError("agents_f32 and agent_values_f32 must both be [B, H, n_agents, d]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev_tensor(out, "out")
        _same(q, out, "out", q.shape, q.dtype)
    with torch.cuda.device(q.device):
        rc = L.agent_attn_broadcast(_ptr(q), _ptr(agents_f32), _ptr(agent_values_f32), _ptr(out),
                                    B, H, N, d, nag, float(scale), _dtype_code(q),
                                    _stream(q.device))
    _check(rc)
    return out


FAULT_BARRIER, FAULT_XCD = 1, 2


def agent_attn_read_faults(workspace=None, device=None) -> int:
    """Wait for torch's current stream, then read and clear the fault word
    (AGENT_ATTN_FAULT_* bits; 0 = every forward since the last read ran
    normally) of `workspace`; with no workspace, of both this module's
    cached workspace for the current stream and the library's own scratch."""
    L = lib()
    if workspace is not None:
        device = workspace.device
    device = torch.device(device if device is not None else "cuda")
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    if workspace is not None:
        targets = [workspace]
    else:
        cached = _ws_cache.get((device.index, torch.cuda.current_stream(device).cuda_stream))
        targets = ([cached] if cached is not None else []) + [None]
    word = 0
    with torch.cuda.device(device):
        for t in targets:
            f = _c_int(0)
            _check(L.agent_attn_read_faults(_ptr(t), _stream(device), ctypes.byref(f)))
            word |= f.value
    return word


def agent_attn_set_wait_limit(polls: int) -> int:
    """Polls at a group barrier before a workgroup gives up (negative: only
    query); returns the previous value."""
    return int(lib().agent_attn_set_wait_limit(int(polls)))


def agent_attn_release() -> None:
    lib().agent_attn_release()
