"""CPU oracle for the Agent Attention forward pass -- TEST INFRASTRUCTURE ONLY.

Plain, slow and deliberately obvious float64 numpy code.  Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it; the product
path (the HIP library and its Python binding) never does, and this module
imports nothing from the product path.

Sources (web pages about Agent Attention, Han et al., arXiv 2312.08874):
  [Paper]  "Agent Attention: On the Integration of Softmax and Linear
           Attention" (paperlayer.ai summary of arXiv 2312.08874v3).
  [JSQMD]  "Agent Attention：Transformer计算量太大？试试这个'代理令牌'的轻量化方案"
           (jsqmd.com news article).
  [CoreUI] "别再死磕Softmax了！清华黄高团队新作Agent Attention…" (coreui.cn
           article).

What is computed, for every batch b and head h independently:
  1. agents:      A = 2-D average pool of Q over the h x w token grid down to
                  an s x s grid ([Paper] §4 Agent Transformer: agents come
                  from pooling by default; §6 Conclusion: A = f(Q); [JSQMD] §2
                  binds agents to the image grid, e.g. 7 x 7 = 49), unless the
                  caller supplies A ([Paper] §4: learnable agents).
  2. aggregation: V_A = softmax(scale * A K^T) V      ([JSQMD] §1 pseudocode,
                  stage one; [Paper] §4: first of two Softmax attentions).
  3. broadcast:   O   = softmax(scale * Q A^T) V_A    ([JSQMD] §1 pseudocode,
                  stage two; [Paper] §4: second Softmax attention).
The composition equals the generalised linear attention
phi_q(Q) phi_k(K)^T V with phi_q(Q) = softmax(scale Q A^T) and
phi_k(K)^T = softmax(scale A K^T) ([Paper] Abstract and §4).

Readings where the pages leave a step open:
  * pooling windows for agent (i, j) cover rows [floor(i h/s), ceil((i+1) h/s))
    and columns [floor(j w/s), ceil((j+1) w/s)) of the row-major grid (token
    n = r*w + c); agents are numbered i*s + j.  For h, w divisible by s these
    are the plain non-overlapping block means.
  * one scale factor (1/sqrt(d) in every workload) is applied in both
    softmaxes, as in the [JSQMD] §1 pseudocode.
  * the broadcast keys are the agents A (not V_A); projections are not part
    of this operator (module_forward adds them around it: q, k, v from one
    packed Linear of the token features in the order q, k, v, heads split
    head-major, q, k, v and the concatenated heads held in the tensor
    format, an optional output Linear).
  * module enhancements ([Paper] §4 Module Enhancements and Implementation
    Details), optional: agent biases B1 and B2 enter the two attentions as
    additive terms of the scaled logits, softmax(scale A K^T + B1) and
    softmax(scale Q A^T + B2).  The pages name their construction from
    column, row and block components but do not give it, so the full bias
    tensors are inputs here: B1 [H, k, N] and B2 [H, N, k], shared by the
    batch (they are per-head parameters).  The depth-wise convolution term
    has kernel size 3 ([Paper] §4 Efficiency: k^2 N C with k = 3): DWC(V) is
    a per-channel 3 x 3 convolution (cross-correlation, as deep-learning
    convolutions are) of V over the h x w grid with zero padding of one,
    weights W [H*d, 3, 3] and bias b [H*d] (channel c of head h is model
    channel h*d + c), added to the output: O = broadcast + DWC(V).
  * softmax runs over the last axis: over the N keys in aggregation, over
    the k agents in broadcast.
Every function is pinned by tests (library cross-checks, closed forms,
invariants and brute force); see tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np


def window_bounds(i: int, n: int, s: int) -> tuple[int, int]:
    """Half-open range of grid rows (or columns) averaged into agent row i."""
    start = (i * n) // s
    stop = -((-(i + 1) * n) // s)          # ceil((i+1) n / s)
    return start, stop


def pool_agents(Q: np.ndarray, h: int, w: int, s: int) -> np.ndarray:
    """A[b, h, i*s+j, :] = mean of Q over agent (i, j)'s window.

    Q: [B, H, h*w, d] float64 -> A: [B, H, s*s, d] float64.
    ([Paper] §4 and §6: agents are pooled from the queries by default.)
    """
    B, H, N, d = Q.shape
    assert N == h * w and 1 <= s <= h and s <= w
    grid = Q.reshape(B, H, h, w, d)
    A = np.empty((B, H, s * s, d), dtype=np.float64)
    for i in range(s):
        r0, r1 = window_bounds(i, h, s)
        for j in range(s):
            c0, c1 = window_bounds(j, w, s)
            A[:, :, i * s + j, :] = grid[:, :, r0:r1, c0:c1, :].mean(axis=(2, 3))
    return A


def softmax_last(S: np.ndarray) -> np.ndarray:
    """Row-wise softmax over the last axis; rows are checked to sum to one."""
    E = np.exp(S - S.max(axis=-1, keepdims=True))
    P = E / E.sum(axis=-1, keepdims=True)
    assert np.allclose(P.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    return P


def aggregate(A: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
              bias=None) -> np.ndarray:
    """Agent aggregation: V_A = softmax(scale * A K^T [+ B1]) V, per (b, h).

    A: [B, H, k, d], K, V: [B, H, N, d] -> V_A: [B, H, k, d].
    bias: None or B1 [H, k, N], added to the scaled logits of every batch
    entry ([Paper] §4 Module Enhancements: agent bias in both attentions).
    ([JSQMD] §1, stage one; [Paper] §4, first Softmax attention.)
    """
    S1 = scale * (A @ np.swapaxes(K, -1, -2))          # [B, H, k, N]
    if bias is not None:
        S1 = S1 + np.asarray(bias, dtype=np.float64)[None]
    return softmax_last(S1) @ V


def broadcast(Q: np.ndarray, A: np.ndarray, V_A: np.ndarray, scale: float,
              bias=None) -> np.ndarray:
    """Agent broadcast: O = softmax(scale * Q A^T [+ B2]) V_A, per (b, h).

    Q: [B, H, N, d], A, V_A: [B, H, k, d] -> O: [B, H, N, d].
    bias: None or B2 [H, N, k], added to the scaled logits of every batch
    entry ([Paper] §4 Module Enhancements).
    ([JSQMD] §1, stage two; [Paper] §4, second Softmax attention.)
    """
    S2 = scale * (Q @ np.swapaxes(A, -1, -2))          # [B, H, N, k]
    if bias is not None:
        S2 = S2 + np.asarray(bias, dtype=np.float64)[None]
    return softmax_last(S2) @ V_A


def dwc(V: np.ndarray, h: int, w: int, weight: np.ndarray, bias=None) -> np.ndarray:
    """Depth-wise 3 x 3 convolution of V over the h x w token grid.

    out[b, hd, r*w + c, ch] = bias[hd*d + ch]
        + sum over dy, dx in {-1, 0, 1} of
          weight[hd*d + ch, dy + 1, dx + 1] * V[b, hd, (r+dy)*w + (c+dx), ch],
    where taps outside the grid contribute zero (padding one).
    V: [B, H, h*w, d]; weight: [H*d, 3, 3]; bias: None (zero) or [H*d].
    ([Paper] §4 Module Enhancements and Efficiency: the depth-wise
    convolution term, kernel size 3.)
    """
    V = np.asarray(V, dtype=np.float64)
    B, H, N, d = V.shape
    assert N == h * w
    W = np.asarray(weight, dtype=np.float64).reshape(H, d, 3, 3)
    bb = np.zeros((H, d)) if bias is None else np.asarray(bias, dtype=np.float64).reshape(H, d)
    grid = V.reshape(B, H, h, w, d)
    out = np.empty_like(grid)
    out[...] = bb[None, :, None, None, :]
    for dy in (-1, 0, 1):
        for dx in (-1, 0, 1):
            # rows r with 0 <= r + dy < h, columns c with 0 <= c + dx < w
            r0, r1 = max(0, -dy), min(h, h - dy)
            c0, c1 = max(0, -dx), min(w, w - dx)
            tap = W[:, :, dy + 1, dx + 1]                      # [H, d]
            out[:, :, r0:r1, c0:c1, :] += (tap[None, :, None, None, :] *
                                           grid[:, :, r0 + dy:r1 + dy, c0 + dx:c1 + dx, :])
    return out.reshape(B, H, N, d)


def forward(Q, K, V, h: int, w: int, s: int, scale: float, A=None, bias_agg=None,
            bias_bcast=None, dwc_weight=None, dwc_bias=None):
    """Full forward.  Returns (O, A, V_A), all float64.

    Q, K, V: [B, H, h*w, d]; A: None (pool Q to s x s) or [B, H, s*s, d].
    Optional module terms: bias_agg B1 [H, k, N], bias_bcast B2 [H, N, k],
    dwc_weight [H*d, 3, 3] with dwc_bias [H*d] (O += DWC(V)).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if A is None:
        A = pool_agents(Q, h, w, s)
    else:
        A = np.asarray(A, dtype=np.float64)
        assert A.shape == Q.shape[:2] + (s * s, Q.shape[3])
    V_A = aggregate(A, K, V, scale, bias_agg)
    O = broadcast(Q, A, V_A, scale, bias_bcast)
    if dwc_weight is not None:
        O = O + dwc(V, h, w, dwc_weight, dwc_bias)
    return O, A, V_A


# ------------------------------------------------------------ full module

def round_to_format(x: np.ndarray, fmt: str) -> np.ndarray:
    """x rounded to nearest-even in the tensor format fmt ("f32", "bf16" or
    "f16") and widened back to float64: the value a tensor of that format
    holds.  bf16 keeps the top 16 bits of the float32 pattern (8-bit
    significand)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if fmt == "f32":
        return x32.astype(np.float64)
    if fmt == "f16":
        return x32.astype(np.float16).astype(np.float64)
    assert fmt == "bf16", fmt
    u = x32.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
         & np.uint32(0xFFFF0000))
    return r.view(np.float32).astype(np.float64)


def module_forward(X, W_qkv, b_qkv, W_out, b_out, H: int, h: int, w: int, s: int,
                   scale: float, fmt: str, A=None, bias_agg=None, bias_bcast=None,
                   dwc_weight=None, dwc_bias=None):
    """The attention module on token features X [B, N, C] ([Paper] §3
    Preliminaries: the projections W_Q, W_K, W_V map the channels to per-head
    queries, keys and values; §4: agent attention with the agent biases and the depth-wise
    convolution term; [CoreUI] §3.1: AgentAttention(dim, num_heads, num_agents)
    maps [B, N, dim] to [B, N, dim]).

    q, k, v = X W_qkv^T + b_qkv split along the 3C outputs in that order,
    each [B, N, C] read as H heads of d = C / H channels (channel c of head
    hd is feature hd*d + c); they are held in the tensor format fmt, as the
    output of a Linear layer in that format is.  O = forward(q, k, v, ...)
    per head, concatenated back to [B, N, C]; with W_out, that concatenation
    is held in fmt and y = O W_out^T + b_out, else y = O.  Weights in the
    Linear layout [out_features, in_features]; b_qkv, W_out, b_out may be
    None.  Returns y [B, N, C] float64 (unrounded).
    """
    X = np.asarray(X, dtype=np.float64)
    B, N, C = X.shape
    assert C % H == 0 and N == h * w
    d = C // H
    W_qkv = np.asarray(W_qkv, dtype=np.float64)
    assert W_qkv.shape == (3 * C, C)
    qkv = X @ W_qkv.T
    if b_qkv is not None:
        qkv = qkv + np.asarray(b_qkv, dtype=np.float64)
    qkv = round_to_format(qkv, fmt)

    def heads(t):   # [B, N, C] -> [B, H, N, d]
        return np.ascontiguousarray(t.reshape(B, N, H, d).transpose(0, 2, 1, 3))

    q, k, v = heads(qkv[..., :C]), heads(qkv[..., C:2 * C]), heads(qkv[..., 2 * C:])
    O, _, _ = forward(q, k, v, h, w, s, scale, A=A, bias_agg=bias_agg, bias_bcast=bias_bcast,
                      dwc_weight=dwc_weight, dwc_bias=dwc_bias)
    o = O.transpose(0, 2, 1, 3).reshape(B, N, C)
    if W_out is None:
        return o
    y = round_to_format(o, fmt) @ np.asarray(W_out, dtype=np.float64).T
    if b_out is not None:
        y = y + np.asarray(b_out, dtype=np.float64)
    return y


# ------------------------------------------------------------------ backward

def pool_agents_backward(dA: np.ndarray, h: int, w: int, s: int) -> np.ndarray:
    """Gradient of pool_agents: each agent's gradient is spread evenly over
    the tokens of its window (the pooling is a mean), and a token in two
    windows (ragged grids) receives both shares.  dA: [B, H, s*s, d] ->
    dQ: [B, H, h*w, d]."""
    B, H, k, d = dA.shape
    dgrid = np.zeros((B, H, h, w, d))
    for i in range(s):
        r0, r1 = window_bounds(i, h, s)
        for j in range(s):
            c0, c1 = window_bounds(j, w, s)
            cnt = (r1 - r0) * (c1 - c0)
            dgrid[:, :, r0:r1, c0:c1, :] += dA[:, :, i * s + j, None, None, :] / cnt
    return dgrid.reshape(B, H, h * w, d)


def softmax_backward(P: np.ndarray, dP: np.ndarray) -> np.ndarray:
    """Gradient of a row softmax P = softmax(S) with respect to S:
    dS = P * (dP - sum over the row of P * dP)."""
    return P * (dP - (P * dP).sum(axis=-1, keepdims=True))


def backward(Q, K, V, dO, h: int, w: int, s: int, scale: float, A=None):
    """Gradients of the forward O = softmax(scale Q A^T) softmax(scale A K^T) V
    with respect to Q, K, V (and A when the caller supplied it), by the chain
    rule through the two Softmax attentions ([Paper] §4; [JSQMD] §1) and
    the pooling (A = f(Q), [Paper] §6).  With pooled agents, Q receives the
    gradient of the broadcast logits plus the pooled agents' gradient spread
    over their windows.  Returns (dQ, dK, dV, dA) with dA None for pooled
    agents, all float64.
    """
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    supplied = A is not None
    A = np.asarray(A, dtype=np.float64) if supplied else pool_agents(Q, h, w, s)
    KT = np.swapaxes(K, -1, -2)
    P1 = softmax_last(scale * (A @ KT))                       # [B, H, k, N]
    V_A = P1 @ V                                              # [B, H, k, d]
    P2 = softmax_last(scale * (Q @ np.swapaxes(A, -1, -2)))   # [B, H, N, k]
    # broadcast: O = P2 V_A
    dV_A = np.swapaxes(P2, -1, -2) @ dO                       # [B, H, k, d]
    dS2 = softmax_backward(P2, dO @ np.swapaxes(V_A, -1, -2))
    dQ = scale * (dS2 @ A)
    dA = scale * (np.swapaxes(dS2, -1, -2) @ Q)
    # aggregation: V_A = P1 V
    dV = np.swapaxes(P1, -1, -2) @ dV_A
    dS1 = softmax_backward(P1, dV_A @ np.swapaxes(V, -1, -2))
    dA = dA + scale * (dS1 @ K)
    dK = scale * (np.swapaxes(dS1, -1, -2) @ A)
    if supplied:
        return dQ, dK, dV, dA
    return dQ + pool_agents_backward(dA, h, w, s), dK, dV, None
