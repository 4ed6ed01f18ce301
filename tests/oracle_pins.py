"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes the oracle module and raises AssertionError if the oracle
disagrees with what the pages and the mathematics fix:
  * independent library routines for the special cases that reduce to them
    (torch's adaptive_avg_pool2d for the pooling, torch's float64
    scaled_dot_product_attention for each of the two Softmax attention
    operations that "Agent Attention: On the Integration of Softmax and Linear
    Attention" (§1, §4) says the method consists of);
  * closed forms (one agent; all keys equal; constant values; hand-derived
    examples with exact rational softmax weights);
  * invariants (key translation, joint key/value permutation, agent
    permutation, outputs as convex combinations of value rows);
  * brute force with explicit loops on tiny inputs, including the explicit
    N x N generalised-linear-attention matrix
    softmax(Q A^T) softmax(A K^T) (Abstract and §4 of the same page).
The mutation tests plant plausible mistakes in the oracle and require that at
least one pin fails for each.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))


def _sdpa(q, k, v, scale):
    return F.scaled_dot_product_attention(_t(q), _t(k), _t(v), scale=scale).numpy()


def _torch_pool(Q, h, w, s):
    B, H, N, d = Q.shape
    x = _t(Q).reshape(B * H, h, w, d).permute(0, 3, 1, 2)
    y = F.adaptive_avg_pool2d(x, (s, s))                  # [B*H, d, s, s]
    return y.permute(0, 2, 3, 1).reshape(B, H, s * s, d).numpy()


# --------------------------------------------------------------------- pooling

def pin_pool_vs_adaptive_avg_pool2d(orc):
    for seed, (B, H, h, w, d, s) in enumerate([
            (2, 3, 14, 14, 8, 7), (1, 2, 7, 9, 5, 4), (1, 1, 5, 3, 4, 3),
            (1, 1, 56, 56, 4, 7), (2, 1, 10, 6, 3, 1), (1, 1, 9, 16, 2, 5)]):
        Q = _rng(seed).standard_normal((B, H, h * w, d))
        A = orc.pool_agents(Q, h, w, s)
        ref = _torch_pool(Q, h, w, s)
        assert A.shape == ref.shape
        assert np.allclose(A, ref, rtol=0, atol=1e-12), (h, w, s)


def pin_pool_explicit_loops(orc):
    """Window sums by explicit token indexing n = r*w + c on a tiny grid."""
    h, w, s, d = 5, 4, 2, 3
    Q = _rng(11).standard_normal((1, 1, h * w, d))
    A = orc.pool_agents(Q, h, w, s)
    # agent row i covers grid rows [floor(i*h/s), ceil((i+1)*h/s))
    rows = {0: [0, 1, 2], 1: [2, 3, 4]}
    cols = {0: [0, 1], 1: [2, 3]}
    for i in range(s):
        for j in range(s):
            acc = [0.0] * d
            cnt = 0
            for r in rows[i]:
                for c in cols[j]:
                    for ch in range(d):
                        acc[ch] += Q[0, 0, r * w + c, ch]
                    cnt += 1
            for ch in range(d):
                assert abs(A[0, 0, i * s + j, ch] - acc[ch] / cnt) < 1e-13


def pin_pool_window_one_is_identity(orc):
    h, w, d = 6, 6, 5
    Q = _rng(12).standard_normal((2, 2, h * w, d))
    assert np.array_equal(orc.pool_agents(Q, h, w, h), Q)


# --------------------------------------------------- the two softmax attentions

def pin_aggregate_is_softmax_attention(orc):
    rng = _rng(21)
    B, H, N, k, d, scale = 2, 3, 37, 9, 16, 0.37
    A = 2.0 * rng.standard_normal((B, H, k, d))
    K = rng.standard_normal((B, H, N, d))
    V = rng.standard_normal((B, H, N, d))
    assert np.allclose(orc.aggregate(A, K, V, scale), _sdpa(A, K, V, scale),
                       rtol=0, atol=1e-12)


def pin_broadcast_is_softmax_attention(orc):
    rng = _rng(22)
    B, H, N, k, d, scale = 2, 3, 41, 9, 16, 0.41
    Q = 2.0 * rng.standard_normal((B, H, N, d))
    A = rng.standard_normal((B, H, k, d))
    VA = rng.standard_normal((B, H, k, d))
    assert np.allclose(orc.broadcast(Q, A, VA, scale), _sdpa(Q, A, VA, scale),
                       rtol=0, atol=1e-12)


def pin_forward_is_pool_then_two_attentions(orc):
    rng = _rng(23)
    B, H, h, w, d, s, scale = 2, 2, 6, 10, 8, 3, 0.5
    Q = 1.5 * rng.standard_normal((B, H, h * w, d))
    K = 1.5 * rng.standard_normal((B, H, h * w, d))
    V = rng.standard_normal((B, H, h * w, d))
    O, A, VA = orc.forward(Q, K, V, h, w, s, scale)
    A_ref = _torch_pool(Q, h, w, s)
    VA_ref = _sdpa(A_ref, K, V, scale)
    O_ref = _sdpa(Q, A_ref, VA_ref, scale)
    for got, ref in ((A, A_ref), (VA, VA_ref), (O, O_ref)):
        assert np.allclose(got, ref, rtol=0, atol=1e-12)
    # caller-supplied agents bypass pooling
    A2 = rng.standard_normal((B, H, s * s, d))
    O2, A2_out, VA2 = orc.forward(Q, K, V, h, w, s, scale, A=A2)
    assert np.array_equal(A2_out, A2)
    assert np.allclose(O2, _sdpa(Q, A2, _sdpa(A2, K, V, scale), scale),
                       rtol=0, atol=1e-12)


def pin_one_agent_per_token_is_textbook_attention(orc):
    """s = h = w: every agent is its own query, so V_A is textbook attention."""
    rng = _rng(24)
    h = w = 5
    Q, K, V = (rng.standard_normal((1, 2, h * w, 8)) for _ in range(3))
    _, A, VA = orc.forward(Q, K, V, h, w, h, 0.6)
    assert np.array_equal(A, Q)
    assert np.allclose(VA, _sdpa(Q, K, V, 0.6), rtol=0, atol=1e-12)


# ------------------------------------------------------------- closed forms

def pin_single_agent_closed_form(orc):
    """s = 1: the broadcast softmax has one entry, so every O row is V_A[0],
    and V_A[0] is the softmax attention of the single query mean(Q)."""
    rng = _rng(31)
    h, w, d, scale = 4, 5, 3, 0.7
    Q, K, V = (rng.standard_normal((1, 1, h * w, d)) for _ in range(3))
    O, _, VA = orc.forward(Q, K, V, h, w, 1, scale)
    N = h * w
    a = [sum(Q[0, 0, n, c] for n in range(N)) / N for c in range(d)]
    logits = [scale * sum(a[c] * K[0, 0, n, c] for c in range(d)) for n in range(N)]
    mx = max(logits)
    e = [math.exp(x - mx) for x in logits]
    z = sum(e)
    va = [sum(e[n] / z * V[0, 0, n, c] for n in range(N)) for c in range(d)]
    assert np.allclose(VA[0, 0, 0], va, rtol=0, atol=1e-13)
    assert np.allclose(O[0, 0], np.broadcast_to(va, (N, d)), rtol=0, atol=1e-13)


def pin_equal_keys_average_values(orc):
    """All keys equal: the aggregation weights are uniform, so every output
    row is the mean of V whatever Q and A are."""
    rng = _rng(32)
    h, w, d, s = 6, 6, 4, 3
    Q = 3 * rng.standard_normal((1, 2, h * w, d))
    K = np.broadcast_to(rng.standard_normal((1, 2, 1, d)), (1, 2, h * w, d)).copy()
    V = rng.standard_normal((1, 2, h * w, d))
    O, _, _ = orc.forward(Q, K, V, h, w, s, 0.9)
    assert np.allclose(O, np.broadcast_to(V.mean(axis=2, keepdims=True), O.shape),
                       rtol=0, atol=1e-13)


def pin_constant_values(orc):
    rng = _rng(33)
    h, w, d, s = 4, 6, 5, 2
    Q, K = (2 * rng.standard_normal((2, 1, h * w, d)) for _ in range(2))
    v = rng.standard_normal((2, 1, 1, d))
    V = np.broadcast_to(v, (2, 1, h * w, d)).copy()
    O, _, _ = orc.forward(Q, K, V, h, w, s, 0.8)
    assert np.allclose(O, np.broadcast_to(v, O.shape), rtol=0, atol=1e-13)


def pin_hand_examples(orc):
    """Two examples worked by hand with exact softmax weights.

    (1) 2x2 grid, one agent (s=1), scale 1.  Q rows (1,1),(1,-1),(1,3),(1,-3)
        pool to A = (1, 0).  Key first components ln1, ln2, ln3, ln1 give
        aggregation weights (1,2,3,1)/7; values (7,0),(0,7),(14,-7),(0,0)
        give V_A = (49, -7)/7 = (7, -1), and every output row is (7, -1).
    (2) 2x2 grid, s=2 (each agent is one token, A = Q), Q = identity rows in
        d=4, scale 1.  K[n, i] = ln m[i][n] makes the aggregation weights
        m[i][n] / sum_n m[i][n]; the broadcast logits are the identity, so
        O[n] = ((e-1) V_A[n] + sum_j V_A[j]) / (e + 3).
    """
    Q = np.array([[1, 1], [1, -1], [1, 3], [1, -3]], float)[None, None]
    K = np.array([[0, 5], [math.log(2), -7], [math.log(3), 2], [0, 0]], float)[None, None]
    V = np.array([[7, 0], [0, 7], [14, -7], [0, 0]], float)[None, None]
    O, A, VA = orc.forward(Q, K, V, 2, 2, 1, 1.0)
    assert np.allclose(A[0, 0], [[1, 0]], rtol=0, atol=1e-15)
    assert np.allclose(VA[0, 0], [[7, -1]], rtol=0, atol=1e-13)
    assert np.allclose(O[0, 0], [[7, -1]] * 4, rtol=0, atol=1e-13)

    m = [[1, 1, 1, 1], [1, 2, 3, 4], [4, 3, 2, 1], [1, 1, 2, 4]]
    Vi = [[3, -1, 0, 2], [5, 4, -2, 0], [-6, 1, 1, 1], [0, 0, 8, -4]]
    Q = np.eye(4)[None, None]
    K = np.array([[math.log(m[i][n]) for i in range(4)] for n in range(4)])[None, None]
    V = np.array(Vi, float)[None, None]
    VA_exact = [[sum(Fraction(m[i][n]) * Vi[n][c] for n in range(4)) / sum(m[i])
                 for c in range(4)] for i in range(4)]
    tot = [sum(VA_exact[j][c] for j in range(4)) for c in range(4)]
    O_exact = [[((math.e - 1) * float(VA_exact[n][c]) + float(tot[c])) / (math.e + 3)
                for c in range(4)] for n in range(4)]
    O, A, VA = orc.forward(Q, K, V, 2, 2, 2, 1.0)
    assert np.array_equal(A[0, 0], np.eye(4))
    assert np.allclose(VA[0, 0], [[float(x) for x in r] for r in VA_exact], rtol=0, atol=1e-13)
    assert np.allclose(O[0, 0], O_exact, rtol=0, atol=1e-13)


# --------------------------------------------------------------- invariants

def pin_key_translation_invariance(orc):
    rng = _rng(41)
    h, w, d, s = 6, 8, 6, 2
    Q, K, V = (rng.standard_normal((2, 2, h * w, d)) for _ in range(3))
    u = rng.standard_normal((2, 2, 1, d))
    O1, _, _ = orc.forward(Q, K, V, h, w, s, 0.5)
    O2, _, _ = orc.forward(Q, K + u, V, h, w, s, 0.5)
    assert np.allclose(O1, O2, rtol=0, atol=1e-12)


def pin_joint_key_value_permutation(orc):
    rng = _rng(42)
    h, w, d, s = 6, 8, 6, 2
    Q, K, V = (rng.standard_normal((2, 2, h * w, d)) for _ in range(3))
    p = rng.permutation(h * w)
    O1, _, _ = orc.forward(Q, K, V, h, w, s, 0.5)
    O2, _, _ = orc.forward(Q, K[:, :, p], V[:, :, p], h, w, s, 0.5)
    assert np.allclose(O1, O2, rtol=0, atol=1e-12)


def pin_agent_permutation(orc):
    rng = _rng(43)
    h, w, d, s = 6, 6, 6, 3
    Q, K, V = (rng.standard_normal((1, 2, h * w, d)) for _ in range(3))
    A = rng.standard_normal((1, 2, s * s, d))
    p = rng.permutation(s * s)
    O1, _, _ = orc.forward(Q, K, V, h, w, s, 0.7, A=A)
    O2, _, _ = orc.forward(Q, K, V, h, w, s, 0.7, A=A[:, :, p])
    assert np.allclose(O1, O2, rtol=0, atol=1e-12)


def pin_outputs_are_convex_combinations(orc):
    rng = _rng(44)
    h, w, d, s = 8, 8, 7, 4
    Q, K = (3 * rng.standard_normal((2, 2, h * w, d)) for _ in range(2))
    V = rng.standard_normal((2, 2, h * w, d))
    O, _, VA = orc.forward(Q, K, V, h, w, s, 0.8)
    lo = V.min(axis=2, keepdims=True) - 1e-12
    hi = V.max(axis=2, keepdims=True) + 1e-12
    assert np.all((VA >= lo) & (VA <= hi))
    assert np.all((O >= lo) & (O <= hi))


# ---------------------------------------------------------------- brute force

def _softmax_loops(row):
    mx = max(row)
    e = [math.exp(x - mx) for x in row]
    z = sum(e)
    return [x / z for x in e]


def pin_brute_force_generalised_linear_attention(orc):
    """O = softmax(s Q A^T) softmax(s A K^T) V with the N x N product formed
    explicitly, by loops, on tiny inputs; for pooled and supplied agents."""
    rng = _rng(51)
    h, w, d, s, scale = 4, 6, 3, 2, 0.9
    N, k = h * w, s * s
    Q, K, V = (1.5 * rng.standard_normal((1, 1, N, d)) for _ in range(3))
    for A in (None, rng.standard_normal((1, 1, k, d))):
        O, A_used, _ = orc.forward(Q, K, V, h, w, s, scale, A=A)
        a = A_used[0, 0]
        q, kk, v = Q[0, 0], K[0, 0], V[0, 0]
        phi_q = [_softmax_loops([scale * sum(q[n, c] * a[i, c] for c in range(d))
                                 for i in range(k)]) for n in range(N)]
        phi_k = [_softmax_loops([scale * sum(a[i, c] * kk[m, c] for c in range(d))
                                 for m in range(N)]) for i in range(k)]
        M = [[sum(phi_q[n][i] * phi_k[i][m] for i in range(k)) for m in range(N)]
             for n in range(N)]
        ref = [[sum(M[n][m] * v[m, c] for m in range(N)) for c in range(d)]
               for n in range(N)]
        assert np.allclose(O[0, 0], ref, rtol=0, atol=1e-12)


# ------------------------------------------- module terms: agent biases, DWC

def _sdpa_mask(q, k, v, mask, scale):
    """torch's float64 attention with an additive float mask on the scaled
    logits (broadcast over the batch)."""
    return F.scaled_dot_product_attention(_t(q), _t(k), _t(v), attn_mask=_t(mask),
                                          scale=scale).numpy()


def pin_aggregate_bias_is_masked_attention(orc):
    """With B1, the aggregation is torch's attention with B1 as its additive
    float mask ([Paper] §4: the bias enters the attention logits)."""
    rng = _rng(61)
    B, H, N, k, d, scale = 2, 3, 11, 5, 4, 0.7
    A, K, V = (rng.standard_normal(sh) for sh in ((B, H, k, d), (B, H, N, d), (B, H, N, d)))
    B1 = 2.0 * rng.standard_normal((H, k, N))
    got = orc.aggregate(A, K, V, scale, B1)
    assert np.allclose(got, _sdpa_mask(A, K, V, B1[None], scale), rtol=0, atol=1e-12)


def pin_broadcast_bias_is_masked_attention(orc):
    rng = _rng(62)
    B, H, N, k, d, scale = 2, 2, 9, 6, 5, 0.6
    Q, A, VA = (rng.standard_normal(sh) for sh in ((B, H, N, d), (B, H, k, d), (B, H, k, d)))
    B2 = 2.0 * rng.standard_normal((H, N, k))
    got = orc.broadcast(Q, A, VA, scale, B2)
    assert np.allclose(got, _sdpa_mask(Q, A, VA, B2[None], scale), rtol=0, atol=1e-12)


def pin_row_constant_bias_changes_nothing(orc):
    """A bias that is constant along the softmax axis cancels (softmax is
    invariant to a per-row shift)."""
    rng = _rng(63)
    B, H, N, k, d, scale = 1, 2, 10, 4, 3, 0.8
    Q, K, V = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    A = rng.standard_normal((B, H, k, d))
    c1 = np.repeat(rng.standard_normal((H, k, 1)) * 5, N, axis=2)
    c2 = np.repeat(rng.standard_normal((H, N, 1)) * 5, k, axis=2)
    assert np.allclose(orc.aggregate(A, K, V, scale, c1), orc.aggregate(A, K, V, scale),
                       rtol=0, atol=1e-12)
    VA = orc.aggregate(A, K, V, scale)
    assert np.allclose(orc.broadcast(Q, A, VA, scale, c2), orc.broadcast(Q, A, VA, scale),
                       rtol=0, atol=1e-12)


def pin_bias_selects_one_key(orc):
    """A bias of 0 on one key and -1e4 elsewhere makes every agent's value
    that key's value row (closed form)."""
    rng = _rng(64)
    B, H, N, k, d = 1, 1, 8, 3, 4
    A, K, V = (rng.standard_normal(sh) for sh in ((B, H, k, d), (B, H, N, d), (B, H, N, d)))
    B1 = np.full((H, k, N), -1e4)
    pick = [5, 0, 7]
    for i, m in enumerate(pick):
        B1[0, i, m] = 0.0
    VA = orc.aggregate(A, K, V, 0.5, B1)
    assert np.allclose(VA[0, 0], V[0, 0, pick], rtol=0, atol=1e-12)


def _dwc_torch(V, h, w, weight, bias):
    B, H, N, d = V.shape
    x = _t(V).reshape(B, H, h, w, d).permute(0, 1, 4, 2, 3).reshape(B, H * d, h, w)
    y = F.conv2d(x, _t(weight).reshape(H * d, 1, 3, 3), _t(bias), padding=1, groups=H * d)
    return y.reshape(B, H, d, h, w).permute(0, 1, 3, 4, 2).reshape(B, H, N, d).numpy()


def pin_dwc_vs_conv2d(orc):
    """DWC equals torch's grouped conv2d (one group per channel, padding 1),
    on a non-square grid so that a row/column mix-up shows."""
    rng = _rng(65)
    B, H, h, w, d = 2, 2, 5, 7, 3
    V = rng.standard_normal((B, H, h * w, d))
    W = rng.standard_normal((H * d, 3, 3))
    b = rng.standard_normal(H * d)
    assert np.allclose(orc.dwc(V, h, w, W, b), _dwc_torch(V, h, w, W, b), rtol=0, atol=1e-12)


def pin_dwc_center_tap_is_identity(orc):
    rng = _rng(66)
    V = rng.standard_normal((1, 2, 12, 4))
    W = np.zeros((8, 3, 3))
    W[:, 1, 1] = 1.0
    assert np.array_equal(orc.dwc(V, 3, 4, W), V)


def pin_dwc_explicit_loops(orc):
    """Per-element loops with explicit bounds checks on a tiny grid."""
    rng = _rng(67)
    B, H, h, w, d = 1, 2, 3, 4, 2
    V = rng.standard_normal((B, H, h * w, d))
    W = rng.standard_normal((H * d, 3, 3))
    b = rng.standard_normal(H * d)
    got = orc.dwc(V, h, w, W, b)
    for hd in range(H):
        for r in range(h):
            for c in range(w):
                for ch in range(d):
                    acc = b[hd * d + ch]
                    for dy in (-1, 0, 1):
                        for dx in (-1, 0, 1):
                            rr, cc = r + dy, c + dx
                            if 0 <= rr < h and 0 <= cc < w:
                                acc += W[hd * d + ch, dy + 1, dx + 1] * V[0, hd, rr * w + cc, ch]
                    assert abs(got[0, hd, r * w + c, ch] - acc) < 1e-12


def pin_forward_module_is_library_composition(orc):
    """Pooling, two masked attentions and conv2d, composed from library
    routines, equal the oracle's forward with every module term."""
    rng = _rng(68)
    B, H, h, w, d, s, scale = 2, 2, 6, 5, 4, 2, 0.5
    N, k = h * w, s * s
    Q, K, V = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    B1 = rng.standard_normal((H, k, N))
    B2 = rng.standard_normal((H, N, k))
    W = rng.standard_normal((H * d, 3, 3))
    b = rng.standard_normal(H * d)
    O, A, _ = orc.forward(Q, K, V, h, w, s, scale, bias_agg=B1, bias_bcast=B2, dwc_weight=W,
                          dwc_bias=b)
    A_ref = _torch_pool(Q, h, w, s)
    VA = _sdpa_mask(A_ref, K, V, B1[None], scale)
    ref = _sdpa_mask(Q, A_ref, VA, B2[None], scale) + _dwc_torch(V, h, w, W, b)
    assert np.allclose(O, ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ backward

def _torch_forward(Q, K, V, h, w, s, scale, A=None):
    """The forward composed of torch library routines (for autograd)."""
    B, H, N, d = Q.shape
    if A is None:
        x = Q.reshape(B * H, h, w, d).permute(0, 3, 1, 2)
        A = F.adaptive_avg_pool2d(x, (s, s)).permute(0, 2, 3, 1).reshape(B, H, s * s, d)
    VA = F.scaled_dot_product_attention(A, K, V, scale=scale)
    return F.scaled_dot_product_attention(Q, A, VA, scale=scale)


def pin_backward_vs_torch_autograd(orc):
    """Gradients equal torch's float64 autograd through adaptive pooling and
    two scaled_dot_product_attention calls, on a ragged grid (windows share
    a row) and with supplied agents."""
    rng = _rng(71)
    B, H, h, w, d, s, scale = 2, 2, 5, 7, 3, 2, 0.7
    N = h * w
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    for A in (None, rng.standard_normal((B, H, s * s, d))):
        dQ, dK, dV, dA = orc.backward(Q, K, V, dO, h, w, s, scale, A=A)
        tq, tk, tv = (_t(x).requires_grad_(True) for x in (Q, K, V))
        ta = None if A is None else _t(A).requires_grad_(True)
        _torch_forward(tq, tk, tv, h, w, s, scale, ta).backward(_t(dO))
        for got, ref in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
            assert np.allclose(got, ref.numpy(), rtol=0, atol=1e-12)
        if A is None:
            assert dA is None
        else:
            assert np.allclose(dA, ta.grad.numpy(), rtol=0, atol=1e-12)


def pin_backward_finite_differences(orc):
    """Central differences of the loss sum(dO * O) along single coordinates
    of Q, K, V and supplied A, on a tiny ragged case."""
    rng = _rng(72)
    B, H, h, w, d, s, scale, eps = 1, 1, 3, 4, 2, 2, 0.8, 1e-6
    N = h * w
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    A0 = rng.standard_normal((B, H, s * s, d))
    for A in (None, A0):
        grads = orc.backward(Q, K, V, dO, h, w, s, scale, A=A)
        names = ("Q", "K", "V") + (("A",) if A is not None else ())
        for gi, name in enumerate(names):
            for _ in range(4):
                base = {"Q": Q, "K": K, "V": V, "A": A}
                idx = tuple(int(rng.integers(0, n)) for n in base[name].shape)
                vals = []
                for sign in (1, -1):
                    pert = {k_: (None if v_ is None else v_.copy()) for k_, v_ in base.items()}
                    pert[name][idx] += sign * eps
                    O, _, _ = orc.forward(pert["Q"], pert["K"], pert["V"], h, w, s, scale,
                                          A=pert["A"])
                    vals.append(float((dO * O).sum()))
                fd = (vals[0] - vals[1]) / (2 * eps)
                assert abs(fd - grads[gi][idx]) < 1e-7, (name, idx, fd, grads[gi][idx])


def pin_backward_sums(orc):
    """Closed forms of sums over the tokens: the key gradients sum to zero
    (the output is invariant to translating every key, as each softmax row
    is to a constant shift) and the value gradients sum to the sum of dO
    (O is a row-stochastic mixing of the values)."""
    rng = _rng(73)
    B, H, h, w, d, s = 2, 3, 6, 6, 4, 3
    Q, K, V, dO = (rng.standard_normal((B, H, h * w, d)) for _ in range(4))
    _, dK, dV, _ = orc.backward(Q, K, V, dO, h, w, s, 0.6)
    assert np.allclose(dK.sum(axis=2), 0.0, rtol=0, atol=1e-12)
    assert np.allclose(dV.sum(axis=2), dO.sum(axis=2), rtol=0, atol=1e-12)


def pin_pool_backward_is_adjoint(orc):
    """<pool(Q), G> = <Q, pool_backward(G)> for random Q and G (the
    pooling's gradient is its adjoint), ragged and divisible grids."""
    rng = _rng(74)
    for (h, w, s) in ((7, 5, 3), (8, 8, 4), (2, 9, 2)):
        Q = rng.standard_normal((1, 2, h * w, 3))
        G = rng.standard_normal((1, 2, s * s, 3))
        lhs = float((orc.pool_agents(Q, h, w, s) * G).sum())
        rhs = float((Q * orc.pool_agents_backward(G, h, w, s)).sum())
        assert abs(lhs - rhs) < 1e-12


# ------------------------------------------------------------- full module

def _torch_round(x, fmt):
    """Rounding through torch's own dtype conversions (RNE)."""
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[fmt]
    return x.to(dt).to(torch.float64)


def _torch_module(X, Wqkv, bqkv, Wout, bout, H, h, w, s, scale, fmt, B1=None, B2=None, Wd=None,
                  bd=None):
    """The module from torch routines: F.linear, dtype casts, adaptive
    pooling, two scaled_dot_product_attention calls (with the biases as
    additive masks) and conv2d."""
    Xt = _t(X)
    B, N, C = X.shape
    d = C // H
    qkv = _torch_round(F.linear(Xt, _t(Wqkv), None if bqkv is None else _t(bqkv)), fmt)
    q, k, v = (qkv[..., i * C:(i + 1) * C].reshape(B, N, H, d).permute(0, 2, 1, 3)
               for i in range(3))
    x = q.reshape(B * H, h, w, d).permute(0, 3, 1, 2)
    A = F.adaptive_avg_pool2d(x, (s, s)).permute(0, 2, 3, 1).reshape(B, H, s * s, d)
    m1 = None if B1 is None else _t(B1)[None]
    m2 = None if B2 is None else _t(B2)[None]
    VA = F.scaled_dot_product_attention(A, k, v, attn_mask=m1, scale=scale)
    O = F.scaled_dot_product_attention(q, A, VA, attn_mask=m2, scale=scale)
    if Wd is not None:
        O = O + _t(_dwc_torch(v.numpy(), h, w, Wd, bd))
    o = O.permute(0, 2, 1, 3).reshape(B, N, C)
    if Wout is None:
        return o.numpy()
    return F.linear(_torch_round(o, fmt), _t(Wout), None if bout is None else _t(bout)).numpy()


def pin_round_to_format(orc):
    """Rounding to bf16 / f16 / f32 equals torch's dtype conversions, and
    hand cases of round-to-nearest-even: 1 + 2^-8 (a tie) goes to 1, 1 +
    3 * 2^-8 to 1 + 2^-6 in bf16, 1 + 2^-11 (a tie) to 1 in f16."""
    rng = _rng(81)
    x = rng.standard_normal(4096) * np.exp(rng.uniform(-20, 20, 4096))
    for fmt in ("bf16", "f16", "f32"):
        ref = _torch_round(_t(np.clip(x, -6e4, 6e4) if fmt == "f16" else x), fmt).numpy()
        got = orc.round_to_format(np.clip(x, -6e4, 6e4) if fmt == "f16" else x, fmt)
        assert np.array_equal(got, ref), fmt
    assert orc.round_to_format(np.array([1 + 2.0 ** -8]), "bf16")[0] == 1.0
    assert orc.round_to_format(np.array([1 + 3 * 2.0 ** -8]), "bf16")[0] == 1 + 2.0 ** -6
    assert orc.round_to_format(np.array([1 + 2.0 ** -11]), "f16")[0] == 1.0


def pin_module_is_library_composition(orc):
    """The module (projections, heads, pooling, two attentions with both
    biases, DWC, output projection) equals its composition from torch
    routines, in bf16 and f32 formats, with and without the output Linear."""
    rng = _rng(82)
    B, H, h, w, s, d = 2, 3, 5, 6, 2, 4
    N, C, k = h * w, H * d, s * s
    X = rng.standard_normal((B, N, C))
    Wqkv = rng.standard_normal((3 * C, C)) / math.sqrt(C)
    bqkv = rng.standard_normal(3 * C) * 0.3
    Wout = rng.standard_normal((C, C)) / math.sqrt(C)
    bout = rng.standard_normal(C) * 0.3
    B1, B2 = rng.standard_normal((H, k, N)), rng.standard_normal((H, N, k))
    Wd, bd = rng.standard_normal((C, 3, 3)) / 3, rng.standard_normal(C) * 0.5
    for fmt in ("bf16", "f32"):
        for wo, bo in ((Wout, bout), (None, None)):
            got = orc.module_forward(X, Wqkv, bqkv, wo, bo, H, h, w, s, 0.5, fmt, bias_agg=B1,
                                     bias_bcast=B2, dwc_weight=Wd, dwc_bias=bd)
            ref = _torch_module(X, Wqkv, bqkv, wo, bo, H, h, w, s, 0.5, fmt, B1, B2, Wd, bd)
            assert np.allclose(got, ref, rtol=0, atol=1e-12), fmt


def pin_module_constant_values(orc):
    """Value projection zero with bias c: every value row is c, so every
    output row is round(c) W_out^T + b_out whatever the queries and keys."""
    rng = _rng(83)
    B, H, h, w, s, d = 2, 2, 4, 4, 2, 4
    N, C = h * w, H * d
    X = rng.standard_normal((B, N, C))
    Wqkv = rng.standard_normal((3 * C, C))
    Wqkv[2 * C:] = 0.0
    bqkv = np.zeros(3 * C)
    c = rng.standard_normal(C)
    bqkv[2 * C:] = c
    Wout, bout = rng.standard_normal((C, C)), rng.standard_normal(C)
    got = orc.module_forward(X, Wqkv, bqkv, Wout, bout, H, h, w, s, 0.7, "bf16")
    cb = orc.round_to_format(c, "bf16")
    ref = orc.round_to_format(cb, "bf16") @ Wout.T + bout
    assert np.allclose(got, np.broadcast_to(ref, got.shape), rtol=0, atol=1e-12)


def pin_module_uniform_scores(orc):
    """Query and key projections zero: every score is 0, both softmaxes are
    uniform, and every output row is the token mean of the values (per head,
    concatenated), y = mean(v) W_out^T + b_out."""
    rng = _rng(84)
    B, H, h, w, s, d = 1, 2, 3, 5, 2, 4
    N, C = h * w, H * d
    X = rng.standard_normal((B, N, C))
    Wqkv = rng.standard_normal((3 * C, C))
    Wqkv[:2 * C] = 0.0
    Wout, bout = rng.standard_normal((C, C)), rng.standard_normal(C)
    got = orc.module_forward(X, Wqkv, None, Wout, bout, H, h, w, s, 0.9, "f32")
    v = _torch_round(_t(X @ Wqkv[2 * C:].T), "f32").numpy()
    ref = _torch_round(_t(v.mean(axis=1)), "f32").numpy() @ Wout.T + bout
    assert np.allclose(got, np.broadcast_to(ref[:, None, :], got.shape), rtol=0, atol=1e-12)


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
