"""Planted mistakes in the oracle must be caught (CPU only).

Each mutant replaces one function of the oracle module with a plausible wrong
version (a dropped term, a wrong sign, axis or index, a transposed operand);
at least one pin must then fail.  A second group shows that the parity
criterion used against the GPU rejects wrong outputs at the workloads' shapes
on the discriminating inputs, while it accepts the rounding that a correct
bf16 kernel performs.
"""
import numpy as np
import pytest

from oracle import agent_oracle as orc
from tests import oracle_pins, parity
from efficient_attention_vision_amd import inputs


def _pool_column_major(Q, h, w, s):
    B, H, N, d = Q.shape
    grid = Q.reshape(B, H, w, h, d).swapaxes(2, 3)      # token n read as c*h + r
    A = np.empty((B, H, s * s, d))
    for i in range(s):
        r0, r1 = orc.window_bounds(i, h, s)
        for j in range(s):
            c0, c1 = orc.window_bounds(j, w, s)
            A[:, :, i * s + j] = grid[:, :, r0:r1, c0:c1].mean(axis=(2, 3))
    return A


def _window_floor(i, n, s):
    """window stop rounded down instead of up."""
    return (i * n) // s, max(((i + 1) * n) // s, (i * n) // s + 1)


def _pool_sum(Q, h, w, s):
    B, H, N, d = Q.shape
    grid = Q.reshape(B, H, h, w, d)
    A = np.empty((B, H, s * s, d))
    for i in range(s):
        r0, r1 = orc.window_bounds(i, h, s)
        for j in range(s):
            c0, c1 = orc.window_bounds(j, w, s)
            A[:, :, i * s + j] = grid[:, :, r0:r1, c0:c1].sum(axis=(2, 3))
    return A


def _agg_no_scale(A, K, V, scale, bias=None):
    return orc.softmax_last(A @ np.swapaxes(K, -1, -2)) @ V


def _agg_wrong_axis(A, K, V, scale, bias=None):
    S = scale * (A @ np.swapaxes(K, -1, -2))
    E = np.exp(S - S.max(axis=-2, keepdims=True))
    return (E / E.sum(axis=-2, keepdims=True)) @ V


def _agg_scale_twice(A, K, V, scale, bias=None):
    return orc.softmax_last(scale * scale * (A @ np.swapaxes(K, -1, -2))) @ V


def _bc_values_as_keys(Q, A, VA, scale, bias=None):
    """the garbled broadcast of one blog post: keys V_A, no scale."""
    return orc.softmax_last(Q @ np.swapaxes(VA, -1, -2)) @ VA


def _bc_wrong_axis(Q, A, VA, scale, bias=None):
    S = scale * (Q @ np.swapaxes(A, -1, -2))
    E = np.exp(S - S.max(axis=-2, keepdims=True))
    return (E / E.sum(axis=-2, keepdims=True)) @ VA


def _bc_no_scale(Q, A, VA, scale, bias=None):
    return orc.softmax_last(Q @ np.swapaxes(A, -1, -2)) @ VA


def _softmax_neg(S):
    E = np.exp(-S - (-S).max(axis=-1, keepdims=True))
    return E / E.sum(axis=-1, keepdims=True)


def _softmax_norm_by_max(S):
    E = np.exp(S - S.max(axis=-1, keepdims=True))
    return E / E.max(axis=-1, keepdims=True)


def _softmax_no_norm(S):
    return np.exp(S - S.max(axis=-1, keepdims=True))


def _forward_swap_kv(Q, K, V, h, w, s, scale, A=None, **module_terms):
    Q, K, V = (np.asarray(x, float) for x in (Q, K, V))
    A = orc.pool_agents(Q, h, w, s) if A is None else np.asarray(A, float)
    VA = orc.aggregate(A, V, K, scale)
    return orc.broadcast(Q, A, VA, scale), A, VA


def _forward_agents_as_values(Q, K, V, h, w, s, scale, A=None, **module_terms):
    Q, K, V = (np.asarray(x, float) for x in (Q, K, V))
    A = orc.pool_agents(Q, h, w, s) if A is None else np.asarray(A, float)
    VA = orc.aggregate(A, K, V, scale)
    return orc.broadcast(Q, A, A, scale), A, VA


def _forward_pool_keys(Q, K, V, h, w, s, scale, A=None, **module_terms):
    Q, K, V = (np.asarray(x, float) for x in (Q, K, V))
    A = orc.pool_agents(K, h, w, s) if A is None else np.asarray(A, float)
    VA = orc.aggregate(A, K, V, scale)
    return orc.broadcast(Q, A, VA, scale), A, VA


def _forward_skip_aggregation(Q, K, V, h, w, s, scale, A=None, **module_terms):
    """a dropped step: broadcast straight from pooled values."""
    Q, K, V = (np.asarray(x, float) for x in (Q, K, V))
    A = orc.pool_agents(Q, h, w, s) if A is None else np.asarray(A, float)
    VA = orc.pool_agents(V, h, w, s)
    return orc.broadcast(Q, A, VA, scale), A, VA


def _agg_bias_scaled(A, K, V, scale, bias=None):
    """bias inside the scaled product: scale * (A K^T + B1)."""
    S = A @ np.swapaxes(K, -1, -2)
    if bias is not None:
        S = S + np.asarray(bias)[None]
    return orc.softmax_last(scale * S) @ V


def _agg_bias_dropped(A, K, V, scale, bias=None):
    return orc.softmax_last(scale * (A @ np.swapaxes(K, -1, -2))) @ V


def _bc_bias_dropped(Q, A, VA, scale, bias=None):
    return orc.softmax_last(scale * (Q @ np.swapaxes(A, -1, -2))) @ VA


def _bc_bias_negated(Q, A, VA, scale, bias=None):
    S = scale * (Q @ np.swapaxes(A, -1, -2))
    if bias is not None:
        S = S - np.asarray(bias)[None]
    return orc.softmax_last(S) @ VA


def _dwc_flipped(V, h, w, weight, bias=None):
    """convolution with the kernel flipped (true convolution, not the
    cross-correlation deep-learning layers compute)."""
    return _orig_dwc(V, h, w, np.asarray(weight)[:, ::-1, ::-1], bias)


def _dwc_wraparound(V, h, w, weight, bias=None):
    """circular instead of zero padding."""
    V = np.asarray(V, float)
    B, H, N, d = V.shape
    W = np.asarray(weight, float).reshape(H, d, 3, 3)
    grid = V.reshape(B, H, h, w, d)
    out = np.zeros_like(grid)
    if bias is not None:
        out += np.asarray(bias, float).reshape(H, d)[None, :, None, None, :]
    for dy in (-1, 0, 1):
        for dx in (-1, 0, 1):
            shifted = np.roll(np.roll(grid, -dy, axis=2), -dx, axis=3)
            out += W[None, :, None, None, :, dy + 1, dx + 1] * shifted
    return out.reshape(B, H, N, d)


def _dwc_transposed_taps(V, h, w, weight, bias=None):
    """dy and dx exchanged in the kernel index."""
    return _orig_dwc(V, h, w, np.swapaxes(np.asarray(weight), 1, 2), bias)


def _dwc_no_bias(V, h, w, weight, bias=None):
    return _orig_dwc(V, h, w, weight, None)


def _forward_dwc_of_queries(Q, K, V, h, w, s, scale, A=None, bias_agg=None, bias_bcast=None,
                            dwc_weight=None, dwc_bias=None):
    O, A_, VA = _orig_forward(Q, K, V, h, w, s, scale, A=A, bias_agg=bias_agg,
                              bias_bcast=bias_bcast)
    if dwc_weight is not None:
        O = O + orc.dwc(Q, h, w, dwc_weight, dwc_bias)
    return O, A_, VA


def _forward_biases_swapped(Q, K, V, h, w, s, scale, A=None, bias_agg=None, bias_bcast=None,
                            dwc_weight=None, dwc_bias=None):
    """B1 and B2 used in the other attention (transposed to fit)."""
    sw = lambda b: None if b is None else np.swapaxes(np.asarray(b), -1, -2)  # noqa: E731
    return _orig_forward(Q, K, V, h, w, s, scale, A=A, bias_agg=sw(bias_bcast),
                         bias_bcast=sw(bias_agg), dwc_weight=dwc_weight, dwc_bias=dwc_bias)


def _softmax_bw_no_centering(P, dP):
    return P * dP


def _softmax_bw_transposed_sum(P, dP):
    return P * (dP - (P * dP).sum(axis=-2, keepdims=True))


def _pool_bw_sum(dA, h, w, s):
    """spread without dividing by the window size."""
    B, H, k, d = dA.shape
    g = np.zeros((B, H, h, w, d))
    for i in range(s):
        r0, r1 = orc.window_bounds(i, h, s)
        for j in range(s):
            c0, c1 = orc.window_bounds(j, w, s)
            g[:, :, r0:r1, c0:c1, :] += dA[:, :, i * s + j, None, None, :]
    return g.reshape(B, H, h * w, d)


def _backward_wrong_probs_for_dv(Q, K, V, dO, h, w, s, scale, A=None):
    """dV through the unnormalised aggregation weights exp(S1 - max)."""
    dQ, dK, dV, dA = _orig_backward(Q, K, V, dO, h, w, s, scale, A=A)
    Q, K = np.asarray(Q, float), np.asarray(K, float)
    A_ = orc.pool_agents(Q, h, w, s) if A is None else np.asarray(A, float)
    S1 = scale * (A_ @ np.swapaxes(K, -1, -2))
    E1 = np.exp(S1 - S1.max(axis=-1, keepdims=True))
    P2 = orc.softmax_last(scale * (Q @ np.swapaxes(A_, -1, -2)))
    dV_A = np.swapaxes(P2, -1, -2) @ np.asarray(dO, float)
    return dQ, dK, np.swapaxes(E1, -1, -2) @ dV_A, dA


def _backward_no_pool_term(Q, K, V, dO, h, w, s, scale, A=None):
    """pooled agents treated as constants (their gradient not sent to Q)."""
    dQ, dK, dV, dA = _orig_backward(Q, K, V, dO, h, w, s, scale, A=np.asarray(
        orc.pool_agents(np.asarray(Q, float), h, w, s)) if A is None else A)
    return dQ, dK, dV, (None if A is None else dA)


def _backward_dk_unscaled(Q, K, V, dO, h, w, s, scale, A=None):
    dQ, dK, dV, dA = _orig_backward(Q, K, V, dO, h, w, s, scale, A=A)
    return dQ, dK / scale, dV, dA


_orig_backward = orc.backward
_orig_dwc = orc.dwc
_orig_forward = orc.forward

# ------------------------------------------------------------- module mutants

_real_module_forward = orc.module_forward
_real_round = orc.round_to_format


def _module_variant(swap_qk=False, channel_major=False, drop_out_bias=False, no_round=False):
    real = _real_module_forward

    def f(X, W_qkv, b_qkv, W_out, b_out, H, h, w, s, scale, fmt, **kw):
        C = np.asarray(X).shape[-1]
        W = np.array(W_qkv, dtype=np.float64)
        b = None if b_qkv is None else np.array(b_qkv, dtype=np.float64)
        if swap_qk:
            W[:C], W[C:2 * C] = W[C:2 * C].copy(), W[:C].copy()
            if b is not None:
                b[:C], b[C:2 * C] = b[C:2 * C].copy(), b[:C].copy()
        if channel_major:   # heads read as [d, H] instead of [H, d]
            d = C // H
            perm = np.arange(C).reshape(d, H).T.reshape(-1)
            W = np.concatenate([W[i * C:(i + 1) * C][perm] for i in range(3)])
            if b is not None:
                b = np.concatenate([b[i * C:(i + 1) * C][perm] for i in range(3)])
            if W_out is not None:
                W_out = np.asarray(W_out)[:, perm]
        if no_round:
            fmt = "f32"
        return real(X, W, b, W_out, None if drop_out_bias else b_out, H, h, w, s, scale, fmt,
                    **kw)
    return f


def _round_truncate(x, fmt):
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if fmt == "bf16":
        return (x32.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    return _real_round(x, fmt)


MUTANTS = {
    "aggregate_bias_inside_scale": ("aggregate", _agg_bias_scaled),
    "aggregate_bias_dropped": ("aggregate", _agg_bias_dropped),
    "broadcast_bias_dropped": ("broadcast", _bc_bias_dropped),
    "broadcast_bias_negated": ("broadcast", _bc_bias_negated),
    "dwc_kernel_flipped": ("dwc", _dwc_flipped),
    "dwc_circular_padding": ("dwc", _dwc_wraparound),
    "dwc_taps_transposed": ("dwc", _dwc_transposed_taps),
    "dwc_bias_dropped": ("dwc", _dwc_no_bias),
    "forward_dwc_of_queries": ("forward", _forward_dwc_of_queries),
    "forward_biases_swapped": ("forward", _forward_biases_swapped),
    "softmax_backward_uncentred": ("softmax_backward", _softmax_bw_no_centering),
    "softmax_backward_column_sum": ("softmax_backward", _softmax_bw_transposed_sum),
    "pool_backward_not_averaged": ("pool_agents_backward", _pool_bw_sum),
    "backward_values_wrong": ("backward", _backward_wrong_probs_for_dv),
    "backward_agents_held_constant": ("backward", _backward_no_pool_term),
    "backward_key_gradient_unscaled": ("backward", _backward_dk_unscaled),
    "pool_column_major": ("pool_agents", _pool_column_major),
    "window_floor_stop": ("window_bounds", _window_floor),
    "pool_sum_not_mean": ("pool_agents", _pool_sum),
    "aggregate_no_scale": ("aggregate", _agg_no_scale),
    "aggregate_softmax_over_agents": ("aggregate", _agg_wrong_axis),
    "aggregate_scale_twice": ("aggregate", _agg_scale_twice),
    "broadcast_values_as_keys": ("broadcast", _bc_values_as_keys),
    "broadcast_softmax_over_tokens": ("broadcast", _bc_wrong_axis),
    "broadcast_no_scale": ("broadcast", _bc_no_scale),
    "softmax_negated": ("softmax_last", _softmax_neg),
    "softmax_divided_by_max": ("softmax_last", _softmax_norm_by_max),
    "softmax_unnormalised": ("softmax_last", _softmax_no_norm),
    "forward_swaps_keys_values": ("forward", _forward_swap_kv),
    "forward_agents_as_values": ("forward", _forward_agents_as_values),
    "forward_pools_keys": ("forward", _forward_pool_keys),
    "forward_skips_aggregation": ("forward", _forward_skip_aggregation),
    "module_swaps_queries_keys": ("module_forward", _module_variant(swap_qk=True)),
    "module_heads_channel_major": ("module_forward", _module_variant(channel_major=True)),
    "module_drops_output_bias": ("module_forward", _module_variant(drop_out_bias=True)),
    "module_skips_rounding": ("module_forward", _module_variant(no_round=True)),
    "round_truncates": ("round_to_format", _round_truncate),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError, ZeroDivisionError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"


# ----------------------------------------------- power of the parity criterion

def _bf16(x):
    return inputs.f32_from_bf16_bits(inputs.bf16_bits_from_f32(
        np.asarray(x, np.float32))).astype(np.float64)


def _emulated_bf16_kernel(Q, K, V, h, w, s, scale, A=None):
    """What a correct kernel is allowed to round: agents, both probability
    matrices and V_A as bf16 matrix-core operands, and O itself."""
    A = orc.pool_agents(Q, h, w, s) if A is None else A
    Ab = _bf16(A)
    P1 = orc.softmax_last(scale * (Ab @ np.swapaxes(K, -1, -2)))
    VA = _bf16(P1) @ V
    P2 = orc.softmax_last(scale * (Q @ np.swapaxes(Ab, -1, -2)))
    return _bf16(_bf16(P2) @ _bf16(VA))


@pytest.fixture(scope="module", params=["deit_s", "pvt_stage1", "sd_unet", "sd_unet_agents"])
def workload_case(request):
    wl = inputs.WORKLOADS[request.param]
    inp = inputs.make_inputs(wl, 0, "discriminating")
    args = (inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w, wl.s, wl.scale)
    A = None if inp.A is None else inp.A.exact
    O, _, _ = orc.forward(*args, A=A)
    return wl, args, A, O


def test_discriminating_inputs_have_order_one_outputs(workload_case):
    wl, args, A, O = workload_case
    assert np.abs(O).max() > 0.5


def test_correct_bf16_rounding_passes(workload_case):
    wl, args, A, O = workload_case
    parity.assert_close(_emulated_bf16_kernel(*args, A=A), O, "bf16", wl.name,
                        kind="discriminating")


WRONG_OUTPUTS = {
    "zeros": lambda args, A: np.zeros_like(args[0]),
    "no_scale": lambda args, A: orc.forward(*args[:-1], 1.0, A=A)[0],
    "values_as_broadcast_keys": lambda args, A: _bc_values_as_keys(
        args[0], None, orc.forward(*args, A=A)[2], args[-1]),
    "broadcast_softmax_over_tokens": lambda args, A: _bc_wrong_axis(
        args[0], *orc.forward(*args, A=A)[1:], args[-1]),
    # (column-major pooling is not listed: on the square grids of these
    # workloads it only renumbers the agents, which O cannot see; the pins
    # catch it on non-square grids)
    "agents_pooled_from_keys": lambda args, A: orc.broadcast(
        args[0], orc.pool_agents(args[1], *args[3:6]),
        orc.aggregate(orc.pool_agents(args[1], *args[3:6]), args[1], args[2], args[-1]),
        args[-1]) if A is None else None,
    "unnormalised_broadcast": lambda args, A: _softmax_no_norm(
        args[-1] * (args[0] @ np.swapaxes(orc.forward(*args, A=A)[1], -1, -2)))
        @ orc.forward(*args, A=A)[2],
}


@pytest.mark.parametrize("wrong", sorted(WRONG_OUTPUTS))
def test_criterion_rejects_wrong_outputs(workload_case, wrong):
    wl, args, A, O = workload_case
    out = WRONG_OUTPUTS[wrong](args, A)
    if out is None:
        pytest.skip("pooling is bypassed when agents are supplied")
    assert not parity.close(out, O, "bf16", kind="discriminating"), \
        f"{wrong} passes on {wl.name}"
