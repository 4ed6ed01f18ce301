"""The oracle against its pins (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import agent_oracle
from tests import oracle_pins
from efficient_attention_vision_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(agent_oracle)


def test_softmax_rows_sum_to_one_and_match_scipy():
    from scipy.special import softmax
    S = np.random.Generator(np.random.PCG64(5)).standard_normal((3, 4, 17)) * 7
    P = oracle.softmax_last(S)
    assert np.allclose(P, softmax(S, axis=-1), rtol=0, atol=1e-15)
    assert np.allclose(P.sum(-1), 1.0, rtol=0, atol=1e-14)


def test_window_bounds_tile_the_grid():
    for n in range(1, 30):
        for s in range(1, n + 1):
            b = [oracle.window_bounds(i, n, s) for i in range(s)]
            assert b[0][0] == 0 and b[-1][1] == n
            for (a0, a1), (b0, b1) in zip(b, b[1:]):
                assert a0 < a1 and b0 <= a1 and b0 >= a0   # ordered, overlapping by <= 1
            if n % s == 0:
                assert all(r1 - r0 == n // s for r0, r1 in b)


@pytest.mark.parametrize("name", ["tiny_small_fixture", "supplied_agents_fixture"])
def test_golden_fixture(name):
    """Regression fixture written by tests/golden/make_golden.py (oracle only)."""
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        g = json.load(f)
    wl = inputs.custom(name, **g["workload"])
    inp = inputs.make_inputs(wl, g["seed"], g["kind"])
    O, A, VA = oracle.forward(inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w,
                              wl.s, wl.scale, A=None if inp.A is None else inp.A.exact)
    assert np.allclose(O, np.array(g["O"]), rtol=0, atol=1e-14)
    assert np.allclose(A, np.array(g["A"]), rtol=0, atol=1e-14)
    assert np.allclose(VA, np.array(g["V_A"]), rtol=0, atol=1e-14)
