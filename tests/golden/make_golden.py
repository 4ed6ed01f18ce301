"""Write the oracle regression fixtures in this folder.

Calls only the oracle and the seeded input generators:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from efficient_attention_vision_amd import inputs  # noqa: E402

FIXTURES = {
    # a 6 x 10 grid pooled to 3 x 3 agents (non-square grid, windows of 2 x 4
    # and 2 x 3/4 columns with one shared column), float32 I/O
    "tiny_small_fixture": dict(workload=dict(B=1, H=2, h=6, w=10, d=8, s=3, dtype="f32",
                                             sigma=1.0),
                               seed=7, kind="iid"),
    # caller-supplied agents, bf16 I/O, discriminating inputs
    "supplied_agents_fixture": dict(workload=dict(B=1, H=1, h=8, w=8, d=8, s=2,
                                                  dtype="bf16", sigma=1.0,
                                                  supplied_agents=True),
                                    seed=3, kind="discriminating"),
}


def main():
    for name, spec in FIXTURES.items():
        wl = inputs.custom(name, **spec["workload"])
        inp = inputs.make_inputs(wl, spec["seed"], spec["kind"])
        O, A, VA = oracle.forward(inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w,
                                  wl.s, wl.scale,
                                  A=None if inp.A is None else inp.A.exact)
        out = dict(spec, O=O.tolist(), A=A.tolist(), V_A=VA.tolist(),
                   note="written by tests/golden/make_golden.py from the float64 oracle")
        with open(os.path.join(HERE, name + ".json"), "w") as f:
            json.dump(out, f)
        print("wrote", name)


if __name__ == "__main__":
    main()
