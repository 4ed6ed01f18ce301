"""The parity criterion used by every GPU-vs-oracle comparison.

Two bounds must both hold against the unrounded float64 oracle:
  * max |out - ref| <= ATOL  (1e-5 for float32 I/O, 2e-2 for bfloat16 I/O
    with float32 accumulation);
  * max |out - ref| / max |ref| <= RTOL  (1e-4 for float32, 1e-2 for bf16).
The relative bound exists because at the workloads' own distributions
max |O| is only a few times the absolute bf16 tolerance, so an output of all
zeros would nearly pass the absolute bound alone.  On the discriminating
inputs (|O| up to about 3.5) the absolute bound is scaled by max(1, max|ref|),
since bf16 output rounding alone is relative.  The bf16 budget follows
from about four roundings of relative size 2^-9 on the path (agents, the two
probability matrices as MFMA operands, and O itself), i.e. under 1 %.
float16 I/O rounds the same four quantities with relative size 2^-11, and
from 128 agents the partial aggregation sums are exchanged as bfloat16
(2^-9 on V_A); emulating all of these in float64 on the five workloads
gives at most 3.6e-3 relative, hence 1e-2 / 5e-3 for f16.
"""
from __future__ import annotations

import numpy as np

ATOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 1e-2}
RTOL = {"f32": 1e-4, "bf16": 1e-2, "f16": 5e-3}


def errors(out: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    if out.size == 0:
        return 0.0, 0.0
    diff = np.abs(out - ref)
    if not np.all(np.isfinite(out)):
        return float("inf"), float("inf")
    mx = float(diff.max())
    scale = float(np.abs(ref).max())
    return mx, (mx / scale if scale > 0 else (0.0 if mx == 0 else float("inf")))


def atol(ref, dtype: str, kind: str = "iid") -> float:
    if kind == "discriminating":
        return ATOL[dtype] * max(1.0, float(np.abs(np.asarray(ref)).max(initial=0.0)))
    return ATOL[dtype]


def close(out, ref, dtype: str, kind: str = "iid") -> bool:
    a, r = errors(out, ref)
    return a <= atol(ref, dtype, kind) and r <= RTOL[dtype]


def assert_close(out, ref, dtype: str, what: str = "", kind: str = "iid") -> None:
    a, r = errors(out, ref)
    at = atol(ref, dtype, kind)
    assert a <= at and r <= RTOL[dtype], (
        f"{what}: max-abs {a:.3e} (tol {at:.1e}), "
        f"relative {r:.3e} (tol {RTOL[dtype]:.0e})")
