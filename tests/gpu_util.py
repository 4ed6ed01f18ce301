"""Host <-> device helpers for the GPU tests (no attention arithmetic)."""
from __future__ import annotations

import numpy as np
import torch

from efficient_attention_vision_amd import inputs


def to_device(op: inputs.Operand | None, device="cuda"):
    if op is None:
        return None
    if op.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(op.storage)).to(device)
    return torch.from_numpy(np.ascontiguousarray(op.storage).view(np.int16)).view(
        torch.float16 if op.dtype == "f16" else torch.bfloat16).to(device)


def f64_to_device(x: np.ndarray, device="cuda"):
    """float64 host array -> float32 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return inputs.f32_from_bf16_bits(bits).astype(np.float64)
    if t.dtype == torch.float16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return inputs.f32_from_f16_bits(bits).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)
