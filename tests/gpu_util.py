"""Helpers of the GPU tests: host <-> device copies of oracle-typed arrays."""
from __future__ import annotations

import numpy as np
import torch


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def from_dev(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def device_inputs(inp: dict) -> dict:
    return {k: to_dev(v) for k, v in inp.items()}
