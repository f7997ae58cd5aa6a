"""Helpers for GPU parity tests: move seeded host inputs to the device and back."""
from __future__ import annotations

import sys

import numpy as np
import torch


def say(*a):
    """Name the case before a GPU step, flushed, so a failing step is identifiable."""
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def f32_dev(v) -> torch.Tensor:
    return torch.tensor(np.asarray(v, dtype=np.float32).reshape(-1), device="cuda")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)
