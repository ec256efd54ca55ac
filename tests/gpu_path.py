"""Helpers for GPU parity tests: move seeded numpy inputs to the device, run the HIP
path through the Python binding of the C ABI, bring results back as numpy."""
from __future__ import annotations

import sys

import numpy as np
import torch

FMT = {"e4m3": 0, "e5m2": 1}


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a fault still shows what ran)."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev_src(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    if x.dtype == np.float32:
        return torch.from_numpy(x).cuda()
    raise TypeError(x.dtype)


def f32(v) -> torch.Tensor:
    return torch.tensor(np.asarray(v, np.float32).reshape(-1)).cuda()


def quantize(x: np.ndarray, fmt: int, scale: float, amax_in: float = 0.0):
    import delayed_scaling_amax_amd as d
    src = dev_src(x)
    dst = torch.empty(src.numel(), dtype=torch.uint8, device="cuda")
    s, a = f32([scale]), f32([amax_in])
    d.fp8_quantize_amax(src, dst, s, a, fmt)
    torch.cuda.synchronize()
    return dst.cpu().numpy().reshape(x.shape), a.cpu().numpy()[0]


def bits(a) -> np.ndarray:
    return np.asarray(a, np.float32).view(np.uint32)
