"""GPU-side helpers for the parity tests: numpy -> device tensors."""

from __future__ import annotations

import sys

import numpy as np
import torch


def announce(*parts):
    """Name the case on stdout before any GPU work (so a crash is attributable)."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def dev(a, device="cuda"):
    """numpy -> contiguous device tensor (uint32 travels as int32 bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.float16)
    return torch.from_numpy(a.copy()).to(device)


def dev_tree(d: dict | None, device="cuda"):
    if d is None:
        return None
    return {k: (dev(v, device) if isinstance(v, np.ndarray) else v) for k, v in d.items()}


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def f16_to_f64(t) -> np.ndarray:
    return host(t).astype(np.float64)
