"""Helpers for the GPU tests: device copies of numpy arrays and case labels
printed (and flushed) before every GPU step, so that a failing run names its
case."""
from __future__ import annotations

import sys

import numpy as np


def case(msg: str) -> None:
    sys.stdout.write(f"[gpu case] {msg}\n")
    sys.stdout.flush()


def dev(a: np.ndarray, bf16: bool = False):
    import torch
    if bf16:
        assert a.dtype == np.uint16
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def scalar_dev(v: float):
    import torch
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))
