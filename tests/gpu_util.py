"""Helpers for the GPU parity tests: upload seeded numpy inputs, compare results."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def dev(a, dtype=torch.float32):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.float64:
        t = t.to(torch.float32)
    return t.to(dtype).to(DEV)


def host(t):
    if t.dtype == torch.bfloat16:
        t = t.to(torch.float32)
    return t.detach().cpu().numpy()


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def bf16_np(a):
    """float64/float32 -> bf16 (nearest even) values as float64, via torch."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float32)))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()
