"""Helpers for the GPU parity tests (host <-> device copies, comparisons)."""
from __future__ import annotations

import numpy as np

DEV = "cuda:0"


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:                      # bf16 bit patterns
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def empty_f32(*shape):
    import torch
    return torch.empty(*shape, dtype=torch.float32, device=DEV)


def nan_f32(*shape):
    import torch
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)


def upper_rel_fro(gpu, ref) -> float:
    iu = np.triu_indices(ref.shape[0])
    g = np.asarray(gpu, dtype=np.float64)[iu]
    r = np.asarray(ref, dtype=np.float64)[iu]
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))


def rel_fro(gpu, ref) -> float:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))


def say(*args):
    print("[gpu]", *args, flush=True)
