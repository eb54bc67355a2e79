"""Shared helpers of the GPU parity tests: moving seeded inputs to the device and the
per-head error metric against the fp64 oracle."""
from __future__ import annotations

import numpy as np

NAMES = "q k v a g e w r".split()


def to_device(inp: dict, device, qkv: str):
    """numpy inputs -> torch tensors on ``device`` (q/k/v in the workload's dtype)."""
    import torch
    qdt = torch.bfloat16 if qkv == "bf16" else torch.float32
    out = {}
    for n in NAMES:
        t = torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.float32))
        out[n] = t.to(device=device, dtype=qdt if n in ("q", "k", "v") else torch.float32)
    return out


def o_err(o, o_ref):
    """[B,H] per-head max relative error of outputs shaped [B,T,H,d]."""
    o = np.asarray(o, dtype=np.float64)
    r = np.asarray(o_ref, dtype=np.float64)
    diff = np.abs(o - r).max(axis=(1, 3))
    scale = np.abs(r).max(axis=(1, 3))
    err = diff / np.maximum(scale, 1e-300)
    err[~np.isfinite(o).all(axis=(1, 3))] = np.inf
    return err


def s_err(s, s_ref):
    """[B,H] per-head max relative error of states shaped [B,H,dk,dv]."""
    s = np.asarray(s, dtype=np.float64)
    r = np.asarray(s_ref, dtype=np.float64)
    diff = np.abs(s - r).max(axis=(2, 3))
    scale = np.abs(r).max(axis=(2, 3))
    err = diff / np.maximum(scale, 1e-300)
    err[~np.isfinite(s).all(axis=(2, 3))] = np.inf
    return err


def to_numpy(t):
    return t.float().cpu().numpy()
