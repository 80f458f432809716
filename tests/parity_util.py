"""Helpers for GPU-vs-oracle parity tests (test infrastructure only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

# Tolerances stated for the operator: rel-L2 <= 2e-2 for bf16 inputs with fp32
# accumulation, <= 1e-4 for fp32 inputs.
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        return float("inf")
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return float(num)
    return float(num / den)


def to_np(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def head_subset(x, heads, state=False):
    """Select (b, h) pairs from [B,T,H,D] (or [B,H,K,V] when state=True) as a [n,T,1,D] array."""
    if x is None:
        return None
    if state:
        return np.stack([x[b, h] for b, h in heads])[:, None]
    return np.stack([x[b, :, h, :] for b, h in heads])[:, :, None, :]


def oracle_fwd_heads(inp, heads):
    """Oracle forward on selected heads of CPU tensors (upcast exactly to fp64)."""
    q, k, v, g = (to_np(inp[n]) for n in ("q", "k", "v", "g"))
    s0 = to_np(inp.get("s0"))
    sel = lambda a: head_subset(a, heads)
    o, sf = oracle.gla_fwd(sel(q), sel(k), sel(v), sel(g), head_subset(s0, heads, state=True))
    return o[:, :, 0, :], sf[:, 0]


def gpu_heads(x, heads, state=False):
    x = to_np(x)
    if state:
        return np.stack([x[b, h] for b, h in heads])
    return np.stack([x[b, :, h, :] for b, h in heads])
