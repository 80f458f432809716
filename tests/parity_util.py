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


LOG2E = 1.4426950408889634


def max_chunk_decay_log2(g, chunk=64):
    """Largest decay of one chunk and key column, -sum_{t in chunk} g_t[i] in
    log2 units, over a [B,T,H,K] (or scalar [B,T,H]) log-gate tensor as stored.
    Returns the maximum over batch, chunks and key columns, per head index."""
    a = to_np(g)
    if a.ndim == 3:
        a = a[..., None]
    B, T, H, K = a.shape
    s = -a.reshape(B, T // chunk, chunk, H, K).sum(axis=2) * LOG2E   # [B, N, H, K]
    return s.max(axis=(0, 1, 3))                                      # [H]


def chunk_rel_l2(x, ref, chunk=64):
    """Largest rel-L2 over (head, 64-token chunk) blocks of [n, T, D] arrays.
    Blocks whose reference norm is zero are compared by their absolute norm."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        return float("inf")
    n, T, D = ref.shape
    xs = x.reshape(n, T // chunk, chunk * D)
    rs = ref.reshape(n, T // chunk, chunk * D)
    num = np.linalg.norm(xs - rs, axis=2)
    den = np.linalg.norm(rs, axis=2)
    r = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(r.max())
