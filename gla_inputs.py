"""Seeded synthetic workloads for the GLA operator.

This module only draws random inputs; it contains none of the operator's
arithmetic.  Both the oracle-side tests and the GPU-side tests / benchmark use
it, so the two sides see identical inputs.

Inputs are drawn on the CPU in float32 with a ``torch.Generator`` seeded per
workload, in a fixed order (q, k, v, then the gate's own draws, then S0, then
do), and cast to the workload's dtype.  The oracle reads the *cast* values.

Gate recipes (all give log gates g <= 0, i.e. alpha = exp(g) in (0, 1]):
  * ``iid``     g = logsigmoid(N(0,1)) / 16 per (t, i) element
  * ``zero``    g = 0 (ungated linear attention)
  * ``lowrank`` g = logsigmoid(x W) / 16 with x ~ N(0,1) in R^{B x T x 16} and
                W ~ N(0,1)/4 in R^{16 x (H K)}: the rank-16 gate projection with
                temperature 16 of the GLA layer, so log gates sit near 0 with a
                heavy negative tail.
  * ``scalar``  one log gate per token and head, g = logsigmoid(N(0,1)) / 16, of
                shape [B, T, H] (the scalar-gate entry points)
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import torch
import torch.nn.functional as F


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    K: int
    V: int
    dtype: str            # "fp32" or "bf16"
    gate: str             # "iid" | "zero" | "lowrank"
    v_scale: str          # "rsqrt_k" or "unit"
    s0: str               # "none" | "zeros" | "normal0.1"
    backward: bool
    seed: int
    doc: str = ""

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 256, 64, 64, "fp32", "iid", "rsqrt_k", "none", False, 1,
                          "tiny GLA forward in fp32, chunk 64"),
    "ungated_1k": Workload("ungated_1k", 4, 8, 1024, 64, 64, "bf16", "zero", "unit", "none", False, 2,
                           "ungated causal linear attention at length 1K"),
    "gla_340m": Workload("gla_340m", 8, 4, 2048, 128, 256, "bf16", "lowrank", "rsqrt_k", "none", False, 3,
                         "GLA layer at the 340M-model head shape"),
    "gla_1p3b_long": Workload("gla_1p3b_long", 2, 4, 8192, 256, 512, "bf16", "lowrank", "rsqrt_k", "normal0.1",
                              False, 4, "GLA layer at the 1.3B-model head shape, length 8K, nonzero S0"),
    "fwdbwd_16k": Workload("fwdbwd_16k", 4, 16, 16384, 128, 128, "bf16", "iid", "rsqrt_k", "zeros", True, 5,
                           "forward + backward at length 16K, 16 heads"),
    "metric_8k": Workload("metric_8k", 2, 4, 8192, 128, 256, "bf16", "lowrank", "rsqrt_k", "none", True, 6,
                          "throughput shape: length 8K, dk 128, dv 256, forward + backward"),
}


def custom(B, H, T, K, V, dtype="bf16", gate="iid", v_scale="rsqrt_k", s0="none", backward=True, seed=0):
    """A workload with the same recipes at any shape (parity-test sizes)."""
    return Workload("custom", B, H, T, K, V, dtype, gate, v_scale, s0, backward, seed)


def make_inputs(w: Workload, device: Optional[str] = None, dht: bool = False) -> Dict[str, torch.Tensor]:
    """Draw the inputs of workload ``w`` (CPU, then moved to ``device`` if given).

    Returns q, k, g [B,T,H,K] (g [B,T,H] for the ``scalar`` gate) and v (+ do)
    [B,T,H,V] in the workload dtype, and s0 / dht [B,H,K,V] in float32 (or None).
    """
    gen = torch.Generator(device="cpu").manual_seed(w.seed)
    B, H, T, K, V = w.B, w.H, w.T, w.K, w.V
    rk = 1.0 / (K ** 0.5)
    q = torch.randn(B, T, H, K, generator=gen) * rk
    k = torch.randn(B, T, H, K, generator=gen) * rk
    v = torch.randn(B, T, H, V, generator=gen)
    if w.v_scale == "rsqrt_k":
        v = v * rk
    if w.gate == "zero":
        g = torch.zeros(B, T, H, K)
    elif w.gate == "iid":
        g = F.logsigmoid(torch.randn(B, T, H, K, generator=gen)) / 16.0
    elif w.gate == "lowrank":
        x = torch.randn(B, T, 16, generator=gen)
        W = torch.randn(16, H * K, generator=gen) / 4.0
        g = (F.logsigmoid(x @ W) / 16.0).reshape(B, T, H, K)
    elif w.gate == "scalar":
        g = F.logsigmoid(torch.randn(B, T, H, generator=gen)) / 16.0
    else:
        raise ValueError(w.gate)
    if w.s0 == "none":
        s0 = None
    elif w.s0 == "zeros":
        s0 = torch.zeros(B, H, K, V)
    elif w.s0 == "normal0.1":
        s0 = torch.randn(B, H, K, V, generator=gen) * 0.1
    else:
        raise ValueError(w.s0)
    out = {}
    dt = w.torch_dtype
    out["q"], out["k"], out["v"], out["g"] = q.to(dt), k.to(dt), v.to(dt), g.to(dt)
    out["s0"] = s0
    if w.backward:
        out["do"] = torch.randn(B, T, H, V, generator=gen).to(dt)
    out["dht"] = (torch.randn(B, H, K, V, generator=gen) * 0.1) if dht else None
    if device is not None:
        out = {kk: (vv.to(device) if vv is not None else None) for kk, vv in out.items()}
    return out


def make_value_gate(B: int, T: int, H: int, V: int, dtype: str = "bf16", seed: int = 0,
                    kind: str = "lowrank") -> torch.Tensor:
    """The value-side log gate h = log beta [B,T,H,V] of general gated linear
    attention, drawn like the key-side gate: ``lowrank`` logsigmoid(x W) / 16
    with x ~ N(0,1) in R^{B x T x 16} and W ~ N(0,1)/4 in R^{16 x H*V}; ``iid``
    logsigmoid(N(0,1)) / 16; ``zero`` all zeros (beta = 1)."""
    gen = torch.Generator().manual_seed(seed)
    if kind == "lowrank":
        x = torch.randn(B, T, 16, generator=gen)
        W = torch.randn(16, H * V, generator=gen) / 4.0
        h = (F.logsigmoid(x @ W) / 16.0).reshape(B, T, H, V)
    elif kind == "iid":
        h = F.logsigmoid(torch.randn(B, T, H, V, generator=gen)) / 16.0
    elif kind == "zero":
        h = torch.zeros(B, T, H, V)
    else:
        raise ValueError(kind)
    return h.to(torch.float32 if dtype == "fp32" else torch.bfloat16)


def make_gate_inputs(B: int, T: int, H: int, V: int, dtype: str = "bf16", seed: int = 0, bias: bool = True,
                     device: Optional[str] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Inputs of the GLA layer's output epilogue (per-head LayerNorm, Swish gate).

    Drawn in float32 on the CPU in the order o, z, ln_w, ln_b, dy:
      o  ~ N(0,1) / sqrt(V)   [B,T,H,V]  (the scale of an attention output row)
      z  ~ N(0,1)             [B,T,H,V]  (the gate's pre-activation x W_r + b_r)
      ln_w ~ 1 + N(0,1)/10, ln_b ~ N(0,1)/10   [V] float32 (never cast)
      dy ~ N(0,1)             [B,T,H,V]
    o, z and dy are cast to ``dtype``; ln_b is None when ``bias`` is false."""
    gen = torch.Generator().manual_seed(seed)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    o = (torch.randn(B, T, H, V, generator=gen) / V ** 0.5).to(dt)
    z = torch.randn(B, T, H, V, generator=gen).to(dt)
    w = 1.0 + torch.randn(V, generator=gen) / 10
    b = torch.randn(V, generator=gen) / 10
    dy = torch.randn(B, T, H, V, generator=gen).to(dt)
    out = {"o": o, "z": z, "ln_w": w, "ln_b": b if bias else None, "dy": dy}
    if device is not None:
        out = {k: (v.to(device) if v is not None else None) for k, v in out.items()}
    return out
