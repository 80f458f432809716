"""GPU parity of the scalar-gate entry points (gla_fwd_scalar, gla_bwd_scalar:
one log gate per token and head) through the C ABI, against the fp64 oracle's
scalar-gate recurrence and its reverse-mode gradient."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_amd as gla
import gla_inputs as gi
import oracle
from tests.parity_util import TOL, note, rel_l2, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _sel(x, heads, state=False):
    if x is None:
        return None
    if state:
        return np.stack([x[b, h] for b, h in heads])[:, None]
    if x.ndim == 3:  # a scalar gate [B,T,H]
        return np.stack([x[b, :, h] for b, h in heads])[:, :, None]
    return np.stack([x[b, :, h, :] for b, h in heads])[:, :, None, :]


def _gpu(x, heads, state=False):
    x = to_np(x)
    if state:
        return np.stack([x[b, h] for b, h in heads])
    if x.ndim == 3:
        return np.stack([x[b, :, h] for b, h in heads])
    return np.stack([x[b, :, h, :] for b, h in heads])


def _inputs(B, H, T, K, V, s0, seed, gate_fn=None, dtype="bf16"):
    w = gi.custom(B, H, T, K, V, dtype=dtype, gate="scalar", s0=s0, backward=True, seed=seed)
    inp = gi.make_inputs(w, dht=True)
    if gate_fn is not None:
        inp["g"] = gate_fn(inp["g"])
    return w, inp


def _check(w, inp, heads=None, backward=True, with_dht=True):
    note("scalar-gate parity: B=%d H=%d T=%d K=%d V=%d s0=%s" % (w.B, w.H, w.T, w.K, w.V, w.s0))
    if heads is None:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    dht = d["dht"] if with_dht else None
    o, sf = gla.gla_fwd_scalar(d["q"], d["k"], d["v"], d["g"], d["s0"])
    torch.cuda.synchronize()
    c = {n: to_np(inp[n]) for n in ("q", "k", "v", "g", "do")}
    s0 = _sel(to_np(inp.get("s0")), heads, state=True)
    o_ref, sf_ref = oracle.gla_fwd_scalar(_sel(c["q"], heads), _sel(c["k"], heads), _sel(c["v"], heads),
                                          _sel(c["g"], heads), s0)
    errs = {"o": rel_l2(_gpu(o, heads), o_ref[:, :, 0, :]), "S_T": rel_l2(_gpu(sf, heads, True), sf_ref[:, 0])}
    if backward:
        dq, dk, dv, dg, ds0 = gla.gla_bwd_scalar(d["q"], d["k"], d["v"], d["g"], d["do"], d["s0"], dht)
        torch.cuda.synchronize()
        ref = oracle.gla_bwd_scalar(_sel(c["q"], heads), _sel(c["k"], heads), _sel(c["v"], heads),
                                    _sel(c["g"], heads), _sel(c["do"], heads), s0,
                                    _sel(to_np(inp["dht"]), heads, state=True) if with_dht else None)
        for name, x, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
            errs[name] = rel_l2(_gpu(x, heads), r[:, :, 0, :])
        errs["dg"] = rel_l2(_gpu(dg, heads), ref[3][:, :, 0])
        errs["dS0"] = rel_l2(_gpu(ds0, heads, True), ref[4][:, 0])
    tol = TOL[w.torch_dtype]
    note("  rel-L2 " + " ".join("%s=%.3e" % kv for kv in errs.items()) + " (tol %.0e)" % tol)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


@pytest.mark.parametrize("B,H,T,K,V,s0", [
    (1, 1, 64, 64, 64, "none"),           # one chunk
    (1, 2, 320, 64, 64, "normal0.1"),     # several segments, S0
    (2, 2, 448, 64, 128, "none"),         # uneven segments
    (1, 2, 256, 128, 64, "normal0.1"),
    (1, 1, 192, 128, 128, "normal0.1"),
    (2, 2, 1024, 128, 256, "normal0.1"),  # the metric's head dims, several segments
    (1, 2, 256, 256, 64, "normal0.1"),
])
def test_scalar_gate_matches_oracle(B, H, T, K, V, s0):
    w, inp = _inputs(B, H, T, K, V, s0, seed=700 + T + K + V)
    _check(w, inp)


def test_scalar_gate_wide_values():
    # dv = 512: a forward kernel; the backward runs two value slices of 256
    w, inp = _inputs(1, 2, 256, 128, 512, "normal0.1", seed=771)
    _check(w, inp)


@pytest.mark.parametrize("K,V,T", [(512, 128, 320), (512, 512, 192)])
def test_scalar_gate_wide_keys(K, V, T):
    # dk = 512: two key slices of 256 that share the per-token gate; dg is the
    # sum of the slices' gate gradients
    w, inp = _inputs(1, 2, T, K, V, "normal0.1", seed=780 + K + V + T)
    _check(w, inp)


def test_scalar_gate_ungated():
    # g = 0: plain causal linear attention
    w, inp = _inputs(2, 2, 256, 64, 64, "none", seed=772, gate_fn=lambda g: torch.zeros_like(g))
    _check(w, inp)


def test_scalar_gate_extreme_decay_exact_path():
    # a token whose decay exceeds the chunk basis range sends its chunk down the exact path
    def strong(g):
        g = g.float()
        g[0, 70, :] = -80.0
        g[0, 130:140, 1] = -12.0
        return g.to(torch.bfloat16)
    w, inp = _inputs(1, 2, 256, 64, 64, "normal0.1", seed=773, gate_fn=strong)
    _check(w, inp)


def test_scalar_gate_metric_size():
    # the throughput shape (B=2 H=4 T=8192 dk=128 dv=256) with scalar gates, two sampled heads
    w, inp = _inputs(2, 4, 8192, 128, 256, "none", seed=774)
    _check(w, inp, heads=[(0, 1), (1, 3)], with_dht=False)


@pytest.mark.parametrize("B,H,T,K,V", [(1, 2, 320, 64, 64), (2, 1, 192, 128, 128), (1, 2, 256, 256, 256)])
def test_scalar_gate_fp32(B, H, T, K, V):
    # fp32: the per-column path on the gate repeated over the key columns, dg
    # summed over them (K = 256 and V = 256 as slices of 128)
    w, inp = _inputs(B, H, T, K, V, "normal0.1", seed=790 + T + K + V, dtype="fp32")
    _check(w, inp)
