"""GPU forward parity: libgla.so (through the C ABI) against the fp64 oracle.

Small shapes are compared on every head; the named workloads run at their
full size, in the same launch configuration the benchmark times, and are
compared on a sample of heads that the oracle recomputes completely.
"""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_amd as gla
import gla_inputs as gi
from tests.parity_util import TOL, gpu_heads, note, oracle_fwd_heads, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run_and_check(w, heads=None, tol=None, inputs=None):
    inp = inputs if inputs is not None else gi.make_inputs(w)
    note("fwd parity: %s B=%d H=%d T=%d K=%d V=%d %s gate=%s s0=%s" % (w.name, w.B, w.H, w.T, w.K, w.V, w.dtype,
                                                                     w.gate, w.s0))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    o, sf = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"], d["s0"])
    torch.cuda.synchronize()
    if heads is None:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    o_ref, s_ref = oracle_fwd_heads(inp, heads)
    eo = rel_l2(gpu_heads(o, heads), o_ref)
    es = rel_l2(gpu_heads(sf, heads, state=True), s_ref)
    tol = tol if tol is not None else TOL[w.torch_dtype]
    note("  rel-L2 o=%.3e S_T=%.3e (tol %.0e)" % (eo, es, tol))
    assert eo <= tol and es <= tol, (eo, es)
    return eo, es


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,H,T,K,V,s0", [
    (1, 1, 64, 64, 64, "none"),        # one chunk
    (1, 2, 320, 64, 64, "normal0.1"),  # five chunks, several segments
    (2, 3, 448, 128, 128, "none"),     # seven chunks: uneven segments
    (1, 2, 256, 64, 128, "normal0.1"),
    (1, 1, 384, 128, 64, "normal0.1"),
])
def test_fwd_small(dtype, B, H, T, K, V, s0):
    w = gi.custom(B, H, T, K, V, dtype=dtype, gate="iid", s0=s0, backward=False, seed=100 + T + K + V)
    _run_and_check(w)


@pytest.mark.parametrize("K,V", [(256, 64), (256, 512), (64, 512)])
def test_fwd_small_wide_bf16(K, V):
    w = gi.custom(1, 2, 192, K, V, dtype="bf16", gate="lowrank", s0="normal0.1", backward=False, seed=7)
    _run_and_check(w)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_ungated(dtype):
    w = gi.custom(2, 2, 256, 64, 128, dtype=dtype, gate="zero", v_scale="unit", backward=False, seed=8)
    _run_and_check(w)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_extreme_gates_exact_path(dtype):
    # hard resets (alpha ~ e^-60) push a chunk's gate range past the factorised
    # path's bound, so those chunks take the element-wise Eq. 4 path
    w = gi.custom(1, 2, 256, 64, 64, dtype=dtype, gate="iid", s0="normal0.1", backward=False, seed=9)
    inp = gi.make_inputs(w)
    g = inp["g"].float()
    g[0, 70, :, :5] = -60.0
    g[0, 200, 1, :] = -45.0
    inp["g"] = g.to(w.torch_dtype)
    _run_and_check(w, inputs=inp)


def test_fwd_empty_sequence_copies_state():
    s0 = torch.randn(2, 3, 64, 64, device=DEV)
    z = torch.empty(2, 0, 3, 64, dtype=torch.bfloat16, device=DEV)
    o, sf = gla.gla_fwd(z, z, z, z, s0)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 64)
    assert torch.equal(sf, s0)


def test_fwd_deterministic():
    w = gi.custom(2, 2, 512, 128, 256, dtype="bf16", gate="lowrank", backward=False, seed=10)
    d = gi.make_inputs(w, device=DEV)
    o1, s1 = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"])
    o2, s2 = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("name,heads", [
    ("tiny_fp32", None),
    ("ungated_1k", None),
    ("gla_340m", [(0, 0), (3, 2), (7, 3)]),
    ("metric_8k", [(0, 1), (1, 3)]),
    ("gla_1p3b_long", [(1, 2)]),
    ("fwdbwd_16k", [(0, 0), (3, 15)]),
])
def test_fwd_named_workloads(name, heads):
    w = gi.WORKLOADS[name]
    _run_and_check(w, heads=heads)
