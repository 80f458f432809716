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
from tests.parity_util import TOL, chunk_rel_l2, gpu_heads, max_chunk_decay_log2, note, oracle_fwd_heads, rel_l2

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
    o_gpu, s_gpu = gpu_heads(o, heads), gpu_heads(sf, heads, state=True)
    eo = rel_l2(o_gpu, o_ref)
    es = rel_l2(s_gpu, s_ref)
    # the same bound on every 64-token chunk of every compared head, and on
    # every head's final state on its own, so that one bad chunk or segment
    # cannot hide under the whole-tensor norm
    eo_c = chunk_rel_l2(o_gpu, o_ref)
    es_h = max(rel_l2(s_gpu[i], s_ref[i]) for i in range(len(heads)))
    tol = tol if tol is not None else TOL[w.torch_dtype]
    note("  rel-L2 o=%.3e S_T=%.3e; worst chunk of o %.3e, worst head of S_T %.3e (tol %.0e)" % (
        eo, es, eo_c, es_h, tol))
    assert eo <= tol and es <= tol, (eo, es)
    assert eo_c <= tol and es_h <= tol, (eo_c, es_h)
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


@pytest.mark.parametrize("K,V,T", [(64, 256, 320), (128, 256, 192), (64, 512, 256), (128, 512, 448)])
def test_fwd_fp32_wide_values(K, V, T):
    # fp32 with V = 256 or 512 runs as value-column slices of 128 (the
    # recurrence never mixes value columns); o and S_T are the slices side by side
    w = gi.custom(1, 2, T, K, V, dtype="fp32", gate="lowrank", s0="normal0.1", backward=False, seed=620 + K + V + T)
    _run_and_check(w)


@pytest.mark.parametrize("dtype,K,V,T", [("bf16", 512, 64, 320), ("bf16", 512, 512, 192), ("fp32", 256, 128, 256),
                                         ("fp32", 512, 256, 192), ("fp32", 256, 64, 448)])
def test_fwd_wide_keys(dtype, K, V, T):
    # K past the kernels' widest (16-bit: 256, fp32: 128) runs as key slices:
    # each state row evolves on its own, o adds the slices' outputs and S_T
    # stacks their row blocks (fp32 K = 512, V = 256 is sliced both ways)
    w = gi.custom(1, 2, T, K, V, dtype=dtype, gate="lowrank", s0="normal0.1", backward=False, seed=660 + K + V + T)
    _run_and_check(w)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fwd_wide_keys_exact_path(dtype):
    # the -70 nat reset lands in the first key slice, the -9 nat run in the second
    w = gi.custom(1, 2, 256, 512, 128, dtype=dtype, gate="iid", s0="normal0.1", backward=False, seed=671)
    _run_and_check(w, inputs=exact_path_inputs(w))


def test_fwd_fp32_wide_values_exact_path():
    w = gi.custom(1, 2, 256, 128, 256, dtype="fp32", gate="iid", s0="normal0.1", backward=False, seed=631)
    _run_and_check(w, inputs=exact_path_inputs(w))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_ungated(dtype):
    w = gi.custom(2, 2, 256, 64, 128, dtype=dtype, gate="zero", v_scale="unit", backward=False, seed=8)
    _run_and_check(w)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_near_basis_limit(dtype):
    # single resets of -60 and -45 nat bring one chunk's decay to about 92 log2
    # units: still inside the 16-bit path's factorised range (96), so bf16 runs
    # the chunk-start basis close to its bound; fp32 (range limit 64) takes the
    # element-wise Eq. 4 path for those chunks
    w = gi.custom(1, 2, 256, 64, 64, dtype=dtype, gate="iid", s0="normal0.1", backward=False, seed=9)
    inp = gi.make_inputs(w)
    g = inp["g"].float()
    g[0, 70, :, :5] = -60.0
    g[0, 200, 1, :] = -45.0
    inp["g"] = g.to(w.torch_dtype)
    decay = max_chunk_decay_log2(inp["g"])
    assert 80.0 < decay.max() < 96.0, decay
    _run_and_check(w, inputs=inp)


def exact_path_inputs(w):
    """Inputs whose gates push chunks past the factorised range: one -70 nat
    reset (101 log2 units) in five key columns of both heads, and -9 nat over ten
    tokens (130 log2 units) in the upper half of head 1's key columns."""
    inp = gi.make_inputs(w, dht=w.backward)
    g = inp["g"].float()
    g[0, 70, :, :5] = -70.0
    g[0, 150:160, 1, w.K // 2:] = -9.0
    inp["g"] = g.to(w.torch_dtype)
    decay = max_chunk_decay_log2(inp["g"])
    assert (decay > 100.0).all(), decay   # every head has a chunk past the bound
    return inp


@pytest.mark.parametrize("dtype,K,V", [("fp32", 64, 64), ("fp32", 64, 128), ("fp32", 128, 128)] + [
    ("bf16", K, V) for K, V in ((64, 64), (64, 128), (128, 128), (128, 256), (64, 512))])
def test_fwd_exact_path(dtype, K, V):
    # chunks whose column decay passes the factorised range (bf16: 96 log2
    # units, fp32: 64) build the intra-chunk matrix element by element in fp32
    # (Eq. 4 with full-precision sub-chunk tiles, Section 4.3)
    w = gi.custom(1, 2, 256, K, V, dtype=dtype, gate="iid", s0="normal0.1", backward=False, seed=9 + K + V)
    _run_and_check(w, inputs=exact_path_inputs(w))


@pytest.mark.parametrize("V", [64, 256])
def test_fwd_exact_path_wide(V):
    # dk = 256 (chunk-record forward): the record kernel's element-wise branch
    w = gi.custom(1, 2, 256, 256, V, dtype="bf16", gate="iid", s0="normal0.1", backward=False, seed=19 + V)
    _run_and_check(w, inputs=exact_path_inputs(w))


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
    ("gla_340m", [(b, h) for b in range(8) for h in range(4) if (b + h) % 3 == 0]),
    ("metric_8k", None),
    ("gla_1p3b_long", None),
    ("fwdbwd_16k", [(b, h) for b in range(4) for h in (0, 5, 10, 15)]),
])
def test_fwd_named_workloads(name, heads):
    w = gi.WORKLOADS[name]
    _run_and_check(w, heads=heads)
