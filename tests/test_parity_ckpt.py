"""GPU parity of the checkpointed training pairs (gla_fwd_ckpt + gla_bwd_ckpt, and
gla_fwd_scalar_ckpt + gla_bwd_scalar_ckpt for one gate per token and head).

The forward keeps the state at the start of each backward segment (the segment
combine writes it when every such start is a forward segment start, else the
walk stores it as it passes that chunk boundary); the backward starts its
segments from those states instead of recomputing them.  The forward's outputs
must equal the plain forward's bit for bit, and the gradients must match the fp64
oracle's reverse-mode gradient to the bf16 bound on every head and every
64-token chunk, at small shapes (several segments, ragged last segment, the
half-segment dv walk) and at the full size of the benchmark workload.
"""
import pytest
import torch

import chunkwise_linear_rnn_amd as gla
import gla_inputs as gi
import oracle
from tests.parity_util import TOL, chunk_rel_l2, gpu_heads, head_subset, note, rel_l2, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(w, heads=None, with_dht=False, inputs=None):
    inp = inputs if inputs is not None else gi.make_inputs(w, dht=with_dht)
    note("ckpt parity: B=%d H=%d T=%d K=%d V=%d %s gate=%s s0=%s dht=%s" % (
        w.B, w.H, w.T, w.K, w.V, w.dtype, w.gate, w.s0, inp.get("dht") is not None))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    assert gla.gla_ckpt_size(w.B, w.T, w.H, w.K, w.V, w.torch_dtype) > 0
    o, sf, ck = gla.gla_fwd_ckpt(d["q"], d["k"], d["v"], d["g"], d["s0"])
    o_ref, sf_ref = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"], d["s0"])
    grads = gla.gla_bwd_ckpt(d["q"], d["k"], d["v"], d["g"], d["do"], ck, d["s0"], d["dht"])
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(sf, sf_ref)
    if heads is None:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    sel = lambda name: head_subset(to_np(inp[name]), heads)
    s0 = head_subset(to_np(inp.get("s0")), heads, state=True)
    dht = head_subset(to_np(inp.get("dht")), heads, state=True)
    ref = oracle.gla_bwd(sel("q"), sel("k"), sel("v"), sel("g"), sel("do"), s0, dht)
    tol = TOL[w.torch_dtype]
    errs, worst = {}, {}
    for name, x, r in zip(("dq", "dk", "dv", "dg", "ds0"), grads, ref):
        if name == "ds0":
            xs, rs = gpu_heads(x, heads, state=True), r[:, 0]
            errs[name] = rel_l2(xs, rs)
            worst[name] = max(rel_l2(xs[i], rs[i]) for i in range(len(heads)))
        else:
            xs, rs = gpu_heads(x, heads), r[:, :, 0, :]
            errs[name] = rel_l2(xs, rs)
            worst[name] = chunk_rel_l2(xs, rs)
    note("  rel-L2 " + " ".join("%s=%.3e" % kv for kv in errs.items()) + " (tol %.0e)" % tol)
    note("  worst chunk/head " + " ".join("%s=%.3e" % kv for kv in worst.items()))
    assert all(v <= tol for v in errs.values()), errs
    assert all(v <= tol for v in worst.values()), worst


@pytest.mark.parametrize("B,H,T,K,V,s0,dht", [
    (1, 2, 320, 64, 64, "normal0.1", True),      # several segments per head
    (2, 2, 448, 64, 128, "none", True),          # uneven segments
    (1, 2, 64 * 9, 128, 128, "normal0.1", False),
    (4, 16, 64 * 13, 128, 256, "normal0.1", True),  # the half-segment dv walk, ragged last segment
    (2, 16, 64 * 21, 128, 256, "none", False),   # a last segment with an empty second half
    (2, 4, 64 * 10, 64, 256, "normal0.1", True),
])
def test_ckpt_small(B, H, T, K, V, s0, dht):
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0=s0, backward=True, seed=700 + T + K + V)
    heads = None if B * H <= 8 else [(0, 0), (B - 1, H - 1), (B // 2, H // 2)]
    _check(w, heads=heads, with_dht=dht)


def test_ckpt_exact_path():
    from tests.test_parity_fwd import exact_path_inputs
    w = gi.custom(2, 4, 64 * 10, 128, 256, dtype="bf16", gate="iid", s0="normal0.1", backward=True, seed=731)
    _check(w, inputs=exact_path_inputs(w))


@pytest.mark.parametrize("name,heads", [
    ("metric_8k", None),
    ("fwdbwd_16k", [(b, h) for b in range(4) for h in (0, 7, 15)]),
])
def test_ckpt_named_workloads(name, heads):
    _check(gi.WORKLOADS[name], heads=heads)


def test_ckpt_absent_for_uncovered_shapes():
    # fp32, K = 256, or one backward segment: no checkpoint; the pair is gla_fwd / gla_bwd
    assert gla.gla_ckpt_size(1, 256, 1, 64, 64, torch.float32) == 0
    assert gla.gla_ckpt_size(2, 8192, 4, 256, 256, torch.bfloat16) == 0
    w = gi.custom(1, 1, 64, 64, 64, dtype="bf16", gate="iid", s0="normal0.1", backward=True, seed=732)
    assert gla.gla_ckpt_size(w.B, w.T, w.H, w.K, w.V, torch.bfloat16) == 0
    d = gi.make_inputs(w, device=DEV, dht=True)
    o, sf, ck = gla.gla_fwd_ckpt(d["q"], d["k"], d["v"], d["g"], d["s0"])
    assert ck is None
    a = gla.gla_bwd_ckpt(d["q"], d["k"], d["v"], d["g"], d["do"], None, d["s0"], d["dht"])
    b = gla.gla_bwd(d["q"], d["k"], d["v"], d["g"], d["do"], d["s0"], d["dht"])
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def _check_scalar(w, inp, heads=None, with_dht=True):
    from tests.test_parity_scalar_gate import _gpu, _sel
    note("scalar ckpt parity: B=%d H=%d T=%d K=%d V=%d s0=%s" % (w.B, w.H, w.T, w.K, w.V, w.s0))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    dht = d["dht"] if with_dht else None
    assert gla.gla_ckpt_size(w.B, w.T, w.H, w.K, w.V, w.torch_dtype) > 0
    o, sf, ck = gla.gla_fwd_scalar_ckpt(d["q"], d["k"], d["v"], d["g"], d["s0"])
    o_ref, sf_ref = gla.gla_fwd_scalar(d["q"], d["k"], d["v"], d["g"], d["s0"])
    grads = gla.gla_bwd_scalar_ckpt(d["q"], d["k"], d["v"], d["g"], d["do"], ck, d["s0"], dht)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(sf, sf_ref)
    if heads is None:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    c = {n: to_np(inp[n]) for n in ("q", "k", "v", "g", "do")}
    ref = oracle.gla_bwd_scalar(_sel(c["q"], heads), _sel(c["k"], heads), _sel(c["v"], heads), _sel(c["g"], heads),
                                _sel(c["do"], heads), _sel(to_np(inp.get("s0")), heads, state=True),
                                _sel(to_np(inp["dht"]), heads, state=True) if with_dht else None)
    errs = {}
    for name, x, r in zip(("dq", "dk", "dv"), grads[:3], ref[:3]):
        errs[name] = rel_l2(_gpu(x, heads), r[:, :, 0, :])
    errs["dg"] = rel_l2(_gpu(grads[3], heads), ref[3][:, :, 0])
    errs["ds0"] = rel_l2(_gpu(grads[4], heads, True), ref[4][:, 0])
    tol = TOL[torch.bfloat16]
    note("  rel-L2 " + " ".join("%s=%.3e" % kv for kv in errs.items()) + " (tol %.0e)" % tol)
    assert all(v <= tol for v in errs.values()), errs


@pytest.mark.parametrize("B,H,T,K,V,s0,dht", [
    (1, 2, 320, 64, 64, "normal0.1", True),        # several segments per head
    (2, 2, 448, 64, 128, "none", True),            # uneven segments
    (4, 16, 64 * 13, 128, 256, "normal0.1", True),  # the half-segment walks, ragged last segment
    (2, 16, 64 * 21, 128, 256, "none", False),     # a last segment with an empty second half
    (2, 4, 8192, 128, 256, "none", False),         # the throughput shape, every head
])
def test_scalar_ckpt(B, H, T, K, V, s0, dht):
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="scalar", s0=s0, backward=True, seed=760 + T + K + V)
    inp = gi.make_inputs(w, dht=True)
    heads = None if B * H <= 8 else [(0, 0), (B - 1, H - 1), (B // 2, H // 2)]
    _check_scalar(w, inp, heads=heads, with_dht=dht)


def test_scalar_ckpt_exact_path():
    # decays past the chunk basis range (one -80 nat reset, a run of -12 nat)
    w = gi.custom(2, 2, 64 * 9, 64, 128, dtype="bf16", gate="scalar", s0="normal0.1", backward=True, seed=781)
    inp = gi.make_inputs(w, dht=True)
    g = inp["g"].float()
    g[0, 70, :] = -80.0
    g[1, 300:310, 1] = -12.0
    inp["g"] = g.to(torch.bfloat16)
    _check_scalar(w, inp)
