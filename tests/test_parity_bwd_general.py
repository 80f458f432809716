"""GPU backward parity of general gated linear attention against the fp64
oracle's chain rule: dq, dk, dv, both gate gradients and dS0, on one chunk,
several segments, both key and value widths, gates past the basis range, and
the benchmark's full size (sampled heads)."""
import pytest
import torch

import chunkwise_linear_rnn_amd as gla
import gla_inputs as gi
import oracle
from tests.parity_util import TOL, gpu_heads, head_subset, note, rel_l2, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GATE_TOL = 1e-2


def _check(w, inp, h, heads):
    note("general bwd parity: B=%d H=%d T=%d K=%d V=%d s0=%s" % (w.B, w.H, w.T, w.K, w.V, w.s0))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    hd = h.to(DEV)
    dq, dk, dv, dg, dh, ds0 = gla.gla_bwd_general(d["q"], d["k"], d["v"], d["g"], hd, d["do"], d["s0"], d["dht"])
    torch.cuda.synchronize()
    sel = lambda a: head_subset(to_np(a), heads)
    sst = lambda a: head_subset(to_np(a), heads, state=True) if a is not None else None
    ref = oracle.gla_bwd_general(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["g"]), sel(h), sel(inp["do"]),
                                 sst(inp["s0"]), sst(inp["dht"]))
    tol = TOL[torch.bfloat16]
    errs = {}
    for name, got, r in zip(("dq", "dk", "dv", "dg", "dh"), (dq, dk, dv, dg, dh), ref[:5]):
        errs[name] = rel_l2(gpu_heads(got, heads), r[:, :, 0, :])
    errs["ds0"] = rel_l2(gpu_heads(ds0, heads, state=True), ref[5][:, 0])
    note("  rel-L2 " + " ".join("%s=%.2e" % kv for kv in errs.items()) + " (tol %.0e)" % tol)
    assert all(e <= tol for e in errs.values()), errs
    # the gate gradients sum dq, dk (dv, o) over each chunk between two exact
    # anchors: their own bound is half the general one
    assert errs["dg"] <= GATE_TOL and errs["dh"] <= GATE_TOL, errs


def _heads(B, H):
    return [(b, hh) for b in range(B) for hh in range(H)] if B * H <= 2 else [(0, 0), (B - 1, H - 1)]


@pytest.mark.parametrize("B,H,T,K,V,s0", [
    (1, 1, 64, 128, 128, "normal0.1"),      # one chunk
    (2, 2, 64 * 9, 128, 256, "normal0.1"),  # one chunk per segment
    (2, 4, 64 * 13, 256, 128, "none"),      # K > V
    (1, 2, 64 * 20, 256, 256, "normal0.1"),
])
def test_bwd_general_heads(B, H, T, K, V, s0):
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0=s0, backward=True, seed=1500 + T + K + V)
    inp = gi.make_inputs(w, dht=True)
    h = gi.make_value_gate(B, T, H, V, seed=1600 + T + V)
    _check(w, inp, h, _heads(B, H))


@pytest.mark.parametrize("B,H,T,K,V,s0", [
    (1, 2, 64 * 5, 512, 128, "normal0.1"),   # two key slices: dv, dh added
    (1, 2, 64 * 6, 128, 512, "normal0.1"),   # two value slices: dq, dk, dg added
    (1, 2, 64 * 3, 512, 512, "none"),        # both
    (1, 2, 64 * 7, 64, 128, "normal0.1"),    # K = 64 padded with zero key columns
    (2, 1, 64 * 5, 256, 64, "normal0.1"),    # V = 64 padded with zero value columns
    (1, 2, 64 * 4, 64, 64, "none"),          # both padded
    (1, 2, 64 * 3, 64, 512, "normal0.1"),    # padded keys, sliced values
])
def test_bwd_general_wide_heads(B, H, T, K, V, s0):
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0=s0, backward=True, seed=1520 + T + K + V)
    inp = gi.make_inputs(w, dht=True)
    h = gi.make_value_gate(B, T, H, V, seed=1620 + T + V)
    _check(w, inp, h, _heads(B, H))


def test_bwd_general_exact_paths_and_no_dht():
    B, H, T, K, V = 2, 2, 64 * 6, 128, 128
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0="normal0.1", backward=True, seed=1701)
    inp = gi.make_inputs(w)
    g = inp["g"].float()
    g[0, 70, 0, :5] = -70.0
    inp["g"] = g.to(torch.bfloat16)
    h = gi.make_value_gate(B, T, H, V, seed=1702).float()
    h[1, 200, 1, :] = -70.0
    h[0, 300:310, 1, 64:] = -9.0
    _check(w, inp, h.to(torch.bfloat16), [(0, 0), (1, 1), (0, 1)])


def test_bwd_general_full_size_sampled_heads():
    w = gi.WORKLOADS["metric_8k"]
    inp = gi.make_inputs(w, dht=True)
    h = gi.make_value_gate(w.B, w.T, w.H, w.V, dtype=w.dtype, seed=w.seed + 1)
    _check(w, inp, h, [(0, 0), (w.B - 1, w.H - 1)])


def test_bwd_general_deterministic():
    w = gi.custom(2, 4, 64 * 11, 128, 256, dtype="bf16", gate="lowrank", s0="normal0.1", backward=True, seed=1710)
    d = gi.make_inputs(w, device=DEV, dht=True)
    h = gi.make_value_gate(2, 64 * 11, 4, 256, seed=1711).to(DEV)
    a = gla.gla_bwd_general(d["q"], d["k"], d["v"], d["g"], h, d["do"], d["s0"], d["dht"])
    b = gla.gla_bwd_general(d["q"], d["k"], d["v"], d["g"], h, d["do"], d["s0"], d["dht"])
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("B,H,T,K,V,s0,dht", [
    (1, 1, 64, 128, 128, "normal0.1", True),      # one chunk: only the S_T anchor
    (2, 2, 64 * 9, 128, 256, "normal0.1", True),  # one chunk per segment
    (2, 4, 64 * 13, 256, 128, "none", False),     # K > V, no dht
    (2, 4, 8192, 128, 256, "normal0.1", True),    # the benchmark's shape
])
def test_bwd_general_ckpt_pair(B, H, T, K, V, s0, dht):
    # the pair runs the same kernels as gla_fwd_general + gla_bwd_general, with
    # the forward's o, chunk-start states and S_T kept instead of recomputed:
    # every result must be bit-identical; the first case also meets the oracle
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0=s0, backward=True, seed=1800 + T + K + V)
    inp = gi.make_inputs(w, dht=dht)
    h = gi.make_value_gate(B, T, H, V, seed=1900 + T + V)
    note("general ckpt pair: B=%d H=%d T=%d K=%d V=%d s0=%s dht=%s" % (B, H, T, K, V, s0, dht))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    hd = h.to(DEV)
    assert gla.gla_general_ckpt_size(B, T, H, K, V, torch.bfloat16) > 0
    o, sf, ck = gla.gla_fwd_general_ckpt(d["q"], d["k"], d["v"], d["g"], hd, d["s0"])
    o_ref, sf_ref = gla.gla_fwd_general(d["q"], d["k"], d["v"], d["g"], hd, d["s0"])
    got = gla.gla_bwd_general_ckpt(d["q"], d["k"], d["v"], d["g"], hd, d["do"], o, ck, d["s0"], d["dht"])
    ref = gla.gla_bwd_general(d["q"], d["k"], d["v"], d["g"], hd, d["do"], d["s0"], d["dht"])
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(sf, sf_ref)
    for name, a, b in zip(("dq", "dk", "dv", "dg", "dh", "ds0"), got, ref):
        assert torch.equal(a, b), name
    if T == 64:
        _check(w, inp, h, _heads(B, H))


def test_general_ckpt_pair_without_checkpoint_is_the_plain_pair():
    # V = 512 (value slices) has no checkpoint: the pair runs gla_fwd_general /
    # gla_bwd_general, bit for bit
    B, H, T, K, V = 1, 2, 64 * 3, 128, 512
    assert gla.gla_general_ckpt_size(B, T, H, K, V, torch.bfloat16) == 0
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0="normal0.1", backward=True, seed=1720)
    d = gi.make_inputs(w, device=DEV, dht=True)
    h = gi.make_value_gate(B, T, H, V, seed=1721).to(DEV)
    o, sf, ck = gla.gla_fwd_general_ckpt(d["q"], d["k"], d["v"], d["g"], h, d["s0"])
    o_ref, sf_ref = gla.gla_fwd_general(d["q"], d["k"], d["v"], d["g"], h, d["s0"])
    a = gla.gla_bwd_general_ckpt(d["q"], d["k"], d["v"], d["g"], h, d["do"], o, ck, d["s0"], d["dht"])
    b = gla.gla_bwd_general(d["q"], d["k"], d["v"], d["g"], h, d["do"], d["s0"], d["dht"])
    torch.cuda.synchronize()
    assert ck is None
    assert torch.equal(o, o_ref) and torch.equal(sf, sf_ref)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
