"""GPU backward parity: gla_bwd (through the C ABI) against the fp64 oracle's
reverse-mode gradient of the recurrence (dq, dk, dv, dg, dS0).

The oracle takes dg through the state (independent of the closed form the GPU
uses), so agreement checks the closed-form gate gradient as well.
"""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_amd as gla
import gla_inputs as gi
import oracle
from tests.parity_util import TOL, chunk_rel_l2, gpu_heads, head_subset, max_chunk_decay_log2, note, rel_l2, to_np
from tests.test_parity_fwd import exact_path_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check_bwd(w, heads=None, with_dht=False, inputs=None, tol=None):
    inp = inputs if inputs is not None else gi.make_inputs(w, dht=with_dht)
    note("bwd parity: B=%d H=%d T=%d K=%d V=%d %s gate=%s s0=%s dht=%s" % (w.B, w.H, w.T, w.K, w.V, w.dtype, w.gate,
                                                                          w.s0, inp.get("dht") is not None))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    dq, dk, dv, dg, ds0 = gla.gla_bwd(d["q"], d["k"], d["v"], d["g"], d["do"], d["s0"], d["dht"])
    torch.cuda.synchronize()
    if heads is None:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    sel = lambda name: head_subset(to_np(inp[name]), heads)
    s0 = head_subset(to_np(inp.get("s0")), heads, state=True)
    dht = head_subset(to_np(inp.get("dht")), heads, state=True)
    ref = oracle.gla_bwd(sel("q"), sel("k"), sel("v"), sel("g"), sel("do"), s0, dht)
    names = ("dq", "dk", "dv", "dg", "ds0")
    got = (dq, dk, dv, dg, ds0)
    tol = tol if tol is not None else TOL[w.torch_dtype]
    errs, worst = {}, {}
    for name, x, r in zip(names, got, ref):
        if name == "ds0":
            xs, rs = gpu_heads(x, heads, state=True), r[:, 0]
            errs[name] = rel_l2(xs, rs)
            worst[name] = max(rel_l2(xs[i], rs[i]) for i in range(len(heads)))
        else:
            xs, rs = gpu_heads(x, heads), r[:, :, 0, :]
            errs[name] = rel_l2(xs, rs)
            worst[name] = chunk_rel_l2(xs, rs)
    note("  rel-L2 " + " ".join("%s=%.3e" % kv for kv in errs.items()) + " (tol %.0e)" % tol)
    note("  worst 64-token chunk (ds0: worst head) " + " ".join("%s=%.3e" % kv for kv in worst.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad
    # the bound holds on every chunk of every compared head as well
    bad = {k: v for k, v in worst.items() if not v <= tol}
    assert not bad, bad
    return errs


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,H,T,K,V,s0,dht", [
    (1, 1, 64, 64, 64, "none", False),          # one chunk
    (1, 2, 320, 64, 64, "normal0.1", True),     # several segments, S0 and dht
    (2, 2, 448, 64, 128, "none", True),         # uneven segments
    (1, 2, 256, 128, 64, "normal0.1", False),
    (1, 1, 192, 128, 128, "normal0.1", True),
])
def test_bwd_small(dtype, B, H, T, K, V, s0, dht):
    w = gi.custom(B, H, T, K, V, dtype=dtype, gate="iid", s0=s0, backward=True, seed=200 + T + K + V)
    _check_bwd(w, with_dht=dht)


@pytest.mark.parametrize("K,V", [(256, 64), (256, 128), (256, 256), (128, 256), (64, 256)])
def test_bwd_wide_bf16(K, V):
    w = gi.custom(1, 2, 256, K, V, dtype="bf16", gate="lowrank", s0="normal0.1", backward=True, seed=11)
    _check_bwd(w, with_dht=True)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_bwd_ungated(dtype):
    w = gi.custom(2, 2, 256, 64, 64, dtype=dtype, gate="zero", v_scale="unit", backward=True, seed=12)
    _check_bwd(w, with_dht=True)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_bwd_near_basis_limit(dtype):
    # resets of -60 and -45 nat: about 92 log2 units of chunk decay, inside the
    # 16-bit factorised range (96); fp32 takes its element-wise path
    w = gi.custom(1, 2, 256, 64, 64, dtype=dtype, gate="iid", s0="normal0.1", backward=True, seed=13)
    inp = gi.make_inputs(w, dht=True)
    g = inp["g"].float()
    g[0, 70, :, :5] = -60.0
    g[0, 200, 1, :] = -45.0
    inp["g"] = g.to(w.torch_dtype)
    decay = max_chunk_decay_log2(inp["g"])
    assert 80.0 < decay.max() < 96.0, decay
    _check_bwd(w, inputs=inp)


@pytest.mark.parametrize("dtype,K,V", [("fp32", 64, 64), ("fp32", 64, 128), ("fp32", 128, 128)] + [
    ("bf16", K, V) for K, V in ((64, 64), (64, 128), (128, 128), (128, 256), (256, 64), (256, 256))])
def test_bwd_exact_path(dtype, K, V):
    # chunks past the factorised range (an asserted decay above 100 log2 units
    # in both heads): the intra-chunk parts of dq, dk and dv element by element
    w = gi.custom(1, 2, 256, K, V, dtype=dtype, gate="iid", s0="normal0.1", backward=True, seed=13 + K + V)
    _check_bwd(w, inputs=exact_path_inputs(w))


def test_bwd_empty_sequence():
    dht = torch.randn(2, 3, 64, 64, device=DEV)
    z = torch.empty(2, 0, 3, 64, dtype=torch.bfloat16, device=DEV)
    dq, dk, dv, dg, ds0 = gla.gla_bwd(z, z, z, z, z, None, dht)
    torch.cuda.synchronize()
    assert dq.shape == (2, 0, 3, 64)
    assert torch.equal(ds0, dht)


def test_bwd_deterministic():
    w = gi.custom(2, 2, 512, 128, 256, dtype="bf16", gate="lowrank", backward=True, seed=14)
    d = gi.make_inputs(w, device=DEV, dht=True)
    a = gla.gla_bwd(d["q"], d["k"], d["v"], d["g"], d["do"], None, d["dht"])
    b = gla.gla_bwd(d["q"], d["k"], d["v"], d["g"], d["do"], None, d["dht"])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name,heads", [
    ("metric_8k", None),
    ("fwdbwd_16k", [(b, h) for b in range(4) for h in (0, 5, 10, 15)]),
])
def test_bwd_named_workloads(name, heads):
    w = gi.WORKLOADS[name]
    _check_bwd(w, heads=heads)


@pytest.mark.parametrize("B,H,T", [
    (4, 16, 64 * 13),   # two segments of 7 and 6 chunks: halves of 4+3 and 4+2 chunks
    (2, 16, 64 * 21),   # segments of 6, 6, 6, 3 chunks: the last one has an empty second half
])
def test_bwd_half_segment_walks_ragged(B, H, T):
    # dk=128, dv=256 bf16 takes the value-width dv walk over half segments, started
    # from the midpoint states of the reverse segment-state pass
    w = gi.custom(B, H, T, 128, 256, dtype="bf16", gate="lowrank", s0="normal0.1", backward=True, seed=500 + T)
    _check_bwd(w, heads=[(0, 0), (B - 1, H - 1)], with_dht=True)


def test_exact_path_deterministic():
    # chunks past the basis range build A element by element; the waves' shares
    # are added in a fixed order, so repeated calls agree bit for bit
    w = gi.custom(1, 2, 256, 128, 256, dtype="bf16", gate="iid", s0="normal0.1", backward=True, seed=14)
    inp = gi.make_inputs(w, dht=True)
    g = inp["g"].float()
    g[0, 70, :, :40] = -60.0
    g[0, 150:160, 1, 64:] = -9.0
    inp["g"] = g.to(torch.bfloat16)
    assert max_chunk_decay_log2(inp["g"])[1] > 96.0
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    outs = []
    for _ in range(2):
        o, sf = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"], d["s0"])
        grads = gla.gla_bwd(d["q"], d["k"], d["v"], d["g"], d["do"], d["s0"], d["dht"])
        torch.cuda.synchronize()
        outs.append([o, sf] + list(grads))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    _check_bwd(w, inputs=inp)


@pytest.mark.parametrize("K,T,s0,dht", [(64, 192, "normal0.1", True), (128, 256, "none", True),
                                       (256, 320, "normal0.1", False)])
def test_bwd_value_width_512(K, T, s0, dht):
    # V = 512 runs as two V = 256 backwards over the value-column halves
    # (the recurrence never mixes value columns); dq, dk, dg add the halves
    w = gi.custom(1, 2, T, K, 512, dtype="bf16", gate="lowrank", s0=s0, backward=True, seed=600 + K + T)
    _check_bwd(w, with_dht=dht)


def test_bwd_value_width_512_exact_path():
    from tests.test_parity_fwd import exact_path_inputs
    w = gi.custom(1, 2, 256, 128, 512, dtype="bf16", gate="iid", s0="normal0.1", backward=True, seed=611)
    _check_bwd(w, inputs=exact_path_inputs(w))


@pytest.mark.parametrize("K,V,T,s0,dht", [(64, 256, 320, "normal0.1", True), (128, 256, 192, "none", True),
                                         (64, 512, 256, "normal0.1", False), (128, 512, 448, "normal0.1", True)])
def test_bwd_fp32_wide_values(K, V, T, s0, dht):
    # fp32 with V = 256 or 512 runs as V / 128 backwards over value-column
    # slices; dv and dS0 are the slices side by side, dq, dk, dg their sums
    w = gi.custom(1, 2, T, K, V, dtype="fp32", gate="lowrank", s0=s0, backward=True, seed=640 + K + V + T)
    _check_bwd(w, with_dht=dht)


def test_bwd_fp32_wide_values_exact_path():
    from tests.test_parity_fwd import exact_path_inputs
    w = gi.custom(1, 2, 256, 64, 512, dtype="fp32", gate="iid", s0="normal0.1", backward=True, seed=651)
    _check_bwd(w, inputs=exact_path_inputs(w))


@pytest.mark.parametrize("dtype,K,V,T,dht", [("bf16", 512, 64, 320, True), ("bf16", 512, 512, 192, True),
                                             ("fp32", 256, 128, 256, True), ("fp32", 512, 256, 192, False),
                                             ("fp32", 256, 64, 448, True)])
def test_bwd_wide_keys(dtype, K, V, T, dht):
    # key slices: dq, dk, dg are the slices' columns, dv their sum, dS0 their
    # row blocks (fp32 K = 512, V = 256 is sliced both ways)
    w = gi.custom(1, 2, T, K, V, dtype=dtype, gate="lowrank", s0="normal0.1", backward=True, seed=680 + K + V + T)
    _check_bwd(w, with_dht=dht)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bwd_wide_keys_exact_path(dtype):
    from tests.test_parity_fwd import exact_path_inputs
    w = gi.custom(1, 2, 256, 512, 128, dtype=dtype, gate="iid", s0="normal0.1", backward=True, seed=691)
    _check_bwd(w, inputs=exact_path_inputs(w))


def test_bwd_1p3b_head_shape_sampled_heads():
    # the 1.3B-model head shape at length 8K (the gla_1p3b_long recipe and seed,
    # with an upstream gradient drawn as well), two heads against the oracle
    w = gi.custom(2, 4, 8192, 256, 512, dtype="bf16", gate="lowrank", s0="normal0.1", backward=True, seed=4)
    _check_bwd(w, heads=[(0, 1), (1, 3)])
