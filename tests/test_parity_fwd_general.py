"""GPU forward parity of general gated linear attention against the fp64 oracle.

The forget gate is the outer product exp(g_t)^T exp(h_t) of a key-side and a
value-side gate.  The cases cover one chunk, one and several chunks per
segment with a ragged last segment, one to eight value blocks per head, both
key widths, chunks whose key-side or value-side decay leaves the basis range
(the element-wise paths of the record kernel), and the h = 0 reduction.
"""
import pytest
import torch

import chunkwise_linear_rnn_amd as gla
import gla_inputs as gi
import oracle
from tests.parity_util import TOL, gpu_heads, head_subset, note, rel_l2, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _oracle(inp, h, heads):
    sel = lambda a: head_subset(to_np(a), heads)
    s0 = inp.get("s0")
    o, sf = oracle.gla_fwd_general(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["g"]), sel(h),
                                   head_subset(to_np(s0), heads, state=True) if s0 is not None else None)
    return o[:, :, 0, :], sf[:, 0]


def _check(w, inp, h, heads):
    note("general fwd parity: B=%d H=%d T=%d K=%d V=%d s0=%s" % (w.B, w.H, w.T, w.K, w.V, w.s0))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    o, sf = gla.gla_fwd_general(d["q"], d["k"], d["v"], d["g"], h.to(DEV), d["s0"])
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(inp, h, heads)
    eo = rel_l2(gpu_heads(o, heads), o_ref)
    es = rel_l2(gpu_heads(sf, heads, state=True), s_ref)
    tol = TOL[torch.bfloat16]
    note("  rel-L2 o=%.3e S_T=%.3e (tol %.0e)" % (eo, es, tol))
    assert eo <= tol and es <= tol, (eo, es)


def _heads(B, H):
    return [(b, hh) for b in range(B) for hh in range(H)] if B * H <= 2 else [(0, 0), (B - 1, H - 1)]


@pytest.mark.parametrize("B,H,T,K,V,s0", [
    (1, 1, 64, 128, 64, "normal0.1"),      # one chunk, one value block
    (1, 2, 64 * 9, 256, 256, "normal0.1"),  # one chunk per segment, two value blocks
    (4, 4, 64 * 12, 128, 128, "none"),      # 12 segments of one chunk
    (2, 2, 64 * 13, 128, 256, "normal0.1"),  # one chunk per segment, 13 segments
    (2, 8, 64 * 21, 256, 512, "normal0.1"),  # 4 segments (6, 6, 6 and 3 chunks), four value blocks
    (1, 2, 64 * 20, 256, 256, "none"),      # 20 segments: the combine holds up to 32 segments in registers
    (1, 1, 64 * 40, 128, 128, "normal0.1"),  # 40 segments: the combine's loop for more than 32
])
def test_fwd_general_heads(B, H, T, K, V, s0):
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0=s0, backward=False, seed=1200 + T + V + K)
    h = gi.make_value_gate(B, T, H, V, seed=1300 + T + V)
    _check(w, gi.make_inputs(w), h, _heads(B, H))


@pytest.mark.parametrize("B,H,T,K,V", [(1, 2, 64 * 5, 512, 128), (2, 2, 64 * 3, 512, 512), (1, 2, 64 * 7, 64, 64),
                                       (2, 2, 64 * 4, 64, 256)])
def test_fwd_general_wide_keys(B, H, T, K, V):
    # dk = 512: two key slices of 256 sharing v and the value-side gate; o adds
    # the slices' outputs, S_T stacks their row blocks.  dk = 64: padded to 128
    # with zero columns of q, k and g (the padded state rows stay zero)
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0="normal0.1", backward=False, seed=1250 + T + V)
    h = gi.make_value_gate(B, T, H, V, seed=1350 + T + V)
    _check(w, gi.make_inputs(w), h, _heads(B, H))


def test_fwd_general_exact_paths():
    # B*H = 16 heads at K = 256, V = 256 give two segments of 8 and 7 chunks;
    # a key-side decay past the basis range at token 70 and a value-side one at
    # tokens 140 (all columns) and 600..609 (half the columns)
    B, H, T, K, V = 4, 4, 64 * 15, 256, 256
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0="normal0.1", backward=False, seed=1401)
    inp = gi.make_inputs(w)
    g = inp["g"].float()
    g[0, 70, 0, :7] = -70.0
    inp["g"] = g.to(torch.bfloat16)
    h = gi.make_value_gate(B, T, H, V, seed=1402).float()
    h[0, 140, 0, :] = -70.0
    h[3, 600:610, 3, 128:] = -9.0
    h[1, 530, 2, 5] = -80.0
    _check(w, inp, h.to(torch.bfloat16), [(0, 0), (3, 3), (1, 2)])


@pytest.mark.parametrize("V", [128, 64])
def test_fwd_general_exact_paths_k128(V):
    # at K = 128 the output walk forms the intra-chunk output itself for value
    # passes in range and takes the record's for passes out of range: a
    # key-side reset at token 70, value-side resets at token 140 (all columns)
    # and 330 (one column), and -9 per token over 300..309 in half the columns
    B, H, T, K = 2, 4, 64 * 9, 128
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0="normal0.1", backward=False, seed=1430 + V)
    inp = gi.make_inputs(w)
    g = inp["g"].float()
    g[0, 70, 0, :7] = -70.0
    inp["g"] = g.to(torch.bfloat16)
    h = gi.make_value_gate(B, T, H, V, seed=1440 + V).float()
    h[0, 140, 0, :] = -70.0
    h[1, 300:310, 2, V // 2:] = -9.0
    h[1, 330, 3, 5] = -80.0
    _check(w, inp, h.to(torch.bfloat16), [(0, 0), (1, 2), (1, 3), (0, 1)])


def test_fwd_general_zero_value_gate_matches_gla_fwd():
    # beta = 1 is the key-side-only operator: the same oracle values as gla_fwd
    B, H, T, K, V = 2, 4, 64 * 7, 128, 256
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0="normal0.1", backward=False, seed=1410)
    inp = gi.make_inputs(w)
    h = gi.make_value_gate(B, T, H, V, kind="zero")
    _check(w, inp, h, [(0, 0), (1, 3)])
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    o1, s1 = gla.gla_fwd_general(d["q"], d["k"], d["v"], d["g"], h.to(DEV), d["s0"])
    o2, s2 = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"], d["s0"])
    torch.cuda.synchronize()
    assert rel_l2(to_np(o1), to_np(o2)) <= 1e-2 and rel_l2(to_np(s1), to_np(s2)) <= 1e-2


def test_fwd_general_deterministic():
    B, H, T, K, V = 2, 8, 64 * 21, 256, 512
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0="normal0.1", backward=False, seed=1420)
    d = gi.make_inputs(w, device=DEV)
    h = gi.make_value_gate(B, T, H, V, seed=1421).to(DEV)
    a = gla.gla_fwd_general(d["q"], d["k"], d["v"], d["g"], h, d["s0"])
    b = gla.gla_fwd_general(d["q"], d["k"], d["v"], d["g"], h, d["s0"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name", ["gla_1p3b_long", "metric_8k"])
def test_fwd_general_full_size_sampled_heads(name):
    # the benchmark's shapes and launch configuration (bench.py --fwd-only
    # --general-gate), h drawn as the bench draws it; two heads against the oracle
    w = gi.WORKLOADS[name]
    inp = gi.make_inputs(w)
    inp.pop("do", None)
    h = gi.make_value_gate(w.B, w.T, w.H, w.V, dtype=w.dtype, seed=w.seed + 1)
    _check(w, inp, h, [(0, 0), (w.B - 1, w.H - 1)])
