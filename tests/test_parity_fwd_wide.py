"""GPU forward parity for 16-bit heads with dk = 256 against the fp64 oracle.

These heads take the chunk-record forward: each chunk's operands (Ql, Kt, the
gate factors and the intra-chunk A) are formed once per chunk and head, then a
state pass, the segment combine and the output walk stream them.  The cases
cover one and several value blocks per head, segments of one and of several
chunks with a ragged last segment, chunks past the basis range inside a
segment (both in the state pass and in the output walk), and scalar gates.
"""
import pytest
import torch

import chunkwise_linear_rnn_amd as gla
import gla_inputs as gi
from tests.parity_util import TOL, gpu_heads, max_chunk_decay_log2, note, oracle_fwd_heads, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(w, inp, heads, scalar=False):
    note("wide fwd parity: B=%d H=%d T=%d K=%d V=%d gate=%s s0=%s scalar=%s" % (w.B, w.H, w.T, w.K, w.V, w.gate,
                                                                             w.s0, scalar))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    fwd = gla.gla_fwd_scalar if scalar else gla.gla_fwd
    o, sf = fwd(d["q"], d["k"], d["v"], d["g"], d["s0"])
    torch.cuda.synchronize()
    if scalar:
        # the oracle's per-column form with the token's gate in every key column
        ref_inp = dict(inp)
        ref_inp["g"] = inp["g"][..., None].expand(w.B, w.T, w.H, w.K).contiguous()
    else:
        ref_inp = inp
    o_ref, s_ref = oracle_fwd_heads(ref_inp, heads)
    eo = rel_l2(gpu_heads(o, heads), o_ref)
    es = rel_l2(gpu_heads(sf, heads, state=True), s_ref)
    tol = TOL[torch.bfloat16]
    note("  rel-L2 o=%.3e S_T=%.3e (tol %.0e)" % (eo, es, tol))
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("B,H,T,V,s0", [
    (1, 1, 64, 128, "normal0.1"),        # one chunk, one segment, one value block
    (1, 2, 64 * 9, 256, "normal0.1"),    # two value blocks, one chunk per segment
    (4, 16, 64 * 13, 256, "none"),       # two segments of 7 and 6 chunks
    (2, 8, 64 * 21, 512, "normal0.1"),   # four value blocks, segments of 6, 6, 6, 3 chunks
    (8, 8, 64 * 10, 64, "normal0.1"),    # dv = 64: 16-column wave slices
])
def test_fwd_wide_heads(B, H, T, V, s0):
    w = gi.custom(B, H, T, 256, V, dtype="bf16", gate="lowrank", s0=s0, backward=False, seed=900 + T + V)
    heads = [(b, h) for b in range(B) for h in range(H)] if B * H <= 2 else [(0, 0), (B - 1, H - 1)]
    _check(w, gi.make_inputs(w), heads)


def test_fwd_wide_exact_path_inside_segments():
    # B*H = 64 heads and two value blocks give two segments of four chunks: a
    # chunk past the basis range (96 log2 units) at token 70 (second chunk of
    # segment 0, in the state pass), at token 330 (second chunk of segment 1, in
    # the output walk), and over tokens 300..309 in half the key columns
    w = gi.custom(4, 16, 64 * 8, 256, 256, dtype="bf16", gate="iid", s0="normal0.1", backward=False, seed=931)
    inp = gi.make_inputs(w)
    g = inp["g"].float()
    g[0, 70, 0, :5] = -70.0
    g[0, 330, 1, :] = -70.0
    g[3, 300:310, 15, 128:] = -9.0
    inp["g"] = g.to(torch.bfloat16)
    assert (max_chunk_decay_log2(inp["g"])[[0, 1, 15]] > 100.0).all()
    _check(w, inp, [(0, 0), (0, 1), (3, 15)])


def test_fwd_wide_deterministic():
    w = gi.custom(2, 8, 64 * 21, 256, 512, dtype="bf16", gate="lowrank", s0="normal0.1", backward=False, seed=932)
    d = gi.make_inputs(w, device=DEV)
    a = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"], d["s0"])
    b = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"], d["s0"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("B,H,T,V", [(1, 2, 256, 512), (2, 8, 64 * 21, 512)])
def test_fwd_wide_scalar_gate(B, H, T, V):
    w = gi.custom(B, H, T, 256, V, dtype="bf16", gate="scalar", s0="normal0.1", backward=False, seed=940 + T)
    heads = [(b, h) for b in range(B) for h in range(H)] if B * H <= 2 else [(0, 0), (B - 1, H - 1)]
    _check(w, gi.make_inputs(w), heads, scalar=True)


def test_fwd_wide_scalar_gate_exact_path():
    # a scalar decay past the basis range sends its chunk down the element-wise
    # path of the record kernel (two segments of four chunks, second chunk of each)
    w = gi.custom(4, 16, 64 * 8, 256, 256, dtype="bf16", gate="scalar", s0="normal0.1", backward=False, seed=951)
    inp = gi.make_inputs(w)
    g = inp["g"].float()
    g[0, 70, 0] = -80.0
    g[0, 330, 1] = -70.0
    g[3, 300:310, 15] = -12.0
    inp["g"] = g.to(torch.bfloat16)
    _check(w, inp, [(0, 0), (0, 1), (3, 15)], scalar=True)
