"""GPU parity of gla_decode, the recurrent (token-by-token) form, through the C ABI.

The reference is the fp64 oracle recurrence run over the same tokens from the
same initial state: gla_decode computes exactly that recurrence (Eq. 3 of the
GLA paper), one token at a time, so o and the updated state are compared with
the oracle's o and final state.  Also checked: a call with T tokens equals T
calls of one token bit for bit (the state round-trips through HBM in fp32), and
decoding a 64-token chunk agrees with the chunked forward.
"""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_amd as gla
import gla_inputs as gi
import oracle
from tests.parity_util import TOL, note, rel_l2, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, H, T, K, V, dtype, gate, seed):
    w = gi.custom(B, H, T, K, V, dtype=dtype, gate=gate, s0="normal0.1", backward=False, seed=seed)
    return w, gi.make_inputs(w)


@pytest.mark.parametrize("B,H,T,K,V,dtype,gate", [
    (1, 1, 1, 64, 64, "fp32", "iid"),       # a single token
    (2, 3, 5, 64, 128, "fp32", "iid"),
    (1, 2, 7, 128, 256, "bf16", "lowrank"),
    (2, 1, 3, 256, 512, "bf16", "lowrank"),
    (1, 2, 4, 512, 128, "bf16", "lowrank"),  # 32 state rows per thread
    (1, 1, 3, 512, 64, "fp32", "iid"),
    (3, 2, 4, 128, 64, "bf16", "zero"),      # ungated: plain causal linear attention
    (1, 2, 70, 64, 64, "bf16", "iid"),       # longer than a chunk, not a multiple of it
])
def test_decode_matches_oracle(B, H, T, K, V, dtype, gate):
    w, inp = _inputs(B, H, T, K, V, dtype, gate, seed=300 + T + K + V)
    note("decode parity: B=%d H=%d T=%d K=%d V=%d %s gate=%s" % (B, H, T, K, V, dtype, gate))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    state = d["s0"].clone()
    o = gla.gla_decode(d["q"], d["k"], d["v"], d["g"], state)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.gla_fwd(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(inp["g"]),
                                  to_np(inp["s0"]))
    eo, es = rel_l2(to_np(o), o_ref), rel_l2(to_np(state), s_ref)
    tol = TOL[w.torch_dtype]
    note("  rel-L2 o=%.3e S_T=%.3e (tol %.0e)" % (eo, es, tol))
    assert eo <= tol and es <= tol, (eo, es)


def test_decode_one_token_at_a_time_is_bitwise_the_same():
    w, inp = _inputs(2, 2, 6, 128, 256, "bf16", "lowrank", seed=41)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    s_all = d["s0"].clone()
    o_all = gla.gla_decode(d["q"], d["k"], d["v"], d["g"], s_all)
    s_one = d["s0"].clone()
    outs = []
    for t in range(w.T):
        sl = lambda x: x[:, t:t + 1].contiguous()
        outs.append(gla.gla_decode(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), s_one))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), o_all)
    assert torch.equal(s_one, s_all)


def test_decode_agrees_with_chunked_forward():
    w, inp = _inputs(2, 2, 64, 128, 128, "bf16", "iid", seed=42)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    state = d["s0"].clone()
    o_dec = gla.gla_decode(d["q"], d["k"], d["v"], d["g"], state)
    o_fwd, s_fwd = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"], d["s0"])
    torch.cuda.synchronize()
    assert rel_l2(to_np(o_dec), to_np(o_fwd)) <= TOL[torch.bfloat16]
    assert rel_l2(to_np(state), to_np(s_fwd)) <= TOL[torch.bfloat16]


def test_decode_empty_is_a_no_op():
    q = torch.zeros(2, 0, 2, 64, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros(2, 0, 2, 64, dtype=torch.bfloat16, device=DEV)
    state = torch.randn(2, 2, 64, 64, device=DEV)
    before = state.clone()
    o = gla.gla_decode(q, q, v, q, state)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 64)
    assert torch.equal(state, before)


@pytest.mark.parametrize("B,H,T,K,V,dtype", [
    (2, 3, 5, 64, 128, "fp32"),
    (1, 2, 70, 128, 256, "bf16"),      # longer than a chunk, not a multiple of it
    (1, 2, 4, 512, 128, "bf16"),
    (1, 1, 3, 256, 512, "fp32"),
])
def test_decode_scalar_gate_matches_oracle(B, H, T, K, V, dtype):
    # one log gate per token and head, against the oracle's scalar-gate recurrence
    w = gi.custom(B, H, T, K, V, dtype=dtype, gate="scalar", s0="normal0.1", backward=False, seed=320 + T + K)
    inp = gi.make_inputs(w)
    note("decode parity (scalar gate): B=%d H=%d T=%d K=%d V=%d %s" % (B, H, T, K, V, dtype))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    state = d["s0"].clone()
    o = gla.gla_decode_scalar(d["q"], d["k"], d["v"], d["g"], state)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.gla_fwd_scalar(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(inp["g"]),
                                         to_np(inp["s0"]))
    eo, es = rel_l2(to_np(o), o_ref), rel_l2(to_np(state), s_ref)
    tol = TOL[w.torch_dtype]
    note("  rel-L2 o=%.3e S_T=%.3e (tol %.0e)" % (eo, es, tol))
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("B,H,T,K,V,dtype", [
    (2, 3, 5, 64, 128, "fp32"),
    (1, 2, 70, 128, 256, "bf16"),
    (1, 1, 3, 256, 512, "bf16"),
    (1, 2, 4, 512, 64, "bf16"),         # 32 state rows per thread, the value gate staged per 64 columns
    (1, 1, 3, 512, 512, "fp32"),
])
def test_decode_general_gate_matches_oracle(B, H, T, K, V, dtype):
    # the outer-product gate exp(g)^T exp(h), against the oracle's general recurrence
    w = gi.custom(B, H, T, K, V, dtype=dtype, gate="lowrank", s0="normal0.1", backward=False, seed=340 + T + K)
    inp = gi.make_inputs(w)
    h = gi.make_value_gate(B, T, H, V, dtype=dtype, seed=350 + T)
    note("decode parity (general gate): B=%d H=%d T=%d K=%d V=%d %s" % (B, H, T, K, V, dtype))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    state = d["s0"].clone()
    o = gla.gla_decode_general(d["q"], d["k"], d["v"], d["g"], h.to(DEV), state)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.gla_fwd_general(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(inp["g"]),
                                          to_np(h), to_np(inp["s0"]))
    eo, es = rel_l2(to_np(o), o_ref), rel_l2(to_np(state), s_ref)
    tol = TOL[w.torch_dtype]
    note("  rel-L2 o=%.3e S_T=%.3e (tol %.0e)" % (eo, es, tol))
    assert eo <= tol and es <= tol, (eo, es)


def test_decode_general_zero_value_gate_is_gla_decode():
    # h = 0 (beta = 1) gives the key-side recurrence exactly (the same fp32 arithmetic)
    w, inp = _inputs(1, 2, 9, 128, 128, "bf16", "lowrank", seed=361)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    h = torch.zeros(1, 9, 2, 128, dtype=torch.bfloat16, device=DEV)
    s_a, s_b = d["s0"].clone(), d["s0"].clone()
    o_a = gla.gla_decode(d["q"], d["k"], d["v"], d["g"], s_a)
    o_b = gla.gla_decode_general(d["q"], d["k"], d["v"], d["g"], h, s_b)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(s_a, s_b)
