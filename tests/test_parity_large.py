"""Parity past 2^31 elements per token tensor.

At B=2, H=2048, T=16384, K=V=64 each token tensor holds 2^32 elements (8 GiB in
bf16), so the rows of the last head lie past every 32-bit element offset.  All
heads but the first and the last hold zeros (a zero log gate is a valid gate,
and zero inputs give zero outputs and gradients), so the drawn data and the
oracle's work stay those of two heads.  The two heads are compared with the
oracle, forward and backward, on the whole tensor and on every 64-token chunk;
heads in between must come out exactly zero, and no output may hold a
non-finite value.
"""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_amd as gla
import gla_inputs as gi
import oracle
from tests.parity_util import TOL, chunk_rel_l2, note, rel_l2, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_fwd_bwd_past_32bit_offsets():
    B, H, T, K, V = 2, 2048, 16384, 64, 64
    assert B * T * H * K == 1 << 32
    heads = [(0, 0), (B - 1, H - 1)]
    w = gi.custom(1, len(heads), T, K, V, dtype="bf16", gate="iid", s0="none", backward=True, seed=4242)
    small = gi.make_inputs(w)
    note("large-offset parity: B=%d H=%d T=%d K=%d V=%d bf16, data in heads %s" % (B, H, T, K, V, heads))
    big = {}
    for name, D in (("q", K), ("k", K), ("g", K), ("v", V), ("do", V)):
        x = torch.zeros(B, T, H, D, dtype=torch.bfloat16, device=DEV)
        for i, (b, h) in enumerate(heads):
            x[b, :, h, :] = small[name][0, :, i, :].to(DEV)
        big[name] = x
    o, sf = gla.gla_fwd(big["q"], big["k"], big["v"], big["g"])
    dq, dk, dv, dg, ds0 = gla.gla_bwd(big["q"], big["k"], big["v"], big["g"], big["do"])
    torch.cuda.synchronize()

    o_ref, s_ref = oracle.gla_fwd(*(to_np(small[n]) for n in ("q", "k", "v", "g")), None)
    bwd_ref = oracle.gla_bwd(*(to_np(small[n]) for n in ("q", "k", "v", "g", "do")), None, None)
    refs = {"o": o_ref, "dq": bwd_ref[0], "dk": bwd_ref[1], "dv": bwd_ref[2], "dg": bwd_ref[3]}
    got = {"o": o, "dq": dq, "dk": dk, "dv": dv, "dg": dg}
    tol = TOL[torch.bfloat16]
    errs, worst = {}, {}
    for name, x in got.items():
        xs = np.stack([to_np(x[b, :, h, :]) for b, h in heads])
        rs = np.stack([refs[name][0, :, i, :] for i in range(len(heads))])
        errs[name] = rel_l2(xs, rs)
        worst[name] = chunk_rel_l2(xs, rs)
    for name, x, r in (("S_T", sf, s_ref), ("ds0", ds0, bwd_ref[4])):
        xs = np.stack([to_np(x[b, h]) for b, h in heads])
        errs[name] = rel_l2(xs, r[0])
    note("  rel-L2 " + " ".join("%s=%.3e" % kv for kv in errs.items()) + " (tol %.0e)" % tol)
    note("  worst 64-token chunk " + " ".join("%s=%.3e" % kv for kv in worst.items()))
    assert all(v <= tol for v in errs.values()), errs
    assert all(v <= tol for v in worst.values()), worst
    for name, x in list(got.items()) + [("S_T", sf), ("ds0", ds0)]:
        assert bool(torch.isfinite(x).all()), name
    for b, h in ((0, 1), (1, 0), (0, H - 1), (1, H // 2)):
        for name, x in got.items():
            assert not bool(x[b, :, h, :].any()), (name, b, h)
        assert not bool(sf[b, h].any()) and not bool(ds0[b, h].any()), (b, h)
