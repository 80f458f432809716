"""Parity past 2^31 elements per tensor, for each family of kernels.

Each case sizes one tensor the kernels index (the token tensors, or decode's
state) past 2^31 elements, so the rows of the last head lie past every 32-bit
element offset.  All heads but the first and the last hold zeros (zero log
gates are valid gates, and zero inputs give zero outputs and gradients), so the
drawn data and the oracle's work stay those of two heads.  The two heads are
compared with the oracle on the whole tensor and on every 64-token chunk; heads
in between must come out exactly zero, and no output may hold a non-finite
value.  Device memory peaks near 100 GiB per case and is released after it.
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


def _spread(x_small, B, H, heads):
    """[1, T, n, ...] -> [B, T, H, ...] on the device, zeros outside `heads`."""
    big = torch.zeros((B, x_small.shape[1], H) + tuple(x_small.shape[3:]), dtype=x_small.dtype, device=DEV)
    for i, (b, h) in enumerate(heads):
        big[b, :, h] = x_small[0, :, i].to(DEV)
    return big


def _spread_state(s_small, B, H, heads):
    big = torch.zeros((B, H) + tuple(s_small.shape[2:]), dtype=s_small.dtype, device=DEV)
    for i, (b, h) in enumerate(heads):
        big[b, h] = s_small[0, i].to(DEV)
    return big


def _compare(got, refs, heads, states=(), tol=None, terms=None):
    """got: name -> [B,T,H,D] device tensor; refs: name -> oracle [1,T,n,D];
    states: (name, device [B,H,K,V], oracle [1,n,K,V]).  terms: name ->
    [n, T] magnitudes of the terms a per-token value sums (see the scalar gate),
    which then replace the reference as the per-chunk scale."""
    errs, worst = {}, {}
    for name, x in got.items():
        xs = np.stack([to_np(x[b, :, h]) for b, h in heads])
        rs = np.stack([refs[name][0, :, i] for i in range(len(heads))])
        if xs.ndim == 2:  # a scalar gate's gradient [B,T,H]: one column
            xs, rs = xs[..., None], rs[..., None]
        errs[name] = rel_l2(xs, rs)
        if terms and name in terms:
            n_, T_ = terms[name].shape
            num = np.linalg.norm((xs - rs).reshape(n_, T_ // 64, -1), axis=2)
            den = np.linalg.norm(terms[name].reshape(n_, T_ // 64, 64), axis=2)
            note("  %s: worst 64-token chunk %.3e against the reference, %.3e against its terms" % (
                name, chunk_rel_l2(xs, rs), float((num / den).max())))
            worst[name] = float((num / den).max())
        else:
            worst[name] = chunk_rel_l2(xs, rs)
    for name, x, r in states:
        errs[name] = rel_l2(np.stack([to_np(x[b, h]) for b, h in heads]), r[0])
    note("  rel-L2 " + " ".join("%s=%.3e" % kv for kv in errs.items()) + " (tol %.0e)" % tol)
    note("  worst 64-token chunk " + " ".join("%s=%.3e" % kv for kv in worst.items()))
    assert all(v <= tol for v in errs.values()), errs
    assert all(v <= tol for v in worst.values()), worst
    for name, x in list(got.items()) + [(n, x) for n, x, _ in states]:
        assert bool(torch.isfinite(x).all()), name


def _zero_heads(tensors, states, B, H):
    for b, h in ((0, 1), (B - 1, 0), (0, H - 1), (B - 1, H // 2)):
        for name, x in tensors.items():
            assert not bool(x[b, :, h].any()), (name, b, h)
        for name, x in states.items():
            assert not bool(x[b, h].any()), (name, b, h)


CASES = [
    # form, B, H, T, K, V, dtype
    ("plain", 2, 2048, 16384, 64, 64, "bf16"),     # q, k, g, v, o: 2^32 elements each
    ("plain", 2, 1040, 16384, 64, 64, "fp32"),     # 2.18e9 elements (8.7 GB) each
    ("scalar", 2, 2048, 16384, 64, 64, "bf16"),
    ("general", 2, 520, 16384, 128, 128, "bf16"),  # 2.18e9 elements each
    ("wide_fwd", 2, 512, 16384, 256, 512, "bf16"),  # q, k, g 2^32, v and o 2^33 elements; records
    ("decode", 2, 65600, 3, 128, 128, "bf16"),     # the state: 2.15e9 fp32 elements
]


@pytest.mark.parametrize("form,B,H,T,K,V,dtype", CASES)
def test_past_32bit_offsets(form, B, H, T, K, V, dtype):
    free, _ = torch.cuda.mem_get_info(0)
    if free < 120 * 2 ** 30:
        pytest.skip("needs about 120 GiB of free device memory (%.0f GiB free)" % (free / 2 ** 30))
    heads = [(0, 0), (B - 1, H - 1)]
    n = len(heads)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tol = TOL[dt]
    note("large-offset parity (%s): B=%d H=%d T=%d K=%d V=%d %s, data in heads %s" % (form, B, H, T, K, V, dtype,
                                                                                      heads))
    gate = "scalar" if form == "scalar" else "iid"
    s0 = "normal0.1" if form in ("decode", "wide_fwd") else "none"
    w = gi.custom(1, n, T, K, V, dtype=dtype, gate=gate, s0=s0, backward=form not in ("decode", "wide_fwd"),
                  seed=4242 + K + V + T)
    sm = gi.make_inputs(w)
    f64 = lambda name: to_np(sm[name])
    d = {name: _spread(sm[name], B, H, heads) for name in ("q", "k", "v", "g") + (("do",) if "do" in sm else ())}
    s0_big = _spread_state(sm["s0"], B, H, heads) if sm.get("s0") is not None else None
    s0_np = to_np(sm["s0"]) if sm.get("s0") is not None else None
    try:
        if form == "plain":
            o, sf = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"])
            dq, dk, dv, dg, ds0 = gla.gla_bwd(d["q"], d["k"], d["v"], d["g"], d["do"])
            torch.cuda.synchronize()
            o_r, s_r = oracle.gla_fwd(f64("q"), f64("k"), f64("v"), f64("g"), None)
            r = oracle.gla_bwd(f64("q"), f64("k"), f64("v"), f64("g"), f64("do"), None, None)
            got = {"o": o, "dq": dq, "dk": dk, "dv": dv, "dg": dg}
            refs = {"o": o_r, "dq": r[0], "dk": r[1], "dv": r[2], "dg": r[3]}
            _compare(got, refs, heads, (("S_T", sf, s_r), ("ds0", ds0, r[4])), tol)
            _zero_heads(got, {"S_T": sf, "ds0": ds0}, B, H)
        elif form == "scalar":
            o, sf = gla.gla_fwd_scalar(d["q"], d["k"], d["v"], d["g"])
            dq, dk, dv, dg, ds0 = gla.gla_bwd_scalar(d["q"], d["k"], d["v"], d["g"], d["do"])
            torch.cuda.synchronize()
            o_r, s_r = oracle.gla_fwd_scalar(f64("q"), f64("k"), f64("v"), f64("g"), None)
            r = oracle.gla_bwd_scalar(f64("q"), f64("k"), f64("v"), f64("g"), f64("do"), None, None)
            got = {"o": o, "dq": dq, "dk": dk, "dv": dv, "dg": dg}
            refs = {"o": o_r, "dq": r[0], "dk": r[1], "dv": r[2], "dg": r[3]}
            # the scalar gate's gradient is the sum over the K key columns of
            # the per-column gradient of the same gate repeated over K (the
            # oracle's per-column backward): those terms cancel, by 7x in a
            # median chunk and up to 14x here, so a chunk's error is measured
            # against the size of the terms it sums rather than of their sum
            per_col = oracle.gla_bwd(f64("q"), f64("k"), f64("v"), np.repeat(f64("g")[..., None], K, axis=3),
                                     f64("do"), None, None)[3]
            terms = {"dg": np.abs(per_col).sum(axis=3)[0].T}
            cancel = terms["dg"].reshape(n, -1, 64) ** 2
            cancel = np.sqrt(cancel.sum(2)) / np.linalg.norm(r[3][0].T.reshape(n, -1, 64), axis=2)
            note("  dg: the key columns' terms cancel by %.1fx (median chunk), %.1fx (largest)" % (
                float(np.median(cancel)), float(cancel.max())))
            _compare(got, refs, heads, (("S_T", sf, s_r), ("ds0", ds0, r[4])), tol, terms)
            _zero_heads(got, {"S_T": sf, "ds0": ds0}, B, H)
        elif form == "general":
            h_sm = gi.make_value_gate(1, T, n, V, seed=4343)
            h_big = _spread(h_sm, B, H, heads)
            o, sf = gla.gla_fwd_general(d["q"], d["k"], d["v"], d["g"], h_big)
            torch.cuda.synchronize()
            o_r, s_r = oracle.gla_fwd_general(f64("q"), f64("k"), f64("v"), f64("g"), to_np(h_sm), None)
            _compare({"o": o}, {"o": o_r}, heads, (("S_T", sf, s_r),), tol)
            _zero_heads({"o": o}, {"S_T": sf}, B, H)
            del o, sf
            torch.cuda.empty_cache()
            dq, dk, dv, dg, dh, ds0 = gla.gla_bwd_general(d["q"], d["k"], d["v"], d["g"], h_big, d["do"])
            torch.cuda.synchronize()
            r = oracle.gla_bwd_general(f64("q"), f64("k"), f64("v"), f64("g"), to_np(h_sm), f64("do"), None, None)
            got = {"dq": dq, "dk": dk, "dv": dv, "dg": dg, "dh": dh}
            refs = {"dq": r[0], "dk": r[1], "dv": r[2], "dg": r[3], "dh": r[4]}
            _compare(got, refs, heads, (("ds0", ds0, r[5]),), tol)
            _zero_heads(got, {"ds0": ds0}, B, H)
        elif form == "wide_fwd":
            o, sf = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"], s0_big)
            torch.cuda.synchronize()
            o_r, s_r = oracle.gla_fwd(f64("q"), f64("k"), f64("v"), f64("g"), s0_np)
            _compare({"o": o}, {"o": o_r}, heads, (("S_T", sf, s_r),), tol)
            _zero_heads({"o": o}, {"S_T": sf}, B, H)
        else:  # decode: T tokens of the recurrence on a state of B*H*K*V > 2^31 elements
            state = s0_big.clone()
            o = gla.gla_decode(d["q"], d["k"], d["v"], d["g"], state)
            torch.cuda.synchronize()
            o_r, s_r = oracle.gla_fwd(f64("q"), f64("k"), f64("v"), f64("g"), s0_np)
            errs = {"o": rel_l2(np.stack([to_np(o[b, :, h]) for b, h in heads]),
                                np.stack([o_r[0, :, i] for i in range(n)])),
                    "state": rel_l2(np.stack([to_np(state[b, h]) for b, h in heads]), s_r[0])}
            note("  rel-L2 " + " ".join("%s=%.3e" % kv for kv in errs.items()) + " (tol %.0e)" % tol)
            assert all(v <= tol for v in errs.values()), errs
            assert bool(torch.isfinite(state).all()) and bool(torch.isfinite(o).all())
            _zero_heads({"o": o}, {"state": state}, B, H)
    finally:
        d.clear()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
