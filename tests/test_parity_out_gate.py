"""GPU parity of the GLA layer's output epilogue (per-head LayerNorm, scale and
shift, Swish output gate; Section 4.4 of the GLA paper) through the C ABI,
against the fp64 oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import chunkwise_linear_rnn_amd as gla
import gla_inputs as gi
import oracle
from tests.parity_util import TOL, note, rel_l2, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(B, T, H, V, dtype, eps, bias, seed, backward=True):
    inp = gi.make_gate_inputs(B, T, H, V, dtype, seed=seed, bias=bias)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    note("out_gate parity: B=%d T=%d H=%d V=%d %s eps=%g bias=%s" % (B, T, H, V, dtype, eps, bias))
    y = gla.gla_out_gate(d["o"], d["z"], d["ln_w"], d["ln_b"], eps)
    torch.cuda.synchronize()
    y_ref = oracle.out_gate(to_np(inp["o"]), to_np(inp["z"]), to_np(inp["ln_w"]), to_np(inp["ln_b"]), eps)
    tol = TOL[torch.float32 if dtype == "fp32" else torch.bfloat16]
    errs = {"y": rel_l2(to_np(y), y_ref)}
    if backward:
        dx, dz, dw, db = gla.gla_out_gate_bwd(d["o"], d["z"], d["ln_w"], d["ln_b"], eps, d["dy"])
        torch.cuda.synchronize()
        ref = oracle.out_gate_bwd(to_np(inp["o"]), to_np(inp["z"]), to_np(inp["ln_w"]), to_np(inp["ln_b"]), eps,
                                  to_np(inp["dy"]))
        errs.update(d_o=rel_l2(to_np(dx), ref[0]), dz=rel_l2(to_np(dz), ref[1]), dln_w=rel_l2(to_np(dw), ref[2]))
        if bias:
            errs["dln_b"] = rel_l2(to_np(db), ref[3])
        else:
            assert db is None
    note("  rel-L2 " + " ".join("%s=%.3e" % kv for kv in errs.items()) + " (tol %.0e)" % tol)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad
    return errs


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("V", [64, 128, 256, 512])
def test_out_gate_matches_oracle(dtype, V):
    # 1 x 7 x 3 = 21 rows: not a multiple of any workgroup's row count (ragged tail)
    _check(1, 7, 3, V, dtype, 1e-5, True, seed=V)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_out_gate_no_bias_and_many_rows(dtype):
    # 2 x 300 x 5 = 3000 rows: several workgroup passes, no shift
    _check(2, 300, 5, 256, dtype, 1e-6, False, seed=7)


def test_out_gate_large_eps_and_single_row():
    _check(1, 1, 1, 128, "bf16", 0.5, True, seed=8)


def test_out_gate_metric_size():
    # the metric workload's output (B=2, T=8192, H=4, V=256, bf16): 65536 rows, and
    # the backward's column sums reduce over all of them in a fixed order
    errs = _check(2, 8192, 4, 256, "bf16", 1e-5, True, seed=9)
    assert errs["dln_w"] < 1e-4 and errs["dln_b"] < 1e-4


def test_out_gate_empty_rows():
    o = torch.zeros(2, 0, 3, 64, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(64, device=DEV)
    b = torch.zeros(64, device=DEV)
    y = gla.gla_out_gate(o, o, w, b)
    assert y.shape == (2, 0, 3, 64)
    dx, dz, dw, db = gla.gla_out_gate_bwd(o, o, w, b, 1e-5, o)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw) == 0 and torch.count_nonzero(db) == 0


def test_out_gate_bwd_deterministic():
    inp = gi.make_gate_inputs(2, 512, 4, 256, "bf16", seed=10, device=DEV)
    r1 = gla.gla_out_gate_bwd(inp["o"], inp["z"], inp["ln_w"], inp["ln_b"], 1e-5, inp["dy"])
    r2 = gla.gla_out_gate_bwd(inp["o"], inp["z"], inp["ln_w"], inp["ln_b"], 1e-5, inp["dy"])
    torch.cuda.synchronize()
    assert all(torch.equal(a, c) for a, c in zip(r1, r2))
