"""GPU check of gla_fwd_noalloc (the forward for callers that cannot allocate):
through the C ABI, its outputs equal gla_fwd's with a caller workspace, bit for
bit (the same kernels on the same inputs), on two calls in a row whose second
input is smaller, so the fixed scratch is reused with a different layout."""
import pytest
import torch

import chunkwise_linear_rnn_amd as gla
import gla_inputs as gi
from tests.parity_util import note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both(w):
    d = gi.make_inputs(w, device=DEV)
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    ws_bytes = gla.gla_fwd_workspace_size(B, T, H, K, V, w.torch_dtype)
    assert 0 < ws_bytes <= 32 << 20, ws_bytes   # several segments: the scratch is used
    o_ref, s_ref = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"], d["s0"])
    o = torch.full_like(o_ref, float("nan"))
    sf = torch.full_like(s_ref, float("nan"))
    gla.gla_fwd_noalloc_into(d["q"], d["k"], d["v"], d["g"], d["s0"], o, sf)
    torch.cuda.synchronize()
    return o, sf, o_ref, s_ref


def test_fwd_noalloc_matches_gla_fwd_twice():
    cases = [gi.custom(2, 4, 8192, 128, 256, dtype="bf16", gate="lowrank", s0="normal0.1", backward=False, seed=61),
             gi.custom(1, 2, 512, 64, 64, dtype="bf16", gate="iid", s0="normal0.1", backward=False, seed=62)]
    for w in cases:
        note("noalloc fwd: B=%d H=%d T=%d K=%d V=%d %s" % (w.B, w.H, w.T, w.K, w.V, w.dtype))
        o, sf, o_ref, s_ref = _both(w)
        assert torch.equal(o, o_ref)
        assert torch.equal(sf, s_ref)


def test_fwd_noalloc_fp32_and_no_final_state():
    w = gi.custom(1, 3, 320, 64, 128, dtype="fp32", gate="iid", backward=False, seed=63)
    d = gi.make_inputs(w, device=DEV)
    o_ref, _ = gla.gla_fwd(d["q"], d["k"], d["v"], d["g"], None)
    o = torch.empty_like(o_ref)
    gla.gla_fwd_noalloc_into(d["q"], d["k"], d["v"], d["g"], None, o, None)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
