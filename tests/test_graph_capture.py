"""The training pairs under HIP graph capture.

gla_fwd_ckpt + gla_bwd_ckpt (and the scalar- and general-gate pairs) only
enqueue kernels on the caller's stream (no
allocation, no memset, no host synchronisation), so a step can be captured
once and replayed.  Each replay here follows eager work on the same buffers
(outputs poisoned with NaN, inputs rewritten) and must reproduce, bit for bit,
what the eager calls give for the inputs present at replay time.
"""
import pytest
import torch

import chunkwise_linear_rnn_amd as gla
import gla_inputs as gi
from tests.parity_util import note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _buffers(B, T, H, K, V, dt, scalar):
    dev = DEV
    out = {
        "o": torch.empty(B, T, H, V, dtype=dt, device=dev),
        "sf": torch.empty(B, H, K, V, dtype=torch.float32, device=dev),
        "dq": torch.empty(B, T, H, K, dtype=dt, device=dev),
        "dk": torch.empty(B, T, H, K, dtype=dt, device=dev),
        "dv": torch.empty(B, T, H, V, dtype=dt, device=dev),
        "dg": torch.empty(*((B, T, H) if scalar else (B, T, H, K)), dtype=dt, device=dev),
        "ds0": torch.empty(B, H, K, V, dtype=torch.float32, device=dev),
    }
    ck = gla.workspace(gla.gla_ckpt_size(B, T, H, K, V, dt), dev)
    wsf = gla.workspace((gla.gla_fwd_scalar_workspace_size if scalar else gla.gla_fwd_workspace_size)(
        B, T, H, K, V, dt), dev)
    wsb = gla.workspace((gla.gla_bwd_scalar_workspace_size if scalar else gla.gla_bwd_workspace_size)(
        B, T, H, K, V, dt), dev)
    return out, ck, wsf, wsb


def _step(d, out, ck, wsf, wsb, scalar):
    gla.gla_fwd_ckpt_into(d["q"], d["k"], d["v"], d["g"], d["s0"], out["o"], out["sf"], ck, wsf,
                          scalar_gate=scalar)
    gla.gla_bwd_ckpt_into(d["q"], d["k"], d["v"], d["g"], d["s0"], ck, d["do"], d["dht"], out["dq"], out["dk"],
                          out["dv"], out["dg"], out["ds0"], wsb, scalar_gate=scalar)


@pytest.mark.parametrize("scalar", [False, True])
def test_training_pair_graph_replays(scalar):
    B, H, T, K, V = 1, 4, 64 * 24, 128, 256
    w = gi.custom(B, H, T, K, V, dtype="bf16", gate="scalar" if scalar else "lowrank", s0="normal0.1",
                  backward=True, seed=900 + int(scalar))
    d = gi.make_inputs(w, device=DEV, dht=True)
    assert gla.gla_ckpt_size(B, T, H, K, V, torch.bfloat16) > 0
    out, ck, wsf, wsb = _buffers(B, T, H, K, V, torch.bfloat16, scalar)

    # warm up on a side stream (as torch asks before capture), then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(d, out, ck, wsf, wsb, scalar)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(d, out, ck, wsf, wsb, scalar)
    torch.cuda.synchronize()

    for rep in range(3):
        # new inputs in place (the graph reads the buffers it was captured on)
        fresh = gi.make_inputs(gi.custom(B, H, T, K, V, dtype="bf16", gate="scalar" if scalar else "lowrank",
                                         s0="normal0.1", backward=True, seed=910 + rep), device=DEV, dht=True)
        for name in ("q", "k", "v", "g", "do", "s0", "dht"):
            d[name].copy_(fresh[name])
        # eager reference for these inputs, on separate outputs
        ref, ck_r, wsf_r, wsb_r = _buffers(B, T, H, K, V, torch.bfloat16, scalar)
        _step(d, ref, ck_r, wsf_r, wsb_r, scalar)
        torch.cuda.synchronize()
        for t in out.values():
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        same = {name: torch.equal(out[name], ref[name]) for name in out}
        note("graph replay %d (scalar gate %s): %s" % (rep, scalar, same))
        assert all(same.values()), same


def test_general_training_pair_graph_replays():
    # the general-gate pair (alpha^T beta gates): forward with checkpoint, then
    # the backward from the forward's o and checkpoint, captured and replayed
    B, H, T, K, V = 1, 4, 64 * 24, 128, 256
    dev, dt = DEV, torch.bfloat16

    def inputs(seed):
        w = gi.custom(B, H, T, K, V, dtype="bf16", gate="lowrank", s0="normal0.1", backward=True, seed=seed)
        d = gi.make_inputs(w, device=dev, dht=True)
        d["h"] = gi.make_value_gate(B, T, H, V, seed=seed + 1).to(dev)
        return d

    def buffers():
        out = {"o": torch.empty(B, T, H, V, dtype=dt, device=dev),
               "sf": torch.empty(B, H, K, V, dtype=torch.float32, device=dev),
               "dq": torch.empty(B, T, H, K, dtype=dt, device=dev), "dk": torch.empty(B, T, H, K, dtype=dt, device=dev),
               "dv": torch.empty(B, T, H, V, dtype=dt, device=dev), "dg": torch.empty(B, T, H, K, dtype=dt, device=dev),
               "dh": torch.empty(B, T, H, V, dtype=dt, device=dev),
               "ds0": torch.empty(B, H, K, V, dtype=torch.float32, device=dev)}
        ck = gla.workspace(gla.gla_general_ckpt_size(B, T, H, K, V, dt), dev)
        wsf = gla.workspace(gla.gla_fwd_general_workspace_size(B, T, H, K, V, dt), dev)
        wsb = gla.workspace(gla.gla_bwd_general_workspace_size(B, T, H, K, V, dt), dev)
        return out, ck, wsf, wsb

    def step(d, out, ck, wsf, wsb):
        gla.gla_fwd_general_ckpt_into(d["q"], d["k"], d["v"], d["g"], d["h"], d["s0"], out["o"], out["sf"], ck, wsf)
        gla.gla_bwd_general_ckpt_into(d["q"], d["k"], d["v"], d["g"], d["h"], d["s0"], out["o"], ck, d["do"], d["dht"],
                                      out["dq"], out["dk"], out["dv"], out["dg"], out["dh"], out["ds0"], wsb)

    d = inputs(930)
    assert gla.gla_general_ckpt_size(B, T, H, K, V, dt) > 0
    out, ck, wsf, wsb = buffers()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(d, out, ck, wsf, wsb)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(d, out, ck, wsf, wsb)
    torch.cuda.synchronize()
    for rep in range(3):
        fresh = inputs(940 + 2 * rep)
        for name in ("q", "k", "v", "g", "h", "do", "s0", "dht"):
            d[name].copy_(fresh[name])
        ref, ck_r, wsf_r, wsb_r = buffers()
        step(d, ref, ck_r, wsf_r, wsb_r)
        torch.cuda.synchronize()
        for t in out.values():
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        same = {name: torch.equal(out[name], ref[name]) for name in out}
        note("general graph replay %d: %s" % (rep, same))
        assert all(same.values()), same
