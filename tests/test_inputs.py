"""The seeded input generator is deterministic and honours each recipe."""
import torch

import gla_inputs as gi


def test_deterministic_and_shapes():
    w = gi.custom(2, 3, 128, 64, 32, dtype="bf16", gate="lowrank", s0="normal0.1", seed=9)
    a = gi.make_inputs(w, dht=True)
    b = gi.make_inputs(w, dht=True)
    for key in ("q", "k", "v", "g", "s0", "do", "dht"):
        assert torch.equal(a[key], b[key]), key
    assert a["q"].shape == (2, 128, 3, 64) and a["v"].shape == (2, 128, 3, 32)
    assert a["s0"].shape == (2, 3, 64, 32) and a["s0"].dtype == torch.float32
    assert a["q"].dtype == torch.bfloat16


def test_gate_recipes():
    for gate in ("iid", "lowrank"):
        x = gi.make_inputs(gi.custom(1, 2, 256, 64, 64, gate=gate, seed=3))
        g = x["g"].float()
        assert (g <= 0).all() and (g > -2).all()
    z = gi.make_inputs(gi.custom(1, 2, 64, 64, 64, gate="zero", seed=3))
    assert (z["g"] == 0).all()


def test_named_workloads_cover_the_configs():
    names = set(gi.WORKLOADS)
    assert {"tiny_fp32", "ungated_1k", "gla_340m", "gla_1p3b_long", "fwdbwd_16k", "metric_8k"} <= names
    m = gi.WORKLOADS["metric_8k"]
    assert (m.B, m.H, m.T, m.K, m.V, m.dtype) == (2, 4, 8192, 128, 256, "bf16")
