"""Pins of the oracle's GLA output epilogue (per-head LayerNorm, Swish output
gate; "Gated Linear Attention Transformers with Hardware-Efficient Training",
Section 4.4) against library routines, calculus and invariants."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import gla_inputs as gi
import oracle


def _rand(R, V, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((R, V)), r.standard_normal((R, V)), 1.0 + 0.3 * r.standard_normal(V),
            0.3 * r.standard_normal(V), r.standard_normal((R, V)))


def _torch_ref(o, z, w, b, eps):
    t = lambda a: None if a is None else torch.from_numpy(np.asarray(a, dtype=np.float64))
    V = o.shape[-1]
    return (F.layer_norm(t(o), (V,), t(w), t(b), eps) * F.silu(t(z))).numpy()


@pytest.mark.parametrize("V,eps,bias", [(4, 1e-5, True), (64, 1e-6, False), (256, 1e-3, True)])
def test_forward_matches_torch_float64(V, eps, bias):
    o, z, w, b, _ = _rand(7, V, seed=V)
    b = b if bias else None
    y = oracle.out_gate(o, z, w, b, eps)
    assert np.allclose(y, _torch_ref(o, z, w, b, eps), rtol=1e-12, atol=1e-13)


def test_shift_invariance_and_constant_rows():
    o, z, w, b, _ = _rand(5, 32, seed=1)
    shift = np.arange(5, dtype=np.float64)[:, None] * 3.0 - 4.0
    assert np.allclose(oracle.out_gate(o + shift, z, w, b, 1e-5), oracle.out_gate(o, z, w, b, 1e-5),
                       rtol=1e-10, atol=1e-12)
    # a constant row normalises to zero: y = b * Swish(z)
    c = np.full((2, 32), 0.7)
    zc = z[:2]
    # (the row mean of a repeated 0.7 carries fp64 rounding, scaled by 1/sqrt(eps))
    assert np.allclose(oracle.out_gate(c, zc, w, b, 1e-5), b * zc / (1 + np.exp(-zc)), rtol=1e-12, atol=1e-11)


def test_unit_moments_without_affine():
    # with w = 1, b = 0 and eps = 0, y / Swish(z) has zero mean and unit (biased) variance per row
    o, z, _, _, _ = _rand(6, 48, seed=2)
    y = oracle.out_gate(o, z, np.ones(48), None, 0.0)
    n = y / (z / (1 + np.exp(-z)))
    assert np.allclose(n.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose((n ** 2).mean(axis=1), 1.0, rtol=1e-12)


def test_backward_matches_torch_autograd_float64():
    o, z, w, b, dy = _rand(9, 16, seed=3)
    to = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    O, Z, W, Bv = to(o), to(z), to(w), to(b)
    y = F.layer_norm(O, (16,), W, Bv, 1e-4) * F.silu(Z)
    (y * torch.from_numpy(dy)).sum().backward()
    dx, dz, dw, db = oracle.out_gate_bwd(o, z, w, b, 1e-4, dy)
    for got, ref in ((dx, O.grad), (dz, Z.grad), (dw, W.grad), (db, Bv.grad)):
        assert np.allclose(got, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_backward_central_finite_differences():
    o, z, w, b, dy = _rand(3, 5, seed=4)
    eps, h = 1e-3, 1e-6
    loss = lambda o_, z_, w_, b_: float((oracle.out_gate(o_, z_, w_, b_, eps) * dy).sum())
    dx, dz, dw, db = oracle.out_gate_bwd(o, z, w, b, eps, dy)
    for name, arr, grad in (("o", o, dx), ("z", z, dz), ("w", w, dw), ("b", b, db)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            args = {"o": o, "z": z, "w": w, "b": b}
            args[name] = p
            lp = loss(args["o"], args["z"], args["w"], args["b"])
            args[name] = m
            lm = loss(args["o"], args["z"], args["w"], args["b"])
            fd[idx] = (lp - lm) / (2 * h)
        assert np.allclose(grad, fd, rtol=1e-6, atol=1e-8), name


def test_gate_inputs_are_seeded():
    a = gi.make_gate_inputs(1, 3, 2, 64, "bf16", seed=5)
    c = gi.make_gate_inputs(1, 3, 2, 64, "bf16", seed=5)
    assert all(torch.equal(a[k], c[k]) for k in a if a[k] is not None)
    assert a["o"].dtype == torch.bfloat16 and a["ln_w"].dtype == torch.float32
