"""Pins of the oracle's scalar-gate functions (one log gate per token and head,
the scalar-decay case of Eq. 3 of the GLA paper) against the quadratic
decay-mask form, finite differences and torch float64 autograd."""
import numpy as np
import torch

import gla_inputs as gi
import oracle


def _mask_form(q, k, v, g, s0):
    """O = ((Q K^T) * D * M) V + (Q * b_t) S_0, D_ts = exp(sum_{r=s+1..t} g_r), per head (torch fp64)."""
    B, T, H, K = q.shape
    cg = torch.cumsum(g, dim=1)  # [B,T,H]
    outs = []
    for h in range(H):
        qh, kh, vh, ch = q[:, :, h], k[:, :, h], v[:, :, h], cg[:, :, h]
        D = torch.exp(ch[:, :, None] - ch[:, None, :])
        M = torch.tril(torch.ones(T, T, dtype=torch.float64))
        A = (qh @ kh.transpose(1, 2)) * D * M
        o = A @ vh
        if s0 is not None:
            o = o + (qh * torch.exp(ch)[..., None]) @ s0[:, h]
        outs.append(o)
    return torch.stack(outs, dim=2)


def _rand(B, T, H, K, V, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, T, H, K)) / 2, r.standard_normal((B, T, H, K)) / 2, r.standard_normal((B, T, H, V)),
            -np.abs(r.standard_normal((B, T, H))) / 3, r.standard_normal((B, H, K, V)) / 3,
            r.standard_normal((B, T, H, V)))


def test_forward_equals_decay_mask_form():
    q, k, v, g, s0, _ = _rand(2, 37, 2, 5, 3, seed=1)
    o, sf = oracle.gla_fwd_scalar(q, k, v, g, s0)
    t = lambda a: torch.from_numpy(a)
    ref = _mask_form(t(q), t(k), t(v), t(g), t(s0)).numpy()
    assert np.allclose(o, ref, rtol=1e-11, atol=1e-12)
    # the final state: S_T = b_T S_0 + sum_s (b_T / b_s) k_s^T v_s
    cg = np.cumsum(g, axis=1)
    w = np.exp(cg[:, -1:, :] - cg)  # [B,T,H]
    sf_ref = np.exp(cg[:, -1])[:, :, None, None] * s0 + np.einsum("bth,bthi,bthj->bhij", w, k, v)
    assert np.allclose(sf, sf_ref, rtol=1e-11, atol=1e-12)


def test_backward_matches_autograd_of_decay_mask_form():
    q, k, v, g, s0, do = _rand(1, 23, 2, 4, 3, seed=2)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    Q, Kt, Vt, G, S0 = T(q), T(k), T(v), T(g), T(s0)
    (_mask_form(Q, Kt, Vt, G, S0) * torch.from_numpy(do)).sum().backward()
    dq, dk, dv, dg, ds0 = oracle.gla_bwd_scalar(q, k, v, g, do, s0, None)
    for got, ref in ((dq, Q.grad), (dk, Kt.grad), (dv, Vt.grad), (dg, G.grad), (ds0, S0.grad)):
        assert np.allclose(got, ref.numpy(), rtol=1e-9, atol=1e-10)


def test_scalar_gate_gradient_central_differences():
    q, k, v, g, s0, do = _rand(1, 6, 1, 3, 2, seed=3)
    dht = np.random.default_rng(4).standard_normal((1, 1, 3, 2))
    loss = lambda gg: float((oracle.gla_fwd_scalar(q, k, v, gg, s0)[0] * do).sum() +
                            (oracle.gla_fwd_scalar(q, k, v, gg, s0)[1] * dht).sum())
    dg = oracle.gla_bwd_scalar(q, k, v, g, do, s0, dht)[3]
    h = 1e-6
    fd = np.zeros_like(g)
    for idx in np.ndindex(g.shape):
        p, m = g.copy(), g.copy()
        p[idx] += h
        m[idx] -= h
        fd[idx] = (loss(p) - loss(m)) / (2 * h)
    assert np.allclose(dg, fd, rtol=1e-6, atol=1e-8)


def test_scalar_inputs_shape():
    w = gi.custom(1, 2, 64, 64, 64, dtype="bf16", gate="scalar", seed=5)
    inp = gi.make_inputs(w)
    assert inp["g"].shape == (1, 64, 2) and float(inp["g"].max()) <= 0.0
