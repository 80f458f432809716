"""Pins of the general-gate oracle's backward (gradients of <o, do> + <S_T, dht>
through S_t = (exp(g_t)^T exp(h_t)) * S_{t-1} + k_t^T v_t; "Gated Linear
Attention Transformers with Hardware-Efficient Training", the chapter summary's
Knowl 12 and Appendix C) against forms that share no code with its chain rule."""
import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_general import _inputs


def _loss(q, k, v, g, h, s0, do, dht):
    o, sf = oracle.gla_fwd_general(q, k, v, g, h, s0)
    return float((o * do).sum() + (sf * dht).sum())


def _case(T, seed, B=1, H=2, K=3, V=2):
    q, k, v, g, h, s0 = _inputs(B, T, H, K, V, seed=seed)
    rng = np.random.default_rng(seed + 100)
    do = rng.standard_normal((B, T, H, V))
    dht = rng.standard_normal((B, H, K, V))
    return q, k, v, g, h, s0, do, dht


@pytest.mark.parametrize("T", [1, 3, 17, 130])
def test_general_bwd_central_differences(T):
    q, k, v, g, h, s0, do, dht = _case(T, seed=40 + T)
    grads = oracle.gla_bwd_general(q, k, v, g, h, do, s0, dht)
    args = [q, k, v, g, h, s0]
    rng = np.random.default_rng(T)
    eps = 1e-6
    for a, ga in zip(args, grads[:5] + (grads[5],)):
        flat = a.reshape(-1)
        idx = range(flat.size) if flat.size <= 60 else rng.choice(flat.size, 60, replace=False)
        for n in idx:
            old = flat[n]
            flat[n] = old + eps
            lp = _loss(*args, do, dht)
            flat[n] = old - eps
            lm = _loss(*args, do, dht)
            flat[n] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - ga.reshape(-1)[n]) <= 1e-6 * (1 + abs(fd)), (n, fd, ga.reshape(-1)[n])


def test_general_bwd_matches_autograd_of_pages_parallel_form():
    # O = (((Q*B)(K/B)^T) * M)(V/D) * D with B, D the cumulative products of the
    # gates (no initial state, no final-state gradient): torch fp64 autograd
    q, k, v, g, h, _ = _inputs(2, 12, 2, 4, 3, seed=7)
    rng = np.random.default_rng(8)
    do = rng.standard_normal(v.shape)
    tq, tk, tv, tg, th = (torch.tensor(x, requires_grad=True) for x in (q, k, v, g, h))
    Bc = torch.exp(torch.cumsum(tg, dim=1))
    Dc = torch.exp(torch.cumsum(th, dim=1))
    Qt = (tq * Bc).permute(0, 2, 1, 3)
    Kt = (tk / Bc).permute(0, 2, 1, 3)
    Vt = (tv / Dc).permute(0, 2, 1, 3)
    T = q.shape[1]
    M = torch.tril(torch.ones(T, T, dtype=torch.float64))
    O = (((Qt @ Kt.transpose(-1, -2)) * M) @ Vt).permute(0, 2, 1, 3) * Dc
    (O * torch.tensor(do)).sum().backward()
    dq, dk, dv, dg, dh, _ = oracle.gla_bwd_general(q, k, v, g, h, do)
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad), (dg, tg.grad), (dh, th.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-9, atol=1e-11)


def test_general_bwd_zero_value_gate_reduces_to_gla_bwd():
    q, k, v, g, h, s0, do, dht = _case(70, seed=9, K=4, V=3)
    h = np.zeros_like(h)
    dq, dk, dv, dg, dh, ds0 = oracle.gla_bwd_general(q, k, v, g, h, do, s0, dht)
    rq, rk, rv, rg, rs0 = oracle.gla_bwd(q, k, v, g, do, s0, dht)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv), (dg, rg), (ds0, rs0)):
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_general_bwd_closed_form_gate_gradients():
    # dg_t = sum_{s>=t} (q_s dq_s - k_s dk_s) + sum_j S_T[i,j] dht[i,j]
    # dh_t = sum_{s>=t} (o_s do_s - v_s dv_s) + sum_i S_T[i,j] dht[i,j]
    q, k, v, g, h, s0, do, dht = _case(150, seed=11, K=4, V=5)
    dq, dk, dv, dg, dh, _ = oracle.gla_bwd_general(q, k, v, g, h, do, s0, dht)
    o, sf = oracle.gla_fwd_general(q, k, v, g, h, s0)
    rc = lambda x: np.flip(np.cumsum(np.flip(x, 1), 1), 1)
    fg = rc(q * dq - k * dk) + (sf * dht).sum(-1)[:, None]
    fh = rc(o * do - v * dv) + (sf * dht).sum(-2)[:, None]
    np.testing.assert_allclose(dg, fg, rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(dh, fh, rtol=1e-9, atol=1e-10)
