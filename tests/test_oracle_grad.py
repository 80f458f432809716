"""Pins for the oracle's backward pass (CPU only).

The oracle differentiates the recurrence through the state (dg from dS and
S_{t-1}); these tests check it against central finite differences of the
forward, against torch float64 autograd of the parallel form (Eq. 4), against
the paper's closed-form gate gradient (Section 4.3) and the closed-form dS_0,
and against hand-derived values.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests import forms

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _rand_case(rng, B, T, H, K, V, s0=True, dht=True):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    x = rng.standard_normal((B, T, H, K))
    g = -np.log1p(np.exp(-x))
    S0 = rng.standard_normal((B, H, K, V)) if s0 else None
    do = rng.standard_normal((B, T, H, V))
    dh = rng.standard_normal((B, H, K, V)) if dht else None
    return q, k, v, g, S0, do, dh


def _loss(q, k, v, g, S0, do, dh):
    o, sf = oracle.gla_fwd(q, k, v, g, S0)
    L = float(np.sum(o * do))
    if dh is not None:
        L += float(np.sum(sf * dh))
    return L


def test_golden_hand_examples():
    for c in json.load(open(GOLDEN))["cases"]:
        B, T, H, K, V = c["B"], c["T"], c["H"], c["K"], c["V"]
        arr = lambda key, *shape: np.array(c[key], dtype=np.float64).reshape(*shape)
        q, k = arr("q", B, T, H, K), arr("k", B, T, H, K)
        v = arr("v", B, T, H, V)
        g = np.log(arr("alpha", B, T, H, K))
        s0, dht = arr("s0", B, H, K, V), arr("dht", B, H, K, V)
        do = arr("do", B, T, H, V)
        dq, dk, dv, dg, ds0 = oracle.gla_bwd(q, k, v, g, do, s0, dht)
        for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg), ("ds0", ds0)):
            np.testing.assert_allclose(got.ravel(), np.array(c[name], dtype=np.float64).ravel(),
                                       rtol=1e-14, atol=1e-14, err_msg=name)


@pytest.mark.parametrize("T", [1, 2, 3, 17, 130])
def test_finite_differences(T):
    rng = np.random.default_rng(2000 + T)
    B, H, K, V = 1, 2, 3, 4
    q, k, v, g, S0, do, dh = _rand_case(rng, B, T, H, K, V)
    dq, dk, dv, dg, ds0 = oracle.gla_bwd(q, k, v, g, do, S0, dh)
    eps = 1e-6
    args = [q, k, v, g, S0]
    grads = [dq, dk, dv, dg, ds0]
    for ai, (x, gx) in enumerate(zip(args, grads)):
        flat = x.reshape(-1)
        # probe a deterministic subset of entries (all of them for tiny T)
        idx = np.arange(flat.size) if flat.size <= 64 else rng.choice(flat.size, 48, replace=False)
        for j in idx:
            orig = flat[j]
            flat[j] = orig + eps
            lp = _loss(*args, do, dh)
            flat[j] = orig - eps
            lm = _loss(*args, do, dh)
            flat[j] = orig
            fd = (lp - lm) / (2 * eps)
            an = gx.reshape(-1)[j]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (ai, j, fd, an)


def test_torch_autograd_of_parallel_form():
    import torch
    rng = np.random.default_rng(21)
    T, K, V = 70, 5, 3
    q, k, v, g, S0, do, dh = _rand_case(rng, 1, T, 1, K, V)
    dq, dk, dv, dg, ds0 = oracle.gla_bwd(q, k, v, g, do, S0, dh)
    ts = [torch.tensor(a[0, :, 0].copy(), dtype=torch.float64, requires_grad=True) for a in (q, k, v, g)]
    s0t = torch.tensor(S0[0, 0], dtype=torch.float64, requires_grad=True)
    L = forms.torch_parallel_loss(*ts, s0t, torch.tensor(do[0, :, 0]), torch.tensor(dh[0, 0]))
    L.backward()
    for got, t in zip((dq, dk, dv, dg), ts):
        np.testing.assert_allclose(got[0, :, 0], t.grad.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(ds0[0, 0], s0t.grad.numpy(), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("with_s0,with_dht", [(False, False), (True, False), (False, True), (True, True)])
def test_closed_form_gate_gradient(with_s0, with_dht):
    # Section 4.3: dlog b_t = q_t*dq_t - k_t*dk_t, dlog alpha_t = sum_{i>=t} dlog b_i; the final-state
    # gradient adds sum_j S_T[i,j] dht[i,j] to dlog b_T and hence to every dg_t.
    rng = np.random.default_rng(22)
    B, T, H, K, V = 2, 150, 2, 4, 6
    q, k, v, g, S0, do, dh = _rand_case(rng, B, T, H, K, V, s0=with_s0, dht=with_dht)
    dq, dk, dv, dg, ds0 = oracle.gla_bwd(q, k, v, g, do, S0, dh)
    dA = q * dq - k * dk
    dg_cf = np.flip(np.cumsum(np.flip(dA, axis=1), axis=1), axis=1)
    if with_dht:
        _, sf = oracle.gla_fwd(q, k, v, g, S0)
        dg_cf = dg_cf + np.sum(sf * dh, axis=-1)[:, None, :, :]
    np.testing.assert_allclose(dg, dg_cf, rtol=1e-9, atol=1e-9)
    if not with_s0:
        # alpha_1 only scales S_0, so dg_1 vanishes exactly without an initial state
        assert np.all(dg[:, 0] == 0.0)


def test_closed_form_ds0():
    # dS_0 = Diag(b_T) dht + sum_t Diag(b_t) q_t^T do_t  (unrolling Eq. 3)
    rng = np.random.default_rng(23)
    B, T, H, K, V = 1, 45, 2, 3, 5
    q, k, v, g, S0, do, dh = _rand_case(rng, B, T, H, K, V)
    *_, ds0 = oracle.gla_bwd(q, k, v, g, do, S0, dh)
    for h in range(H):
        logb = np.cumsum(g[0, :, h], axis=0)
        ref = np.exp(logb[-1])[:, None] * dh[0, h]
        for t in range(T):
            ref += np.outer(np.exp(logb[t]) * q[0, t, h], do[0, t, h])
        np.testing.assert_allclose(ds0[0, h], ref, rtol=1e-11, atol=1e-11)


def test_checkpoint_boundaries_consistent():
    # T spanning several 64-token recompute segments must give the same gradients as
    # the closed forms on a ragged length.
    rng = np.random.default_rng(24)
    B, T, H, K, V = 1, 193, 1, 2, 3
    q, k, v, g, S0, do, dh = _rand_case(rng, B, T, H, K, V)
    dq, dk, dv, dg, ds0 = oracle.gla_bwd(q, k, v, g, do, S0, dh)
    # dv_s = sum_{t>=s} A_ts do_t + (k_s * b_T/b_s) dht, A from Eq. 4
    logb = np.cumsum(g[0, :, 0], axis=0)
    for s in (0, 63, 64, 127, 128, 192):
        acc = np.exp(logb[-1] - logb[s]) * k[0, s, 0] @ dh[0, 0]
        for t in range(s, T):
            a_ts = np.sum(q[0, t, 0] * k[0, s, 0] * np.exp(logb[t] - logb[s]))
            acc = acc + a_ts * do[0, t, 0]
        np.testing.assert_allclose(dv[0, s, 0], acc, rtol=1e-10, atol=1e-10)
