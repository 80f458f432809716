"""Pins of the general-gate oracle (alpha^T beta forget gate) against forms that
share no code with its token recurrence ("Gated Linear Attention Transformers
with Hardware-Efficient Training", the chapter summary's Knowl 12 and
Appendix C)."""
import numpy as np
import pytest

import oracle


def _inputs(B, T, H, K, V, seed, scale=1.0, s0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, K)) / np.sqrt(K)
    k = rng.standard_normal((B, T, H, K)) / np.sqrt(K)
    v = rng.standard_normal((B, T, H, V))
    g = -np.log1p(np.exp(-rng.standard_normal((B, T, H, K)))) * scale  # logsigmoid
    h = -np.log1p(np.exp(-rng.standard_normal((B, T, H, V)))) * scale
    st = rng.standard_normal((B, H, K, V)) * 0.1 if s0 else None
    return q, k, v, g, h, st


def _brute(q, k, v, g, h, s0):
    # o_t[j] = sum_{s<=t} sum_i q_ti k_si v_sj prod_{r=s+1..t} alpha_ri beta_rj
    #        + sum_i q_ti S0_ij prod_{r<=t} alpha_ri beta_rj
    B, T, H, K = q.shape
    V = v.shape[-1]
    o = np.zeros((B, T, H, V))
    sf = np.zeros((B, H, K, V))
    for b in range(B):
        for hh in range(H):
            for t in range(T):
                for j in range(V):
                    acc = 0.0
                    for i in range(K):
                        for s in range(t + 1):
                            decay = np.exp(g[b, s + 1:t + 1, hh, i].sum() + h[b, s + 1:t + 1, hh, j].sum())
                            acc += q[b, t, hh, i] * k[b, s, hh, i] * v[b, s, hh, j] * decay
                        if s0 is not None:
                            acc += q[b, t, hh, i] * s0[b, hh, i, j] * np.exp(g[b, :t + 1, hh, i].sum() + h[b, :t + 1, hh, j].sum())
                    o[b, t, hh, j] = acc
            for i in range(K):
                for j in range(V):
                    acc = 0.0
                    for s in range(T):
                        acc += k[b, s, hh, i] * v[b, s, hh, j] * np.exp(g[b, s + 1:, hh, i].sum() + h[b, s + 1:, hh, j].sum())
                    if s0 is not None:
                        acc += s0[b, hh, i, j] * np.exp(g[b, :, hh, i].sum() + h[b, :, hh, j].sum())
                    sf[b, hh, i, j] = acc
    return o, sf


def test_general_matches_brute_force():
    q, k, v, g, h, s0 = _inputs(1, 7, 2, 3, 4, seed=1)
    o, sf = oracle.gla_fwd_general(q, k, v, g, h, s0)
    ob, sb = _brute(q, k, v, g, h, s0)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sf, sb, rtol=1e-12, atol=1e-13)


def test_general_matches_pages_parallel_form():
    # Q~ = Q*B, K~ = K/B, V~ = V/D, O = (((Q~ K~^T) * M) V~) * D with b_t, d_t the
    # running products of alpha and beta (zero initial state, mild gates)
    q, k, v, g, h, _ = _inputs(2, 12, 1, 5, 6, seed=2, scale=0.25, s0=False)
    o, _ = oracle.gla_fwd_general(q, k, v, g, h)
    for b in range(2):
        Bm = np.exp(np.cumsum(g[b, :, 0], axis=0))
        Dm = np.exp(np.cumsum(h[b, :, 0], axis=0))
        Qt, Kt, Vt = q[b, :, 0] * Bm, k[b, :, 0] / Bm, v[b, :, 0] / Dm
        M = np.tril(np.ones((12, 12)))
        ref = ((Qt @ Kt.T) * M) @ Vt * Dm
        np.testing.assert_allclose(o[b, :, 0], ref, rtol=1e-10, atol=1e-12)


def test_general_reduces_to_gla_when_beta_is_one():
    q, k, v, g, h, s0 = _inputs(2, 40, 2, 8, 16, seed=3)
    o, sf = oracle.gla_fwd_general(q, k, v, g, np.zeros_like(h), s0)
    og, sg = oracle.gla_fwd(q, k, v, g, s0)
    np.testing.assert_allclose(o, og, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sf, sg, rtol=1e-13, atol=1e-14)


def test_general_key_and_value_roles_swap_under_transposition():
    # with alpha = 1 the state's transpose follows a key-gated recurrence with v
    # as key and k as value; o_t = q_t S_t then equals (S_t^T q_t^T)^T: check the
    # final state against the GLA oracle run on the transposed problem
    q, k, v, g, h, s0 = _inputs(1, 30, 2, 6, 5, seed=4)
    _, sf = oracle.gla_fwd_general(q, k, v, np.zeros_like(g), h, s0)
    _, sT = oracle.gla_fwd(v, v, k, h, np.swapaxes(s0, -1, -2))
    np.testing.assert_allclose(sf, np.swapaxes(sT, -1, -2), rtol=1e-12, atol=1e-13)
