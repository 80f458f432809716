"""Pins for the oracle's forward pass (CPU only).

Each test checks the fp64 token-by-token recurrence against something other
than itself: a hand-derived fixture, the brute-force parallel form (Eq. 4), the
ungated textbook form (Eq. 1), the scalar-decay mask form, the chunkwise form
at many chunk and sub-chunk sizes, state passing across segments, and
linearity / permutation properties.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests import forms

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _rand_case(rng, B, T, H, K, V, gate_scale=1.0, s0=True):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    # log-sigmoid gates in (-inf, 0): alpha in (0, 1) as the gate definition requires
    x = rng.standard_normal((B, T, H, K)) * gate_scale
    g = -np.log1p(np.exp(-x))
    S0 = rng.standard_normal((B, H, K, V)) if s0 else None
    return q, k, v, g, S0


def _head(a, b, h):
    return a[b, :, h, :]


def test_golden_hand_examples():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        B, T, H, K, V = c["B"], c["T"], c["H"], c["K"], c["V"]
        q = np.array(c["q"], dtype=np.float64).reshape(B, T, H, K)
        k = np.array(c["k"], dtype=np.float64).reshape(B, T, H, K)
        v = np.array(c["v"], dtype=np.float64).reshape(B, T, H, V)
        g = np.log(np.array(c["alpha"], dtype=np.float64)).reshape(B, T, H, K)
        s0 = np.array(c["s0"], dtype=np.float64).reshape(B, H, K, V)
        o, sf = oracle.gla_fwd(q, k, v, g, s0)
        np.testing.assert_allclose(o.ravel(), np.array(c["o"], dtype=np.float64).ravel(), rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(sf.ravel(), np.array(c["s_final"], dtype=np.float64).ravel(), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("T,K,V", [(1, 3, 4), (2, 4, 3), (17, 5, 7), (64, 8, 4), (130, 6, 5)])
def test_matches_parallel_form_eq4(T, K, V):
    rng = np.random.default_rng(1000 + T)
    B, H = 2, 3
    q, k, v, g, S0 = _rand_case(rng, B, T, H, K, V)
    o, sf = oracle.gla_fwd(q, k, v, g, S0)
    for b in range(B):
        for h in range(H):
            o_ref, s_ref = forms.parallel_form(_head(q, b, h), _head(k, b, h), _head(v, b, h), _head(g, b, h), S0[b, h])
            np.testing.assert_allclose(o[b, :, h, :], o_ref, rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(sf[b, h], s_ref, rtol=1e-11, atol=1e-11)


def test_zero_state_and_no_state_agree():
    rng = np.random.default_rng(7)
    q, k, v, g, _ = _rand_case(rng, 1, 9, 2, 3, 4, s0=False)
    o1, s1 = oracle.gla_fwd(q, k, v, g, None)
    o2, s2 = oracle.gla_fwd(q, k, v, g, np.zeros((1, 2, 3, 4)))
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_ungated_reduces_to_causal_linear_attention():
    # g = 0 means alpha = 1: Eq. 1, O = ((Q K^T) * M) V (+ Q S_0 for a nonzero S_0)
    rng = np.random.default_rng(11)
    B, T, H, K, V = 2, 40, 2, 6, 5
    q, k, v, _, S0 = _rand_case(rng, B, T, H, K, V)
    g = np.zeros((B, T, H, K))
    o, sf = oracle.gla_fwd(q, k, v, g, S0)
    for b in range(B):
        for h in range(H):
            ref = forms.causal_linear_attention(_head(q, b, h), _head(k, b, h), _head(v, b, h), S0[b, h])
            np.testing.assert_allclose(o[b, :, h, :], ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(sf[b, h], S0[b, h] + _head(k, b, h).T @ _head(v, b, h), rtol=1e-12, atol=1e-12)


def test_scalar_gate_decay_mask():
    rng = np.random.default_rng(12)
    T, K, V = 33, 4, 3
    q = rng.standard_normal((1, T, 1, K)); k = rng.standard_normal((1, T, 1, K)); v = rng.standard_normal((1, T, 1, V))
    gamma = -np.abs(rng.standard_normal(T)) * 0.3
    g = np.repeat(gamma[None, :, None, None], K, axis=3)
    o, _ = oracle.gla_fwd(q, k, v, g)
    ref = forms.scalar_decay_form(q[0, :, 0], k[0, :, 0], v[0, :, 0], gamma)
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=1e-12, atol=1e-12)
    # constant decay lambda: mask lambda^(t-s) (Lightning Attention-2's M_ij)
    lam = 0.9
    g2 = np.full((1, T, 1, K), np.log(lam))
    o2, _ = oracle.gla_fwd(q, k, v, g2)
    tt = np.arange(T)
    Mlam = np.where(tt[:, None] >= tt[None, :], lam ** (tt[:, None] - tt[None, :]).clip(min=0), 0.0)
    ref2 = ((q[0, :, 0] @ k[0, :, 0].T) * Mlam) @ v[0, :, 0]
    np.testing.assert_allclose(o2[0, :, 0], ref2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("C,c", [(1, 1), (2, 1), (8, 4), (16, 4), (16, 16), (64, 16), (64, 1), (200, 16)])
def test_chunk_size_invariance(C, c):
    # Section 2.2: C = 1 is the recurrent form, C = L the parallel form; every C in between is exact.
    rng = np.random.default_rng(13)
    T, K, V = 130, 5, 6  # ragged: 130 is not a multiple of 8, 16 or 64
    q, k, v, g, S0 = _rand_case(rng, 1, T, 1, K, V, gate_scale=2.0)
    o, sf = oracle.gla_fwd(q, k, v, g, S0)
    o_c, s_c, _ = forms.chunkwise_form(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], S0[0, 0], C=C, c=c)
    np.testing.assert_allclose(o[0, :, 0], o_c, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(sf[0, 0], s_c, rtol=1e-11, atol=1e-11)


def test_segment_invariance_state_passing():
    # S_0 carried over from an earlier segment (Section 2.2): running T1 then T-T1 equals running T.
    rng = np.random.default_rng(14)
    B, T, H, K, V = 2, 100, 2, 4, 3
    q, k, v, g, S0 = _rand_case(rng, B, T, H, K, V)
    o, sf = oracle.gla_fwd(q, k, v, g, S0)
    for T1 in (1, 37, 64, 99):
        oa, sa = oracle.gla_fwd(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], S0)
        ob, sb = oracle.gla_fwd(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], sa)
        assert np.array_equal(np.concatenate([oa, ob], axis=1), o)
        assert np.array_equal(sb, sf)


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(15)
    S0 = rng.standard_normal((2, 3, 4, 5))
    z = np.zeros((2, 0, 3, 4)); zv = np.zeros((2, 0, 3, 5))
    o, sf = oracle.gla_fwd(z, z, zv, z, S0)
    assert o.shape == (2, 0, 3, 5)
    assert np.array_equal(sf, S0)


def test_linearity_and_permutation():
    rng = np.random.default_rng(16)
    B, T, H, K, V = 2, 20, 3, 4, 5
    q, k, v, g, S0 = _rand_case(rng, B, T, H, K, V)
    _, _, v2, _, S02 = _rand_case(rng, B, T, H, K, V)
    a, c = 0.7, -1.3
    o1, s1 = oracle.gla_fwd(q, k, v, g, S0)
    o2, s2 = oracle.gla_fwd(q, k, v2, g, S02)
    o3, s3 = oracle.gla_fwd(q, k, a * v + c * v2, g, a * S0 + c * S02)
    np.testing.assert_allclose(o3, a * o1 + c * o2, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s3, a * s1 + c * s2, rtol=1e-11, atol=1e-11)
    o4, _ = oracle.gla_fwd(2.5 * q, k, v, g, S0)
    np.testing.assert_allclose(o4, 2.5 * o1, rtol=1e-12, atol=1e-12)
    # heads and batch are independent (Section 4.4): permuting them permutes the outputs
    hp = [2, 0, 1]
    o5, s5 = oracle.gla_fwd(q[::-1][:, :, hp], k[::-1][:, :, hp], v[::-1][:, :, hp], g[::-1][:, :, hp], S0[::-1][:, hp])
    assert np.array_equal(o5, o1[::-1][:, :, hp])
    assert np.array_equal(s5, s1[::-1][:, hp])
