"""Second, independent CPU forms of the GLA operator used to pin the oracle.

Every function here is a *different* formula from the oracle's token loop, each
written from its own passage of "Gated Linear Attention Transformers with
Hardware-Efficient Training" (and, for the scalar-decay mask, "Lightning
Attention-2"); none imports the oracle or the GPU library.  All are fp64 numpy
(or fp64 torch for autograd) on a single head: q, k, g are [T, K], v is [T, V],
states are [K, V].
"""
from __future__ import annotations

import numpy as np


def parallel_form(q, k, v, g, s0=None):
    """Brute-force parallel form, Section 4.1, Eq. 4 (log-space P) plus the S_0 term.

    o_t = (q_t * b_t) S_0 + sum_{s<=t} (sum_i q_ti k_si exp(logb_ti - logb_si)) v_s
    S_T = Diag(b_T) S_0 + sum_s Diag(b_T / b_s) k_s^T v_s
    with logb_t = sum_{r<=t} g_r (b_t = prod_{j<=t} alpha_j, Section 4.1).
    The S_0 terms come from unrolling Eq. 3 down to S_0.
    """
    T, K = q.shape
    V = v.shape[1]
    logb = np.cumsum(g, axis=0)
    o = np.zeros((T, V))
    for t in range(T):
        for s in range(t + 1):
            p = np.sum(q[t] * k[s] * np.exp(logb[t] - logb[s]))
            o[t] += p * v[s]
    sT = np.zeros((K, V))
    for s in range(T):
        sT += np.outer(k[s] * np.exp(logb[T - 1] - logb[s]), v[s])
    if s0 is not None:
        for t in range(T):
            o[t] += (q[t] * np.exp(logb[t])) @ s0
        if T > 0:
            sT += np.exp(logb[T - 1])[:, None] * s0
        else:
            sT += s0
    return o, sT


def causal_linear_attention(q, k, v, s0=None):
    """Ungated case, Section 2.1, Eq. 1 parallel form: O = ((Q K^T) * M) V (+ Q S_0)."""
    T = q.shape[0]
    M = np.tril(np.ones((T, T)))
    o = ((q @ k.T) * M) @ v
    if s0 is not None:
        o = o + q @ s0
    return o


def scalar_decay_form(q, k, v, gamma):
    """Scalar gate g_t[i] = gamma_t for every i: O = ((Q K^T) * D * M) V with
    D_ts = exp(sum_{r=s+1}^{t} gamma_r).  For constant gamma = log(lambda) this is
    the decay mask M_ts = lambda^(t-s) of Lightning Attention-2 (Section 3.2.1).
    """
    T = q.shape[0]
    cg = np.cumsum(gamma)
    D = np.exp(cg[:, None] - cg[None, :])
    M = np.tril(np.ones((T, T)))
    return ((q @ k.T) * D * M) @ v


def chunkwise_form(q, k, v, g, s0=None, C=64, c=16):
    """Chunkwise form with secondary chunking, written from Section 4.2 (Lambda,
    Gamma, gamma; inter-chunk state recurrence and O_inter = (Q*Lambda) S) and
    Section 4.3 / the chapter summary's Knowl 3 (sub-chunks of size c; pairs of
    different sub-chunks through a reference row of the query sub-chunk; pairs
    inside a sub-chunk element-wise in log space).

    Returns (o, s_final, states) where states[n] is the state before chunk n.
    The last chunk may be shorter than C (ragged tail).
    """
    T, K = q.shape
    V = v.shape[1]
    S = np.zeros((K, V)) if s0 is None else s0.copy()
    o = np.zeros((T, V))
    states = []
    for start in range(0, T, C):
        end = min(start + C, T)
        qc, kc, vc, gc = q[start:end], k[start:end], v[start:end], g[start:end]
        L = end - start
        Bc = np.cumsum(gc, axis=0)              # intra-chunk log b_t / b_{iC}
        lam = np.exp(Bc)                        # Lambda
        gam_rows = np.exp(Bc[-1][None, :] - Bc)  # Gamma
        gam = np.exp(Bc[-1])                    # gamma
        states.append(S.copy())
        o_inter = (qc * lam) @ S
        P = np.zeros((L, L))
        for i0 in range(0, L, c):
            i1 = min(i0 + c, L)
            # intra-sub-chunk: Eq. 4 element by element
            for t in range(i0, i1):
                for s in range(i0, t + 1):
                    P[t, s] = np.sum(qc[t] * kc[s] * np.exp(Bc[t] - Bc[s]))
            # inter-sub-chunk: reference = first row of the query sub-chunk
            z = Bc[i0]
            qs = qc[i0:i1] * np.exp(Bc[i0:i1] - z)
            for j0 in range(0, i0, c):
                j1 = min(j0 + c, i0)
                ks = kc[j0:j1] * np.exp(z - Bc[j0:j1])
                P[i0:i1, j0:j1] = qs @ ks.T
        o[start:end] = o_inter + P @ vc
        S = gam[:, None] * S + (kc * gam_rows).T @ vc
    return o, S, states


def torch_parallel_loss(q, k, v, g, s0, d_o, dht):
    """fp64 torch graph of the Eq. 4 parallel form and the S_T closed form, for autograd.

    Inputs are float64 torch tensors with requires_grad set by the caller.
    Returns the scalar <o, do> + <S_T, dht>.
    """
    import torch
    T = q.shape[0]
    logb = torch.cumsum(g, dim=0)
    diff = logb[:, None, :] - logb[None, :, :]              # [t, s, i]
    mask = torch.tril(torch.ones(T, T, dtype=torch.float64))
    # only s <= t is used; zero the exponent elsewhere so exp stays finite
    diff = torch.where(mask[:, :, None] > 0, diff, torch.zeros_like(diff))
    P = torch.einsum("ti,si,tsi->ts", q, k, torch.exp(diff)) * mask
    o = P @ v + (q * torch.exp(logb)) @ s0
    sT = (k * torch.exp(logb[-1][None, :] - logb)).T @ v + torch.exp(logb[-1])[:, None] * s0
    return (o * d_o).sum() + (sT * dht).sum()
