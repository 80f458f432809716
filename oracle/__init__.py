"""CPU fp64 oracle for gated linear attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library
(``chunkwise_linear_rnn_amd``) never imports it and it never imports the
product; the two share no code.

The arithmetic lives in ``gla_oracle.c`` (plain C, fp64, the token-by-token
recurrence of "Gated Linear Attention Transformers with Hardware-Efficient
Training", Section 4.1, Eq. 3, and its reverse-mode gradient).  This module
only builds that file with gcc and marshals numpy arrays to it.

Parity status of each function is recorded in its docstring; both are pinned by
the ``-m "not gpu"`` tests (``tests/test_oracle_*.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


SAN_LIB_PATH = os.path.join(_HERE, "liboracle_hostsan.so")


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile ``gla_oracle.c`` into ``liboracle.so`` with gcc (fp64, no fast-math).
    sanitize: ``liboracle_hostsan.so`` instead, with AddressSanitizer and
    UndefinedBehaviorSanitizer (load it with GLA_ORACLE_LIBRARY in a process
    that preloads the sanitizer runtime)."""
    out = SAN_LIB_PATH if sanitize else _LIB_PATH
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(_SRC):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           "-std=c99", "-o", tmp, _SRC, "-lm"]
    if sanitize:
        cmd[1:1] = ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("GLA_ORACLE_LIBRARY")
    if not path:
        path = _LIB_PATH
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    L = ctypes.c_long
    lib.oracle_gla_fwd.argtypes = [L, L, L, L, L, dp, dp, dp, dp, dp, dp, dp]
    lib.oracle_gla_fwd.restype = ctypes.c_int
    lib.oracle_gla_bwd.argtypes = [L, L, L, L, L, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp]
    lib.oracle_gla_bwd.restype = ctypes.c_int
    lib.oracle_gla_fwd_general.argtypes = [L, L, L, L, L, dp, dp, dp, dp, dp, dp, dp, dp]
    lib.oracle_gla_fwd_general.restype = ctypes.c_int
    lib.oracle_gla_bwd_general.argtypes = [L, L, L, L, L] + [dp] * 14
    lib.oracle_gla_bwd_general.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    D = ctypes.c_double
    lib.oracle_out_gate_fwd.argtypes = [L, L, dp, dp, dp, dp, D, dp]
    lib.oracle_out_gate_fwd.restype = ctypes.c_int
    lib.oracle_out_gate_bwd.argtypes = [L, L, dp, dp, dp, dp, D, dp, dp, dp, dp, dp]
    lib.oracle_out_gate_bwd.restype = ctypes.c_int
    _lib = lib
    return lib


def _as_f64(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor -> exact upcast on the CPU
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    """Threads the OpenMP runtime of the oracle will use (OMP_NUM_THREADS)."""
    return int(_load().oracle_num_threads())


def gla_fwd(q, k, v, g, s0=None) -> Tuple[np.ndarray, np.ndarray]:
    """Forward recurrence in fp64: returns (o [B,T,H,V], s_final [B,H,K,V]).

    Follows "Gated Linear Attention Transformers with Hardware-Efficient
    Training", Section 4.1, Eq. 3 (S_t = Diag(exp g_t) S_{t-1} + k_t^T v_t,
    o_t = q_t S_t), with S_0 = s0 or zero (Section 2.2).
    Pinned by: brute-force Eq. 4 parallel form, the ungated Eq. 1 reduction,
    the scalar-gate decay-mask form, chunk-size invariance, segment invariance,
    linearity, and a hand-computed golden fixture.
    """
    q, k, v, g = (_as_f64(x) for x in (q, k, v, g))
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert k.shape == (B, T, H, K) and g.shape == (B, T, H, K) and v.shape == (B, T, H, V)
    s0 = _as_f64(s0)
    if s0 is not None:
        assert s0.shape == (B, H, K, V)
    o = np.zeros((B, T, H, V), dtype=np.float64)
    sf = np.zeros((B, H, K, V), dtype=np.float64)
    rc = _load().oracle_gla_fwd(B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0), _ptr(o), _ptr(sf))
    if rc != 0:
        raise RuntimeError("oracle_gla_fwd failed with code %d" % rc)
    return o, sf


def gla_fwd_general(q, k, v, g, h, s0=None) -> Tuple[np.ndarray, np.ndarray]:
    """General gated linear attention forward in fp64: (o [B,T,H,V], s_final).

    Follows "Gated Linear Attention Transformers with Hardware-Efficient
    Training", the chapter summary's Knowl 12 and Appendix C: the forget gate is
    the outer product alpha_t^T beta_t of a key-side gate alpha_t = exp(g_t)
    [B,T,H,K] and a value-side gate beta_t = exp(h_t) [B,T,H,V],
    S_t = (alpha_t^T beta_t) * S_{t-1} + k_t^T v_t, o_t = q_t S_t.
    Pinned by: the brute-force double-product form, the pages' parallel form
    O = (((Q*B)(K/B)^T) * M)(V/D) * D, its h = 0 reduction to gla_fwd, and the
    closed-form final state.
    """
    q, k, v, g, h = (_as_f64(x) for x in (q, k, v, g, h))
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert k.shape == (B, T, H, K) and g.shape == (B, T, H, K)
    assert v.shape == (B, T, H, V) and h.shape == (B, T, H, V)
    s0 = _as_f64(s0)
    if s0 is not None:
        assert s0.shape == (B, H, K, V)
    o = np.zeros((B, T, H, V), dtype=np.float64)
    sf = np.zeros((B, H, K, V), dtype=np.float64)
    rc = _load().oracle_gla_fwd_general(B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h), _ptr(s0),
                                        _ptr(o), _ptr(sf))
    if rc != 0:
        raise RuntimeError("oracle_gla_fwd_general failed with code %d" % rc)
    return o, sf


def gla_bwd(q, k, v, g, d_o, s0=None, dht=None):
    """Reverse-mode gradient of the fp64 recurrence for loss <o,do> + <S_T,dht>.

    Returns (dq, dk, dv, dg, ds0).  dg is the gradient with respect to the log
    gate g, taken through d(exp(g_t) S_{t-1})/dg_t -- independent of the
    paper's closed form (Section 4.3), which the tests check against it.
    Pinned by: central finite differences, torch float64 autograd of the
    parallel form (Eq. 4), the closed-form gate gradient, the closed-form
    dS_0, dg_1 = 0 when S_0 = 0, and a hand-computed T = 2 fixture.
    """
    q, k, v, g, d_o = (_as_f64(x) for x in (q, k, v, g, d_o))
    B, T, H, K = q.shape
    V = v.shape[-1]
    s0 = _as_f64(s0)
    dht = _as_f64(dht)
    dq = np.zeros((B, T, H, K)); dk = np.zeros((B, T, H, K)); dg = np.zeros((B, T, H, K))
    dv = np.zeros((B, T, H, V)); ds0 = np.zeros((B, H, K, V))
    rc = _load().oracle_gla_bwd(B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0), _ptr(d_o),
                                _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(ds0))
    if rc != 0:
        raise RuntimeError("oracle_gla_bwd failed with code %d" % rc)
    return dq, dk, dv, dg, ds0


def out_gate(o, z, w, b=None, eps=1e-5) -> np.ndarray:
    """GLA layer output epilogue in fp64: y = Swish(z) * (LN(o) * w + b), per row.

    Follows "Gated Linear Attention Transformers with Hardware-Efficient
    Training", Section 4.4: LayerNorm of each head's output row over its V
    channels (mean, biased variance, eps inside the square root), per-channel
    scale w and shift b shared by the heads, times r = Swish(z), z the gate's
    pre-activation.  o, z: [..., V]; w, b: [V].
    Pinned by: torch float64 layer_norm and silu (library routines), shift
    invariance, a constant row giving y = b * Swish(z), unit row moments with
    w = 1, b = 0.
    """
    o, z, w = _as_f64(o), _as_f64(z), _as_f64(w)
    b = _as_f64(b)
    V = o.shape[-1]
    assert z.shape == o.shape and w.shape == (V,) and (b is None or b.shape == (V,))
    R = o.size // V
    y = np.zeros_like(o)
    rc = _load().oracle_out_gate_fwd(R, V, _ptr(o), _ptr(z), _ptr(w), _ptr(b), float(eps), _ptr(y))
    if rc != 0:
        raise RuntimeError("oracle_out_gate_fwd failed with code %d" % rc)
    return y


def out_gate_bwd(o, z, w, b, eps, dy):
    """Reverse-mode gradient of <y, dy> for out_gate: (do, dz, dw, db), fp64.

    The chain rule taken step by step through the forward as written.  Pinned
    by: central finite differences and torch float64 autograd of layer_norm and
    silu.
    """
    o, z, w, dy = _as_f64(o), _as_f64(z), _as_f64(w), _as_f64(dy)
    b = _as_f64(b)
    V = o.shape[-1]
    R = o.size // V
    dx = np.zeros_like(o); dz = np.zeros_like(o); dw = np.zeros(V); db = np.zeros(V)
    rc = _load().oracle_out_gate_bwd(R, V, _ptr(o), _ptr(z), _ptr(w), _ptr(b), float(eps), _ptr(dy), _ptr(dx),
                                     _ptr(dz), _ptr(dw), _ptr(db))
    if rc != 0:
        raise RuntimeError("oracle_out_gate_bwd failed with code %d" % rc)
    return dx, dz, dw, db


def gla_fwd_scalar(q, k, v, g, s0=None) -> Tuple[np.ndarray, np.ndarray]:
    """Forward recurrence with a scalar gate per token and head, g [B,T,H].

    The scalar-decay case of Eq. 3 (alpha_t = exp(g_t) times the all-ones row):
    every key column of the state decays by the same factor, so this is
    gla_fwd with g broadcast over the K columns.  Pinned by: the quadratic
    decay-mask form O = ((Q K^T) * D * M) V + (Q * b_t) S_0 with
    D_ts = exp(g_{s+1} + ... + g_t), computed independently in the tests.
    """
    g = _as_f64(g)
    K = _as_f64(q).shape[-1]
    return gla_fwd(q, k, v, np.repeat(g[..., None], K, axis=-1), s0)


def gla_bwd_scalar(q, k, v, g, d_o, s0=None, dht=None):
    """Gradients for gla_fwd_scalar: (dq, dk, dv, dg [B,T,H], ds0).

    The chain rule through the broadcast: the scalar gate's gradient is the sum
    over key columns of the per-column gate gradient.  Pinned by: central finite
    differences in the scalar gate and torch float64 autograd of the decay-mask
    form.
    """
    g = _as_f64(g)
    K = _as_f64(q).shape[-1]
    dq, dk, dv, dg, ds0 = gla_bwd(q, k, v, np.repeat(g[..., None], K, axis=-1), d_o, s0, dht)
    return dq, dk, dv, dg.sum(axis=-1), ds0


def gla_bwd_general(q, k, v, g, h, d_o, s0=None, dht=None):
    """Reverse-mode gradient of gla_fwd_general (fp64) for the loss
    <o, d_o> + <S_T, dht>: returns (dq, dk, dv, dg, dh, ds0), dg and dh with
    respect to the log gates g (key side) and h (value side).  The chain rule
    through S_t = (exp(g_t)^T exp(h_t)) * S_{t-1} + k_t^T v_t, token by token
    ("Gated Linear Attention Transformers with Hardware-Efficient Training", the
    chapter summary's Knowl 12 and Appendix C), with states replayed from
    checkpoints.  Pinned by central finite differences, torch fp64 autograd of the
    pages' parallel form, the h = 0 reduction to gla_bwd and the pages' closed forms
    of the two gate gradients.
    """
    q, k, v, g, h, d_o = (_as_f64(x) for x in (q, k, v, g, h, d_o))
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert k.shape == (B, T, H, K) and g.shape == (B, T, H, K)
    assert v.shape == (B, T, H, V) and h.shape == (B, T, H, V) and d_o.shape == (B, T, H, V)
    s0, dht = _as_f64(s0), _as_f64(dht)
    dq = np.zeros_like(q); dk = np.zeros_like(k); dg = np.zeros_like(g)
    dv = np.zeros_like(v); dh = np.zeros_like(h)
    ds0 = np.zeros((B, H, K, V), dtype=np.float64)
    rc = _load().oracle_gla_bwd_general(B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h), _ptr(s0),
                                        _ptr(d_o), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dh),
                                        _ptr(ds0))
    if rc != 0:
        raise RuntimeError("oracle_gla_bwd_general failed with code %d" % rc)
    return dq, dk, dv, dg, dh, ds0
