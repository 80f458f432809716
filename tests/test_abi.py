"""C-ABI contract checks that need no GPU.

The library must load without a device, export every symbol include/gla.h
declares, and reject every invalid argument with its status code before making
any HIP call (the pointers used below are never dereferenced).
"""
import ctypes
import os
import re

import pytest

import chunkwise_linear_rnn_amd as gla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP = range(7)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gla.LIB_PATH):
        from chunkwise_linear_rnn_amd import build
        build.build()
    return gla.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gla_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert set(declared) == set(gla.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert L.gla_abi_version() == 1


def test_status_strings_total(L):
    for code in range(-1, 9):
        s = L.gla_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0


def _shape(B=2, T=128, H=3, K=64, V=64, chunk=64, dtype=gla.GLA_DTYPE_BF16, reserved=0):
    return gla.GlaShape(B, T, H, K, V, chunk, dtype, reserved)


P = ctypes.c_void_p(0x10000)  # aligned fake device pointer: validation never dereferences it


def _fwd(L, shape, q=P, k=P, v=P, g=P, s0=None, o=P, sf=None, ws=P, wsb=1 << 40):
    return L.gla_fwd(ctypes.byref(shape) if shape is not None else None, q, k, v, g, s0, o, sf, ws, wsb, None)


def _bwd(L, shape, dq=P, ws=P, wsb=1 << 40, dht=None):
    return L.gla_bwd(ctypes.byref(shape), P, P, P, P, None, P, dht, dq, P, P, P, None, ws, wsb, None)


def test_validation_codes(L):
    assert _fwd(L, None) == ERR_NULL
    assert _fwd(L, _shape(), q=None) == ERR_NULL
    assert _fwd(L, _shape(B=-1)) == ERR_SHAPE
    assert _fwd(L, _shape(K=0)) == ERR_SHAPE
    assert _fwd(L, _shape(T=100)) == ERR_SHAPE
    assert _fwd(L, _shape(chunk=32)) == ERR_UNSUPPORTED
    assert _fwd(L, _shape(K=96)) == ERR_UNSUPPORTED
    assert _fwd(L, _shape(V=1024)) == ERR_UNSUPPORTED
    assert _fwd(L, _shape(dtype=7)) == ERR_UNSUPPORTED
    assert _fwd(L, _shape(K=1024, dtype=gla.GLA_DTYPE_FP32)) == ERR_UNSUPPORTED
    assert _fwd(L, _shape(K=1024)) == ERR_UNSUPPORTED
    assert _fwd(L, _shape(reserved=1)) == ERR_UNSUPPORTED
    assert _fwd(L, _shape(), k=ctypes.c_void_p(0x10008)) == ERR_ALIGN
    assert _fwd(L, _shape(), s0=ctypes.c_void_p(0x10004)) == ERR_ALIGN
    assert b"16-byte" in L.gla_last_error_detail()
    big = _shape(B=1, H=1, T=64 * 64)
    need = L.gla_fwd_workspace_size(ctypes.byref(big))
    if need > 0:
        assert _fwd(L, big, wsb=need - 1) == ERR_WORKSPACE
        assert _fwd(L, big, ws=None, wsb=need) == ERR_WORKSPACE
    assert _bwd(L, _shape(), dq=None) == ERR_NULL
    assert _bwd(L, _shape(T=65)) == ERR_SHAPE
    need_b = L.gla_bwd_workspace_size(ctypes.byref(_shape()))
    assert need_b > 0
    assert _bwd(L, _shape(), wsb=need_b - 1) == ERR_WORKSPACE


def test_workspace_sizes(L):
    # invalid shapes report 0; sizes are a pure function of the shape
    assert L.gla_fwd_workspace_size(ctypes.byref(_shape(T=100))) == 0
    s = _shape(B=2, H=4, T=8192, K=128, V=256)
    a = L.gla_fwd_workspace_size(ctypes.byref(s))
    b = L.gla_fwd_workspace_size(ctypes.byref(s))
    assert a == b and a % 4 == 0
    # per-segment states dominate: at least one [K, V] state per head when segmented
    assert a == 0 or a >= 2 * 4 * 128 * 256 * 4
    bw = L.gla_bwd_workspace_size(ctypes.byref(s))
    assert bw >= 2 * 2 * 4 * 128 * 256 * 4
    # 16-bit heads with dk = 256 also hold one prepared-operand record per chunk
    # and head (Ql, Kt^T, A: 2*64*256 + 64*64 two-byte values, gate factors)
    wide = _shape(B=2, H=4, T=8192, K=256, V=512)
    records = 2 * 4 * (8192 // 64) * (2 * 2 * 64 * 256 + 2 * 64 * 64)
    assert L.gla_fwd_workspace_size(ctypes.byref(wide)) >= records
    one = _shape(B=1, H=1, T=64, K=256, V=64)  # a single segment still needs its record
    assert L.gla_fwd_workspace_size(ctypes.byref(one)) >= 2 * 2 * 64 * 256 + 2 * 64 * 64


def _dec(L, shape, q=P, k=P, v=P, g=P, state=P, o=P):
    return L.gla_decode(ctypes.byref(shape) if shape is not None else None, q, k, v, g, state, o, None)


def test_size_limits(L):
    # past each documented limit the shape check rejects the call before
    # anything else; just inside it the (pure) size functions accept the shape
    ok = lambda sh: L.gla_bwd_workspace_size(ctypes.byref(sh)) > 0
    assert _fwd(L, _shape(B=(1 << 20) + 1, H=1, T=64)) == ERR_SHAPE
    assert b"heads" in L.gla_last_error_detail()
    assert ok(_shape(B=1 << 20, H=1, T=64))
    assert _fwd(L, _shape(B=1, H=1, T=1 << 30)) == ERR_SHAPE
    assert b"token-heads" in L.gla_last_error_detail()
    assert ok(_shape(B=1, H=1, T=(1 << 30) - 64))
    assert _bwd(L, _shape(B=1, H=1 << 16, T=64, K=512, V=64)) == ERR_SHAPE
    assert b"H*max(K,V)" in L.gla_last_error_detail()
    assert ok(_shape(B=1, H=(1 << 16) - 1, T=64, K=512, V=64))
    assert _dec(L, _shape(B=1 << 24, H=1, T=1, V=64)) == ERR_SHAPE
    assert _dec(L, _shape(B=1 << 22, H=1, T=1, V=256)) == ERR_SHAPE
    assert b"workgroups" in L.gla_last_error_detail()


def test_decode_validation_codes(L):
    # the recurrent form takes any T (no chunk constraint) and needs the state
    assert _dec(L, None) == ERR_NULL
    assert _dec(L, _shape(T=0)) == OK
    assert _dec(L, _shape(B=0, T=5)) == OK
    assert _dec(L, _shape(T=5), state=None) == ERR_NULL
    assert _dec(L, _shape(T=5), o=None) == ERR_NULL
    assert _dec(L, _shape(T=-1)) == ERR_SHAPE
    assert _dec(L, _shape(T=5, K=96)) == ERR_UNSUPPORTED
    assert _dec(L, _shape(T=5, K=1024)) == ERR_UNSUPPORTED
    assert _dec(L, _shape(T=5, V=1024)) == ERR_UNSUPPORTED
    assert _dec(L, _shape(T=5, dtype=7)) == ERR_UNSUPPORTED
    assert _dec(L, _shape(T=5, reserved=1)) == ERR_UNSUPPORTED
    assert _dec(L, _shape(T=5), state=ctypes.c_void_p(0x10004)) == ERR_ALIGN
    assert b"state" in L.gla_last_error_detail()
    # the scalar- and general-gate forms validate the same way; h is required
    sc = lambda shape, **kw: L.gla_decode_scalar(ctypes.byref(shape), P, P, P, kw.get("g", P), kw.get("state", P),
                                                 P, None)
    ge = lambda shape, **kw: L.gla_decode_general(ctypes.byref(shape), P, P, P, P, kw.get("h", P),
                                                  kw.get("state", P), P, None)
    assert sc(_shape(T=0)) == OK and ge(_shape(T=0)) == OK
    assert sc(_shape(T=5), g=None) == ERR_NULL
    assert sc(_shape(T=5, K=96)) == ERR_UNSUPPORTED
    assert ge(_shape(T=5), h=None) == ERR_NULL
    assert ge(_shape(T=5), h=ctypes.c_void_p(0x10002)) == ERR_ALIGN
    assert b"h" in L.gla_last_error_detail()
    assert ge(_shape(T=5, V=1024)) == ERR_UNSUPPORTED


def _gate(L, shape, o=P, z=P, w=P, b=None, eps=1e-5, y=P):
    return L.gla_out_gate(ctypes.byref(shape) if shape is not None else None, o, z, w, b, eps, y, None)


def _gate_bwd(L, shape, o=P, z=P, w=P, b=None, eps=1e-5, dy=P, dx=P, dz=P, dw=P, db=None, ws=P, wsb=1 << 30):
    return L.gla_out_gate_bwd(ctypes.byref(shape) if shape is not None else None, o, z, w, b, eps, dy, dx, dz, dw,
                              db, ws, wsb, None)


def test_out_gate_validation_codes(L):
    # rows of V channels; K and chunk are not used, T need not be a multiple of 64
    assert _gate(L, None) == ERR_NULL
    assert _gate(L, _shape(T=0)) == OK
    assert _gate(L, _shape(B=0, T=5, chunk=7, K=3)) == OK
    assert _gate(L, _shape(T=5), z=None) == ERR_NULL
    assert _gate(L, _shape(T=5), w=None) == ERR_NULL
    assert _gate(L, _shape(T=-1)) == ERR_SHAPE
    assert _gate(L, _shape(T=5, V=96)) == ERR_UNSUPPORTED
    assert _gate(L, _shape(T=5, dtype=7)) == ERR_UNSUPPORTED
    assert _gate(L, _shape(T=5), eps=-1.0) == ERR_UNSUPPORTED
    assert _gate(L, _shape(T=5), eps=float("nan")) == ERR_UNSUPPORTED
    assert _gate(L, _shape(T=5), y=ctypes.c_void_p(0x10008)) == ERR_ALIGN
    assert b"y" in L.gla_last_error_detail()
    # backward: inputs, outputs and the workspace are checked before any launch
    ws = L.gla_out_gate_bwd_workspace_size(ctypes.byref(_shape(T=5, V=256)))
    assert ws >= 2 * 256 * 256 * 4
    assert L.gla_out_gate_bwd_workspace_size(ctypes.byref(_shape(T=5, V=96))) == 0
    assert _gate_bwd(L, _shape(T=0), dw=None) == OK
    assert _gate_bwd(L, _shape(T=5), dz=None) == ERR_NULL
    assert _gate_bwd(L, _shape(T=5), ws=None) == ERR_WORKSPACE
    assert _gate_bwd(L, _shape(T=5), wsb=16) == ERR_WORKSPACE
    assert _gate_bwd(L, _shape(T=5), dw=ctypes.c_void_p(0x10004)) == ERR_ALIGN
    assert _gate_bwd(L, _shape(T=5, V=1024)) == ERR_UNSUPPORTED


def test_fp32_wide_values_run_as_slices(L):
    # fp32 takes V = 256 and 512 as slices of 128 value columns: the workspace
    # holds one slice's v, o (forward) or v, d_o, dv and the key-side partial
    # sums (backward) plus that slice's own workspace, whatever the slice count
    f32 = gla.GLA_DTYPE_FP32
    fw = lambda V: L.gla_fwd_workspace_size(ctypes.byref(_shape(B=2, H=4, T=1024, K=128, V=V, dtype=f32)))
    bw = lambda V: L.gla_bwd_workspace_size(ctypes.byref(_shape(B=2, H=4, T=1024, K=128, V=V, dtype=f32)))
    rows = 2 * 4 * 1024
    assert fw(256) == fw(512) and fw(256) >= 2 * rows * 128 * 4
    assert bw(256) == bw(512) and bw(256) >= 3 * rows * 128 * 4 + 3 * rows * 128 * 4
    for V in (256, 512):
        s = _shape(T=128, K=64, V=V, dtype=f32)
        need_f = L.gla_fwd_workspace_size(ctypes.byref(s))
        assert need_f > 0 and _fwd(L, s, wsb=need_f - 1) == ERR_WORKSPACE
        need_b = L.gla_bwd_workspace_size(ctypes.byref(s))
        assert need_b > 0 and _bwd(L, s, wsb=need_b - 1) == ERR_WORKSPACE
    assert L.gla_ckpt_size(ctypes.byref(_shape(T=1024, K=128, V=256, dtype=f32))) == 0


def test_wide_keys_run_as_slices(L):
    # K past the kernels' widest (16-bit: 256, fp32: 128) runs as key slices:
    # the workspace holds one slice's q, k, g columns (per-column gates), the
    # partial output (forward) or dq, dk, dg and the partial dv (backward), its
    # state rows and that slice's own workspace
    rows = 2 * 4 * 1024
    for dtype, W, e in ((gla.GLA_DTYPE_BF16, 256, 2), (gla.GLA_DTYPE_FP32, 128, 4)):
        for K in (2 * W, 512):
            s = _shape(B=2, H=4, T=1024, K=K, V=128, dtype=dtype)
            sub = _shape(B=2, H=4, T=1024, K=W, V=128, dtype=dtype)
            f, fs = L.gla_fwd_workspace_size(ctypes.byref(s)), L.gla_fwd_workspace_size(ctypes.byref(sub))
            b, bs = L.gla_bwd_workspace_size(ctypes.byref(s)), L.gla_bwd_workspace_size(ctypes.byref(sub))
            assert f >= fs + 3 * rows * W * e + rows * 128 * e
            assert b >= bs + 6 * rows * W * e + rows * 128 * e
            assert _fwd(L, s, wsb=f - 1) == ERR_WORKSPACE
            assert _bwd(L, s, wsb=b - 1) == ERR_WORKSPACE
    # the scalar gate is shared by the slices: no per-slice gate copy, one dg partial
    s = _shape(B=2, H=4, T=1024, K=512, V=128)
    assert L.gla_bwd_scalar_workspace_size(ctypes.byref(s)) > 0
    assert L.gla_ckpt_size(ctypes.byref(_shape(T=8192, K=512, V=128))) == 0


def test_scalar_gate_entry_points_validate(L):
    # fp32: the per-column path on the gate repeated over the key columns, plus
    # the repeated gate and the per-column dg ([B,T,H,K] fp32 each)
    s32 = _shape(T=128, K=128, V=128, dtype=gla.GLA_DTYPE_FP32)
    rows = 2 * 128 * 3
    assert (L.gla_bwd_scalar_workspace_size(ctypes.byref(s32)) >=
            L.gla_bwd_workspace_size(ctypes.byref(s32)) + 2 * rows * 128 * 4)
    assert (L.gla_fwd_scalar_workspace_size(ctypes.byref(s32)) >=
            L.gla_fwd_workspace_size(ctypes.byref(s32)) + rows * 128 * 4)
    b16 = _shape(T=128, K=128, V=128)
    assert L.gla_fwd_scalar_workspace_size(ctypes.byref(b16)) == L.gla_fwd_workspace_size(ctypes.byref(b16))
    assert L.gla_fwd_scalar_workspace_size(ctypes.byref(_shape(T=100))) == 0
    s16 = _shape(T=128, K=128, V=256)
    assert L.gla_bwd_scalar_workspace_size(ctypes.byref(s16)) >= L.gla_bwd_workspace_size(ctypes.byref(s16))
    fwd = lambda shape, **kw: L.gla_fwd_scalar(ctypes.byref(shape), P, P, P, kw.get("g", P), None, P, None,
                                               kw.get("ws", P), 1 << 30, None)
    assert fwd(s32, ws=None) == ERR_WORKSPACE
    assert fwd(_shape(T=100)) == ERR_SHAPE
    assert fwd(_shape(T=128), g=None) == ERR_NULL
    assert fwd(_shape(T=128), g=ctypes.c_void_p(0x10002)) == ERR_ALIGN
    assert fwd(_shape(T=0)) == OK


def test_general_gate_entry_point_validates(L):
    # bf16; the kernels take K in {128, 256} (K = 64 padded to 128, K = 512 as
    # two key slices); one record per chunk and head holding the key side (Ql,
    # Kt^T and gate factors) and the value side (three [64, V] tiles and the
    # column decays)
    ws = lambda shape: L.gla_fwd_general_workspace_size(ctypes.byref(shape))
    assert ws(_shape(T=128, dtype=gla.GLA_DTYPE_FP32)) == 0
    assert ws(_shape(T=128, K=64, V=64)) > ws(_shape(T=128, K=128, V=64)) > 0
    assert ws(_shape(T=128, K=96, V=64)) == 0
    assert ws(_shape(T=100, K=128)) == 0
    s = _shape(B=2, H=4, T=8192, K=256, V=512)
    assert ws(s) == ws(s) and ws(s) >= 2 * 4 * 128 * (2 * 2 * 64 * 256 + 3 * 2 * 64 * 512)
    fwd = lambda shape, **kw: L.gla_fwd_general(ctypes.byref(shape), P, P, P, P, kw.get("h", P), None, P, None,
                                                kw.get("ws", P), 1 << 40, None)
    assert fwd(_shape(T=128, K=128, dtype=gla.GLA_DTYPE_FP32)) == ERR_UNSUPPORTED
    assert fwd(_shape(T=128, K=1024, V=64)) == ERR_UNSUPPORTED
    assert fwd(_shape(T=128, K=64, V=64), ws=None) == ERR_WORKSPACE
    assert fwd(_shape(T=100, K=128)) == ERR_SHAPE
    assert fwd(_shape(T=128, K=128), h=None) == ERR_NULL
    assert fwd(_shape(T=128, K=128), h=ctypes.c_void_p(0x10002)) == ERR_ALIGN
    assert fwd(_shape(T=128, K=128), ws=None) == ERR_WORKSPACE
    assert fwd(_shape(T=0, K=128)) == OK


def test_general_gate_backward_validates(L):
    ws = lambda shape: L.gla_bwd_general_workspace_size(ctypes.byref(shape))
    assert ws(_shape(T=128, K=128, V=128, dtype=gla.GLA_DTYPE_FP32)) == 0
    # K or V = 64: padded to 128 with zero columns
    assert ws(_shape(T=128, K=64, V=128)) > ws(_shape(T=128, K=128, V=128)) > 0
    assert ws(_shape(T=128, K=128, V=64)) > ws(_shape(T=128, K=128, V=128))
    assert ws(_shape(T=128, K=64, V=64)) > 0
    # V = 512 as two value slices, K = 512 as two key slices, around the K, V <= 256 backward
    sub = ws(_shape(T=128, K=128, V=256))
    assert ws(_shape(T=128, K=128, V=512)) > sub > 0
    assert ws(_shape(T=128, K=512, V=512)) > ws(_shape(T=128, K=256, V=512)) > 0
    s = _shape(B=2, H=4, T=8192, K=128, V=256)
    # at least the chunk-start states of the forward and of the reversed dS pass
    assert ws(s) == ws(s) and ws(s) >= 2 * (2 * 4 * 128 * 128 * 256 * 2)
    bwd = lambda shape, **kw: L.gla_bwd_general(ctypes.byref(shape), P, P, P, P, kw.get("h", P), None, P, None,
                                                P, P, P, P, kw.get("dh", P), None, kw.get("ws", P), 1 << 40, None)
    assert bwd(_shape(T=128, K=128, V=128, dtype=gla.GLA_DTYPE_FP32)) == ERR_UNSUPPORTED
    assert bwd(_shape(T=128, K=256, V=1024)) == ERR_UNSUPPORTED
    assert bwd(_shape(T=128, K=64, V=64), ws=None) == ERR_WORKSPACE
    assert bwd(_shape(T=100, K=128, V=128)) == ERR_SHAPE
    assert bwd(_shape(T=128, K=128, V=128), h=None) == ERR_NULL
    assert bwd(_shape(T=128, K=128, V=128), dh=None) == ERR_NULL
    assert bwd(_shape(T=128, K=128, V=128), h=ctypes.c_void_p(0x10002)) == ERR_ALIGN
    assert bwd(_shape(T=128, K=128, V=128), ws=None) == ERR_WORKSPACE
    assert bwd(_shape(T=0, K=128, V=128)) == OK


def test_binding_rejects_non_contiguous_q():
    # a q sliced out of a fused projection (or expanded with stride 0) must be
    # refused by every wrapper before the library is called: the kernels read
    # dense [B,T,H,K] rows
    import torch

    B, T, H, K, V = 1, 64, 2, 64, 64
    fused = torch.zeros(B, T, H, 3 * K, dtype=torch.bfloat16)
    q_slice = fused[..., :K]
    q_bcast = torch.zeros(1, 1, 1, K, dtype=torch.bfloat16).expand(B, T, H, K)
    k = torch.zeros(B, T, H, K, dtype=torch.bfloat16)
    g = torch.zeros(B, T, H, K, dtype=torch.bfloat16)
    gs = torch.zeros(B, T, H, dtype=torch.bfloat16)
    v = torch.zeros(B, T, H, V, dtype=torch.bfloat16)
    hv = torch.zeros(B, T, H, V, dtype=torch.bfloat16)
    state = torch.zeros(B, H, K, V)
    for q in (q_slice, q_bcast):
        assert not q.is_contiguous()
        calls = [
            lambda: gla.gla_fwd(q, k, v, g),
            lambda: gla.gla_bwd(q, k, v, g, v),
            lambda: gla.gla_fwd_scalar(q, k, v, gs),
            lambda: gla.gla_bwd_scalar(q, k, v, gs, v),
            lambda: gla.gla_fwd_general(q, k, v, g, hv),
            lambda: gla.gla_bwd_general(q, k, v, g, hv, v),
            lambda: gla.gla_decode(q, k, v, g, state),
        ]
        for call in calls:
            with pytest.raises(ValueError, match="q must be contiguous"):
                call()


def test_fwd_noalloc_validates_before_any_hip_call(L):
    # gla_fwd_noalloc checks every argument, and that the shape's scratch fits
    # the library's fixed array, before it looks up that array on the device
    na = lambda shape, **kw: L.gla_fwd_noalloc(ctypes.byref(shape) if shape is not None else None, kw.get("q", P),
                                               P, P, P, kw.get("s0", None), kw.get("o", P), None, None)
    assert na(None) == ERR_NULL
    assert na(_shape(), q=None) == ERR_NULL
    assert na(_shape(), o=None) == ERR_NULL
    assert na(_shape(T=100)) == ERR_SHAPE
    assert na(_shape(K=96)) == ERR_UNSUPPORTED
    assert na(_shape(), s0=ctypes.c_void_p(0x10004)) == ERR_ALIGN
    assert na(_shape(T=0)) == OK            # nothing to compute, no scratch needed
    wide = _shape(B=2, H=4, T=8192, K=256, V=512)
    assert L.gla_fwd_workspace_size(ctypes.byref(wide)) > 32 << 20
    assert na(wide) == ERR_WORKSPACE
    assert b"fixed scratch" in L.gla_last_error_detail()


def test_ckpt_entry_points_validate(L):
    size = lambda shape: L.gla_ckpt_size(ctypes.byref(shape))
    s = _shape(B=2, H=4, T=8192, K=128, V=256)
    assert size(s) == size(s) > 0
    assert size(s) % (128 * 256 * 2) == 0              # whole bf16 states
    assert size(_shape(dtype=gla.GLA_DTYPE_FP32)) == 0  # fp32: no checkpoint
    assert size(_shape(K=256, V=256, T=8192)) == 0      # wide heads: no checkpoint
    assert size(_shape(B=1, H=1, T=64)) == 0            # one segment
    assert size(_shape(V=512, T=8192)) == 0             # V = 512: the column-half backward, no checkpoint
    assert size(_shape(V=1024, T=8192)) == 0            # not a backward shape
    fwd = lambda shape, ck=P: L.gla_fwd_ckpt(ctypes.byref(shape), P, P, P, P, None, P, None, ck, P, 1 << 40, None)
    bwd = lambda shape, ck=P: L.gla_bwd_ckpt(ctypes.byref(shape), P, P, P, P, None, ck, P, None, P, P, P, P, None,
                                             P, 1 << 40, None)
    assert fwd(s, ck=None) == ERR_NULL
    assert bwd(s, ck=None) == ERR_NULL
    assert fwd(s, ck=ctypes.c_void_p(0x10008)) == ERR_ALIGN
    assert bwd(s, ck=ctypes.c_void_p(0x10008)) == ERR_ALIGN
    assert fwd(_shape(T=100)) == ERR_SHAPE
    assert bwd(_shape(V=1024)) == ERR_UNSUPPORTED
    assert bwd(_shape(K=1024, dtype=gla.GLA_DTYPE_FP32)) == ERR_UNSUPPORTED


def test_scalar_ckpt_entry_points_validate(L):
    # the scalar gate's pair takes gla_ckpt_size's checkpoint and the scalar workspaces
    s = _shape(B=2, H=4, T=8192, K=128, V=256)
    fwd = lambda shape, ck=P: L.gla_fwd_scalar_ckpt(ctypes.byref(shape), P, P, P, P, None, P, None, ck, P, 1 << 40,
                                                    None)
    bwd = lambda shape, ck=P: L.gla_bwd_scalar_ckpt(ctypes.byref(shape), P, P, P, P, None, ck, P, None, P, P, P, P,
                                                    None, P, 1 << 40, None)
    assert fwd(s, ck=None) == ERR_NULL
    assert bwd(s, ck=None) == ERR_NULL
    assert fwd(s, ck=ctypes.c_void_p(0x10008)) == ERR_ALIGN
    assert bwd(s, ck=ctypes.c_void_p(0x10008)) == ERR_ALIGN
    assert fwd(_shape(T=100)) == ERR_SHAPE
    assert bwd(_shape(K=1024)) == ERR_UNSUPPORTED
    assert fwd(_shape(T=0)) == OK
    # the workspace is checked before anything is enqueued
    ws_b = L.gla_bwd_scalar_workspace_size(ctypes.byref(s))
    assert ws_b > 0
    assert L.gla_bwd_scalar_ckpt(ctypes.byref(s), P, P, P, P, None, P, P, None, P, P, P, P, None, P, ws_b - 1,
                                 None) == ERR_WORKSPACE


def test_general_ckpt_entry_points_validate(L):
    size = lambda shape: L.gla_general_ckpt_size(ctypes.byref(shape))
    s = _shape(B=2, H=4, T=8192, K=128, V=256)
    # the states before every chunk (bf16), then S_T (fp32) at a 256-byte offset
    assert size(s) == 8 * 128 * 128 * 256 * 2 + 8 * 128 * 256 * 4
    assert size(_shape(K=256, V=128, T=640)) > 0
    assert size(_shape(dtype=gla.GLA_DTYPE_FP32)) == 0   # the general path takes bf16
    assert size(_shape(K=64)) == 0                       # K not in {128, 256}
    assert size(_shape(K=128, V=512, T=8192)) == 0       # V = 512: the value-sliced backward, no checkpoint
    assert size(_shape(K=512, V=128, T=8192)) == 0       # K = 512: the key-sliced backward, no checkpoint
    assert size(_shape(T=0)) == 0
    fwd = lambda shape, ck=P, o=P: L.gla_fwd_general_ckpt(ctypes.byref(shape), P, P, P, P, P, None, o, None, ck, P,
                                                          1 << 40, None)
    bwd = lambda shape, ck=P, o=P: L.gla_bwd_general_ckpt(ctypes.byref(shape), P, P, P, P, P, None, o, ck, P, None,
                                                          P, P, P, P, P, None, P, 1 << 40, None)
    assert fwd(s, ck=None) == ERR_NULL
    assert bwd(s, ck=None) == ERR_NULL
    assert bwd(s, o=None) == ERR_NULL
    assert fwd(s, ck=ctypes.c_void_p(0x10008)) == ERR_ALIGN
    assert bwd(s, ck=ctypes.c_void_p(0x10008)) == ERR_ALIGN
    assert bwd(s, o=ctypes.c_void_p(0x10008)) == ERR_ALIGN
    assert fwd(_shape(T=100)) == ERR_SHAPE
    # a shape without a checkpoint runs the plain pair: ckpt and o may be NULL, and the
    # plain calls' own checks apply (o is the forward's output; the backward's workspace)
    nock = _shape(K=128, V=512, T=8192)
    assert fwd(nock, ck=None, o=None) == ERR_NULL
    assert b"o" in L.gla_last_error_detail()
    assert L.gla_bwd_general_ckpt(ctypes.byref(nock), P, P, P, P, P, None, None, None, P, None, P, P, P, P, P, None,
                                  None, 1 << 40, None) == ERR_WORKSPACE
    assert fwd(_shape(dtype=gla.GLA_DTYPE_FP32)) == ERR_UNSUPPORTED
    assert fwd(_shape(K=1024, V=128)) == ERR_UNSUPPORTED
    empty = _shape(T=0, K=128, V=128)
    assert fwd(empty, ck=None, o=None) == OK              # nothing to compute: no checkpoint needed
    assert bwd(empty, ck=None, o=None) == OK
