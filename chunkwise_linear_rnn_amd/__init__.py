"""Chunkwise gated linear attention (GLA) for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libgla.so`` (declared in
``include/gla.h``).  PyTorch is used only to own device memory and to name the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing or a call fails, an
exception is raised.

Functions mirror the ABI:
  gla_fwd(q, k, v, g, s0=None, ...)         -> (o, s_final)
  gla_bwd(q, k, v, g, d_o, s0=None, dht=None) -> (dq, dk, dv, dg, ds0)
  gla_fwd_scalar / gla_bwd_scalar            (the same with a scalar gate g [B,T,H] per token and head)
  gla_fwd_ckpt / gla_bwd_ckpt, gla_fwd_scalar_ckpt / gla_bwd_scalar_ckpt  (training pairs with a checkpoint)
  gla_decode(q, k, v, g, state)              -> o   (recurrent form; state updated in place)
  gla_out_gate(o, z, ln_w, ln_b, eps)        -> y   (per-head LayerNorm, Swish output gate)
  gla_out_gate_bwd(o, z, ln_w, ln_b, eps, dy) -> (d_o, dz, dln_w, dln_b)
  gla_fwd_workspace_size / gla_bwd_workspace_size / gla_out_gate_bwd_workspace_size
Layouts: q, k, g [B,T,H,K]; v, o, d_o, z, y [B,T,H,V]; states [B,H,K,V] float32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GLA_LIBRARY selects another build of the same ABI (the host-sanitizer build
# of the validation layer, whose launchers are stubs); default: libgla.so here.
LIB_PATH = os.environ.get("GLA_LIBRARY") or os.path.join(_HERE, "libgla.so")

GLA_DTYPE_FP32 = 0
GLA_DTYPE_BF16 = 1
CHUNK = 64


class GlaShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("K", ctypes.c_int64), ("V", ctypes.c_int64), ("chunk", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class LaunchRecorder(ctypes.Structure):
    """gla_launch_recorder_t: caller-owned events the library records around its launches."""
    _fields_ = [("capacity", ctypes.c_int32), ("count", ctypes.c_int32), ("failed", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("start", ctypes.POINTER(ctypes.c_void_p)),
                ("stop", ctypes.POINTER(ctypes.c_void_p)), ("name", ctypes.POINTER(ctypes.c_char_p))]


class GlaError(RuntimeError):
    def __init__(self, status: int, detail: str, message: str):
        super().__init__("%s (%s)" % (message, detail) if detail else message)
        self.status = status


EXPORTS = ["gla_fwd", "gla_bwd", "gla_fwd_scalar", "gla_bwd_scalar", "gla_decode", "gla_out_gate",
           "gla_out_gate_bwd", "gla_fwd_workspace_size", "gla_bwd_workspace_size", "gla_bwd_scalar_workspace_size",
           "gla_fwd_scalar_workspace_size", "gla_fwd_scalar_ckpt", "gla_bwd_scalar_ckpt",
           "gla_decode_scalar", "gla_decode_general",
           "gla_out_gate_bwd_workspace_size", "gla_fwd_general", "gla_fwd_general_workspace_size",
           "gla_bwd_general", "gla_bwd_general_workspace_size",
           "gla_status_string", "gla_last_error_detail", "gla_abi_version",
           "gla_set_launch_recorder", "gla_fwd_noalloc", "gla_ckpt_size", "gla_fwd_ckpt", "gla_bwd_ckpt",
           "gla_general_ckpt_size", "gla_fwd_general_ckpt", "gla_bwd_general_ckpt"]

_lib = None


def lib():
    """Load libgla.so (built by ``build.build()``); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libgla.so not built: run `python -m chunkwise_linear_rnn_amd.build` "
                           "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    sh = ctypes.POINTER(GlaShape)
    L.gla_fwd.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.gla_fwd.restype = ctypes.c_int
    L.gla_bwd.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.gla_bwd.restype = ctypes.c_int
    L.gla_ckpt_size.argtypes = [sh]
    L.gla_ckpt_size.restype = ctypes.c_size_t
    L.gla_fwd_ckpt.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.gla_fwd_ckpt.restype = ctypes.c_int
    L.gla_bwd_ckpt.argtypes = [sh] + [vp] * 14 + [ctypes.c_size_t, vp]
    L.gla_bwd_ckpt.restype = ctypes.c_int
    L.gla_fwd_scalar_ckpt.argtypes = L.gla_fwd_ckpt.argtypes
    L.gla_fwd_scalar_ckpt.restype = ctypes.c_int
    L.gla_bwd_scalar_ckpt.argtypes = L.gla_bwd_ckpt.argtypes
    L.gla_bwd_scalar_ckpt.restype = ctypes.c_int
    L.gla_fwd_noalloc.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, vp]
    L.gla_fwd_noalloc.restype = ctypes.c_int
    L.gla_fwd_scalar.argtypes = L.gla_fwd.argtypes
    L.gla_fwd_scalar.restype = ctypes.c_int
    L.gla_bwd_scalar.argtypes = L.gla_bwd.argtypes
    L.gla_bwd_scalar.restype = ctypes.c_int
    L.gla_bwd_scalar_workspace_size.argtypes = [sh]
    L.gla_fwd_scalar_workspace_size.argtypes = [sh]
    L.gla_fwd_scalar_workspace_size.restype = ctypes.c_size_t
    L.gla_fwd_general.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.gla_fwd_general.restype = ctypes.c_int
    L.gla_fwd_general_workspace_size.argtypes = [sh]
    L.gla_bwd_general.argtypes = [sh] + [vp] * 15 + [ctypes.c_size_t, vp]
    L.gla_bwd_general.restype = ctypes.c_int
    L.gla_bwd_general_workspace_size.argtypes = [sh]
    L.gla_bwd_general_workspace_size.restype = ctypes.c_size_t
    L.gla_fwd_general_workspace_size.restype = ctypes.c_size_t
    L.gla_general_ckpt_size.argtypes = [sh]
    L.gla_general_ckpt_size.restype = ctypes.c_size_t
    L.gla_fwd_general_ckpt.argtypes = [sh] + [vp] * 10 + [ctypes.c_size_t, vp]
    L.gla_fwd_general_ckpt.restype = ctypes.c_int
    L.gla_bwd_general_ckpt.argtypes = [sh] + [vp] * 17 + [ctypes.c_size_t, vp]
    L.gla_bwd_general_ckpt.restype = ctypes.c_int
    L.gla_bwd_scalar_workspace_size.restype = ctypes.c_size_t
    L.gla_decode.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp]
    L.gla_decode.restype = ctypes.c_int
    L.gla_decode_scalar.argtypes = L.gla_decode.argtypes
    L.gla_decode_scalar.restype = ctypes.c_int
    L.gla_decode_general.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, vp]
    L.gla_decode_general.restype = ctypes.c_int
    fl = ctypes.c_float
    L.gla_out_gate.argtypes = [sh, vp, vp, vp, vp, fl, vp, vp]
    L.gla_out_gate.restype = ctypes.c_int
    L.gla_out_gate_bwd.argtypes = [sh, vp, vp, vp, vp, fl, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.gla_out_gate_bwd.restype = ctypes.c_int
    L.gla_out_gate_bwd_workspace_size.argtypes = [sh]
    L.gla_out_gate_bwd_workspace_size.restype = ctypes.c_size_t
    L.gla_fwd_workspace_size.argtypes = [sh]
    L.gla_fwd_workspace_size.restype = ctypes.c_size_t
    L.gla_bwd_workspace_size.argtypes = [sh]
    L.gla_bwd_workspace_size.restype = ctypes.c_size_t
    L.gla_status_string.argtypes = [ctypes.c_int]
    L.gla_status_string.restype = ctypes.c_char_p
    L.gla_last_error_detail.argtypes = []
    L.gla_last_error_detail.restype = ctypes.c_char_p
    L.gla_abi_version.restype = ctypes.c_int
    L.gla_set_launch_recorder.argtypes = [ctypes.POINTER(LaunchRecorder)]
    L.gla_set_launch_recorder.restype = None
    _lib = L
    return L


def make_shape(B, T, H, K, V, dtype) -> GlaShape:
    if isinstance(dtype, torch.dtype):
        dtype = GLA_DTYPE_BF16 if dtype == torch.bfloat16 else (GLA_DTYPE_FP32 if dtype == torch.float32 else -1)
    return GlaShape(B, T, H, K, V, CHUNK, dtype, 0)


def _check(rc: int):
    if rc != 0:
        L = lib()
        raise GlaError(rc, L.gla_last_error_detail().decode(), L.gla_status_string(rc).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def gla_fwd_workspace_size(B, T, H, K, V, dtype) -> int:
    return int(lib().gla_fwd_workspace_size(ctypes.byref(make_shape(B, T, H, K, V, dtype))))


def gla_bwd_workspace_size(B, T, H, K, V, dtype) -> int:
    return int(lib().gla_bwd_workspace_size(ctypes.byref(make_shape(B, T, H, K, V, dtype))))


def _dims(q, v):
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B,T,H,D] (got %d and %d dims)" % (q.dim(), v.dim()))
    B, T, H, K = q.shape
    return B, T, H, K, v.shape[-1]


def _need(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def gla_fwd_into(q, k, v, g, s0, o, s_final, ws, stream=None, scalar_gate=False):
    """Call the ABI with caller-owned outputs and workspace (nothing allocated).
    scalar_gate: g is [B,T,H] and gla_fwd_scalar is called."""
    B, T, H, K, V = _dims(q, v)
    shape = make_shape(B, T, H, K, V, q.dtype)
    nbytes = 0 if ws is None else ws.numel()
    fn = lib().gla_fwd_scalar if scalar_gate else lib().gla_fwd
    _check(fn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0), _ptr(o), _ptr(s_final), _ptr(ws),
              nbytes, _stream(stream)))


def gla_fwd_noalloc_into(q, k, v, g, s0, o, s_final, stream=None):
    """gla_fwd_noalloc: the forward with the library's fixed device scratch
    instead of a workspace (outputs caller-owned; nothing allocated)."""
    B, T, H, K, V = _dims(q, v)
    shape = make_shape(B, T, H, K, V, q.dtype)
    _check(lib().gla_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0), _ptr(o),
                                 _ptr(s_final), _stream(stream)))


def gla_bwd_into(q, k, v, g, s0, d_o, dht, dq, dk, dv, dg, ds0, ws, stream=None, scalar_gate=False):
    B, T, H, K, V = _dims(q, v)
    shape = make_shape(B, T, H, K, V, q.dtype)
    nbytes = 0 if ws is None else ws.numel()
    fn = lib().gla_bwd_scalar if scalar_gate else lib().gla_bwd
    _check(fn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0), _ptr(d_o), _ptr(dht), _ptr(dq),
              _ptr(dk), _ptr(dv), _ptr(dg), _ptr(ds0), _ptr(ws), nbytes, _stream(stream)))


def gla_ckpt_size(B, T, H, K, V, dtype) -> int:
    return int(lib().gla_ckpt_size(ctypes.byref(make_shape(B, T, H, K, V, dtype))))


def gla_fwd_ckpt_into(q, k, v, g, s0, o, s_final, ckpt, ws, stream=None, scalar_gate=False):
    """gla_fwd_ckpt with caller-owned outputs, checkpoint and workspace
    (scalar_gate: g is [B,T,H] and gla_fwd_scalar_ckpt is called)."""
    B, T, H, K, V = _dims(q, v)
    shape = make_shape(B, T, H, K, V, q.dtype)
    nbytes = 0 if ws is None else ws.numel()
    fn = lib().gla_fwd_scalar_ckpt if scalar_gate else lib().gla_fwd_ckpt
    _check(fn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0), _ptr(o),
                              _ptr(s_final), _ptr(ckpt), _ptr(ws), nbytes, _stream(stream)))


def gla_bwd_ckpt_into(q, k, v, g, s0, ckpt, d_o, dht, dq, dk, dv, dg, ds0, ws, stream=None, scalar_gate=False):
    B, T, H, K, V = _dims(q, v)
    shape = make_shape(B, T, H, K, V, q.dtype)
    nbytes = 0 if ws is None else ws.numel()
    fn = lib().gla_bwd_scalar_ckpt if scalar_gate else lib().gla_bwd_ckpt
    _check(fn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0), _ptr(ckpt),
                              _ptr(d_o), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(ds0), _ptr(ws),
                              nbytes, _stream(stream)))


def gla_fwd_ckpt(q, k, v, g, s0=None, output_final_state=True, stream=None):
    """(o, S_T, ckpt): gla_fwd that also keeps the backward's segment-start
    states (None when the shape has no checkpoint; gla_bwd_ckpt then recomputes)."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)),
                         ("v", v, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(s0, "s0", (B, H, K, V), torch.float32, dev)
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    sf = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if output_final_state else None
    ck = workspace(gla_ckpt_size(B, T, H, K, V, dt), dev)
    ws = workspace(gla_fwd_workspace_size(B, T, H, K, V, dt), dev)
    gla_fwd_ckpt_into(q, k, v, g, s0, o, sf, ck, ws, stream)
    return o, sf, ck


def gla_bwd_ckpt(q, k, v, g, d_o, ckpt, s0=None, dht=None, output_ds0=True, stream=None):
    """gla_bwd starting from the segment states gla_fwd_ckpt kept for the same inputs."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)),
                         ("v", v, (B, T, H, V)), ("d_o", d_o, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(s0, "s0", (B, H, K, V), torch.float32, dev)
    _need(dht, "dht", (B, H, K, V), torch.float32, dev)
    need = gla_ckpt_size(B, T, H, K, V, dt)
    if need > 0 and (ckpt is None or ckpt.numel() * ckpt.element_size() < need or ckpt.device != dev
                     or not ckpt.is_contiguous()):
        raise ValueError("ckpt must be the contiguous %d-byte checkpoint of gla_fwd_ckpt on %s" % (need, dev))
    dq = torch.empty_like(q); dk = torch.empty_like(k); dg = torch.empty_like(g); dv = torch.empty_like(v)
    ds0 = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if output_ds0 else None
    ws = workspace(gla_bwd_workspace_size(B, T, H, K, V, dt), dev)
    gla_bwd_ckpt_into(q, k, v, g, s0, ckpt if need > 0 else None, d_o, dht, dq, dk, dv, dg, ds0, ws, stream)
    return dq, dk, dv, dg, ds0


def gla_fwd_scalar_ckpt(q, k, v, g, s0=None, output_final_state=True, stream=None):
    """(o, S_T, ckpt): gla_fwd_scalar that also keeps the backward's segment-start
    states (None when the shape has no checkpoint)."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H)),
                         ("v", v, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(s0, "s0", (B, H, K, V), torch.float32, dev)
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    sf = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if output_final_state else None
    ck = workspace(gla_ckpt_size(B, T, H, K, V, dt), dev)
    ws = workspace(gla_fwd_scalar_workspace_size(B, T, H, K, V, dt), dev)
    gla_fwd_ckpt_into(q, k, v, g, s0, o, sf, ck, ws, stream, scalar_gate=True)
    return o, sf, ck


def gla_bwd_scalar_ckpt(q, k, v, g, d_o, ckpt, s0=None, dht=None, output_ds0=True, stream=None):
    """gla_bwd_scalar starting from the segment states gla_fwd_scalar_ckpt kept."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H)),
                         ("v", v, (B, T, H, V)), ("d_o", d_o, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(s0, "s0", (B, H, K, V), torch.float32, dev)
    _need(dht, "dht", (B, H, K, V), torch.float32, dev)
    need = gla_ckpt_size(B, T, H, K, V, dt)
    if need > 0 and (ckpt is None or ckpt.numel() * ckpt.element_size() < need or ckpt.device != dev
                     or not ckpt.is_contiguous()):
        raise ValueError("ckpt must be the contiguous %d-byte checkpoint of gla_fwd_scalar_ckpt on %s" % (need, dev))
    dq = torch.empty_like(q); dk = torch.empty_like(k); dg = torch.empty_like(g); dv = torch.empty_like(v)
    ds0 = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if output_ds0 else None
    ws = workspace(gla_bwd_scalar_workspace_size(B, T, H, K, V, dt), dev)
    gla_bwd_ckpt_into(q, k, v, g, s0, ckpt if need > 0 else None, d_o, dht, dq, dk, dv, dg, ds0, ws, stream,
                      scalar_gate=True)
    return dq, dk, dv, dg, ds0


def gla_fwd_scalar_workspace_size(B, T, H, K, V, dtype) -> int:
    return int(lib().gla_fwd_scalar_workspace_size(ctypes.byref(make_shape(B, T, H, K, V, dtype))))


def gla_bwd_scalar_workspace_size(B, T, H, K, V, dtype) -> int:
    return int(lib().gla_bwd_scalar_workspace_size(ctypes.byref(make_shape(B, T, H, K, V, dtype))))


def gla_fwd(q, k, v, g, s0=None, output_final_state=True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """o, S_T = GLA forward.  q, k, g: [B,T,H,K]; v: [B,T,H,V]; s0: [B,H,K,V] fp32 or None."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)), ("v", v, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(q, "q", (B, T, H, K), dt, dev)
    _need(s0, "s0", (B, H, K, V), torch.float32, dev)
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    sf = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if output_final_state else None
    ws = workspace(gla_fwd_workspace_size(B, T, H, K, V, dt), dev)
    gla_fwd_into(q, k, v, g, s0, o, sf, ws, stream)
    return o, sf


def gla_bwd(q, k, v, g, d_o, s0=None, dht=None, output_ds0=True, stream=None):
    """dq, dk, dv, dg, dS0 of <o, d_o> + <S_T, dht> (states recomputed inside)."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)),
                         ("v", v, (B, T, H, V)), ("d_o", d_o, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(s0, "s0", (B, H, K, V), torch.float32, dev)
    _need(dht, "dht", (B, H, K, V), torch.float32, dev)
    dq = torch.empty_like(q); dk = torch.empty_like(k); dg = torch.empty_like(g); dv = torch.empty_like(v)
    ds0 = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if output_ds0 else None
    ws = workspace(gla_bwd_workspace_size(B, T, H, K, V, dt), dev)
    gla_bwd_into(q, k, v, g, s0, d_o, dht, dq, dk, dv, dg, ds0, ws, stream)
    return dq, dk, dv, dg, ds0


def gla_fwd_scalar(q, k, v, g, s0=None, output_final_state=True, stream=None):
    """gla_fwd with a scalar gate g [B,T,H] per token and head."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H)),
                         ("v", v, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(s0, "s0", (B, H, K, V), torch.float32, dev)
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    sf = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if output_final_state else None
    ws = workspace(gla_fwd_scalar_workspace_size(B, T, H, K, V, dt), dev)
    gla_fwd_into(q, k, v, g, s0, o, sf, ws, stream, scalar_gate=True)
    return o, sf


def gla_bwd_scalar(q, k, v, g, d_o, s0=None, dht=None, output_ds0=True, stream=None):
    """gla_bwd with a scalar gate g [B,T,H]; dg is [B,T,H]."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H)),
                         ("v", v, (B, T, H, V)), ("d_o", d_o, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(s0, "s0", (B, H, K, V), torch.float32, dev)
    _need(dht, "dht", (B, H, K, V), torch.float32, dev)
    dq = torch.empty_like(q); dk = torch.empty_like(k); dg = torch.empty_like(g); dv = torch.empty_like(v)
    ds0 = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if output_ds0 else None
    ws = workspace(gla_bwd_scalar_workspace_size(B, T, H, K, V, dt), dev)
    gla_bwd_into(q, k, v, g, s0, d_o, dht, dq, dk, dv, dg, ds0, ws, stream, scalar_gate=True)
    return dq, dk, dv, dg, ds0


def gla_fwd_general_workspace_size(B, T, H, K, V, dtype) -> int:
    return int(lib().gla_fwd_general_workspace_size(ctypes.byref(make_shape(B, T, H, K, V, dtype))))


def gla_fwd_general_into(q, k, v, g, h, s0, o, s_final, ws, stream=None):
    """gla_fwd_general with caller-owned outputs and workspace (nothing allocated)."""
    B, T, H, K, V = _dims(q, v)
    shape = make_shape(B, T, H, K, V, q.dtype)
    nbytes = 0 if ws is None else ws.numel()
    _check(lib().gla_fwd_general(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h), _ptr(s0), _ptr(o),
                                 _ptr(s_final), _ptr(ws), nbytes, _stream(stream)))


def gla_fwd_general(q, k, v, g, h, s0=None, output_final_state=True, stream=None):
    """o, S_T of general gated linear attention, forget gate exp(g_t)^T exp(h_t).

    q, k, g: [B,T,H,K]; v, h: [B,T,H,V] (bf16); s0: [B,H,K,V] fp32 or None."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)),
                         ("v", v, (B, T, H, V)), ("h", h, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(s0, "s0", (B, H, K, V), torch.float32, dev)
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    sf = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if output_final_state else None
    ws = workspace(gla_fwd_general_workspace_size(B, T, H, K, V, dt), dev)
    gla_fwd_general_into(q, k, v, g, h, s0, o, sf, ws, stream)
    return o, sf


def gla_bwd_general_workspace_size(B, T, H, K, V, dtype) -> int:
    return int(lib().gla_bwd_general_workspace_size(ctypes.byref(make_shape(B, T, H, K, V, dtype))))


def gla_bwd_general_into(q, k, v, g, h, s0, d_o, dht, dq, dk, dv, dg, dh, ds0, ws, stream=None):
    B, T, H, K, V = _dims(q, v)
    shape = make_shape(B, T, H, K, V, q.dtype)
    nbytes = 0 if ws is None else ws.numel()
    _check(lib().gla_bwd_general(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h), _ptr(s0),
                                 _ptr(d_o), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dh), _ptr(ds0),
                                 _ptr(ws), nbytes, _stream(stream)))


def gla_bwd_general(q, k, v, g, h, d_o, s0=None, dht=None, output_ds0=True, stream=None):
    """dq, dk, dv, dg, dh, dS0 of <o, d_o> + <S_T, dht> for gla_fwd_general (bf16)."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)),
                         ("v", v, (B, T, H, V)), ("h", h, (B, T, H, V)), ("d_o", d_o, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(s0, "s0", (B, H, K, V), torch.float32, dev)
    _need(dht, "dht", (B, H, K, V), torch.float32, dev)
    dq = torch.empty_like(q); dk = torch.empty_like(k); dg = torch.empty_like(g)
    dv = torch.empty_like(v); dh = torch.empty_like(h)
    ds0 = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if output_ds0 else None
    ws = workspace(gla_bwd_general_workspace_size(B, T, H, K, V, dt), dev)
    gla_bwd_general_into(q, k, v, g, h, s0, d_o, dht, dq, dk, dv, dg, dh, ds0, ws, stream)
    return dq, dk, dv, dg, dh, ds0


def gla_general_ckpt_size(B, T, H, K, V, dtype) -> int:
    return int(lib().gla_general_ckpt_size(ctypes.byref(make_shape(B, T, H, K, V, dtype))))


def gla_fwd_general_ckpt_into(q, k, v, g, h, s0, o, s_final, ckpt, ws, stream=None):
    """gla_fwd_general_ckpt with caller-owned outputs, checkpoint and workspace."""
    B, T, H, K, V = _dims(q, v)
    shape = make_shape(B, T, H, K, V, q.dtype)
    nbytes = 0 if ws is None else ws.numel()
    _check(lib().gla_fwd_general_ckpt(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h), _ptr(s0),
                                      _ptr(o), _ptr(s_final), _ptr(ckpt), _ptr(ws), nbytes, _stream(stream)))


def gla_bwd_general_ckpt_into(q, k, v, g, h, s0, o, ckpt, d_o, dht, dq, dk, dv, dg, dh, ds0, ws, stream=None):
    B, T, H, K, V = _dims(q, v)
    shape = make_shape(B, T, H, K, V, q.dtype)
    nbytes = 0 if ws is None else ws.numel()
    _check(lib().gla_bwd_general_ckpt(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h), _ptr(s0),
                                      _ptr(o), _ptr(ckpt), _ptr(d_o), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv),
                                      _ptr(dg), _ptr(dh), _ptr(ds0), _ptr(ws), nbytes, _stream(stream)))


def gla_fwd_general_ckpt(q, k, v, g, h, s0=None, output_final_state=True, stream=None):
    """(o, S_T, ckpt): gla_fwd_general that also keeps its state before every
    chunk and S_T for gla_bwd_general_ckpt (shapes of gla_bwd_general)."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)),
                         ("v", v, (B, T, H, V)), ("h", h, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(s0, "s0", (B, H, K, V), torch.float32, dev)
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    sf = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if output_final_state else None
    ck = workspace(gla_general_ckpt_size(B, T, H, K, V, dt), dev)
    ws = workspace(gla_fwd_general_workspace_size(B, T, H, K, V, dt), dev)
    gla_fwd_general_ckpt_into(q, k, v, g, h, s0, o, sf, ck, ws, stream)
    return o, sf, ck


def gla_bwd_general_ckpt(q, k, v, g, h, d_o, o, ckpt, s0=None, dht=None, output_ds0=True, stream=None):
    """gla_bwd_general from the forward's o and the checkpoint gla_fwd_general_ckpt
    kept for the same inputs (no forward is rerun)."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)),
                         ("v", v, (B, T, H, V)), ("h", h, (B, T, H, V)), ("d_o", d_o, (B, T, H, V)),
                         ("o", o, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(s0, "s0", (B, H, K, V), torch.float32, dev)
    _need(dht, "dht", (B, H, K, V), torch.float32, dev)
    need = gla_general_ckpt_size(B, T, H, K, V, dt)
    if need > 0 and (ckpt is None or ckpt.numel() * ckpt.element_size() < need or ckpt.device != dev
                     or not ckpt.is_contiguous()):
        raise ValueError("ckpt must be the contiguous %d-byte checkpoint of gla_fwd_general_ckpt on %s" % (need, dev))
    dq = torch.empty_like(q); dk = torch.empty_like(k); dg = torch.empty_like(g)
    dv = torch.empty_like(v); dh = torch.empty_like(h)
    ds0 = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if output_ds0 else None
    ws = workspace(gla_bwd_general_workspace_size(B, T, H, K, V, dt), dev)
    gla_bwd_general_ckpt_into(q, k, v, g, h, s0, o, ckpt, d_o, dht, dq, dk, dv, dg, dh, ds0, ws, stream)
    return dq, dk, dv, dg, dh, ds0


def gla_decode_into(q, k, v, g, state, o, stream=None, h=None, scalar_gate=False):
    """The decode call on caller-owned o: gla_decode, gla_decode_scalar (g [B,T,H])
    or, with h [B,T,H,V], gla_decode_general."""
    B, T, H, K, V = _dims(q, v)
    shape = make_shape(B, T, H, K, V, q.dtype)
    if h is not None:
        _check(lib().gla_decode_general(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h),
                                        _ptr(state), _ptr(o), _stream(stream)))
        return
    fn = lib().gla_decode_scalar if scalar_gate else lib().gla_decode
    _check(fn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(state), _ptr(o), _stream(stream)))


def gla_decode(q, k, v, g, state, stream=None) -> torch.Tensor:
    """o for T tokens of the recurrent form; `state` [B,H,K,V] fp32 is updated in place.

    q, k, g: [B,T,H,K]; v: [B,T,H,V].  T is any count (no chunk constraint)."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)), ("v", v, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    _need(q, "q", (B, T, H, K), dt, dev)
    if state is None:
        raise ValueError("state is required (it is read and updated in place)")
    _need(state, "state", (B, H, K, V), torch.float32, dev)
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    gla_decode_into(q, k, v, g, state, o, stream)
    return o


def gla_decode_scalar(q, k, v, g, state, stream=None) -> torch.Tensor:
    """gla_decode with one log gate per token and head, g [B,T,H]."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H)),
                         ("v", v, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    if state is None:
        raise ValueError("state is required (it is read and updated in place)")
    _need(state, "state", (B, H, K, V), torch.float32, dev)
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    gla_decode_into(q, k, v, g, state, o, stream, scalar_gate=True)
    return o


def gla_decode_general(q, k, v, g, h, state, stream=None) -> torch.Tensor:
    """gla_decode with the general gate exp(g)^T exp(h); h [B,T,H,V] like v."""
    B, T, H, K, V = _dims(q, v)
    dev, dt = q.device, q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)),
                         ("v", v, (B, T, H, V)), ("h", h, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    if state is None:
        raise ValueError("state is required (it is read and updated in place)")
    _need(state, "state", (B, H, K, V), torch.float32, dev)
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    gla_decode_into(q, k, v, g, state, o, stream, h=h)
    return o


def _gate_args(o, z, ln_w, ln_b):
    if o.dim() != 4:
        raise ValueError("o must be [B,T,H,V]")
    B, T, H, V = o.shape
    dev, dt = o.device, o.dtype
    _need(o, "o", (B, T, H, V), dt, dev)
    _need(z, "z", (B, T, H, V), dt, dev)
    if ln_w is None:
        raise ValueError("ln_w is required")
    _need(ln_w, "ln_w", (V,), torch.float32, dev)
    _need(ln_b, "ln_b", (V,), torch.float32, dev)
    return B, T, H, V, dev, dt


def gla_out_gate_bwd_workspace_size(B, T, H, V, dtype) -> int:
    return int(lib().gla_out_gate_bwd_workspace_size(ctypes.byref(make_shape(B, T, H, 0, V, dtype))))


def gla_out_gate_into(o, z, ln_w, ln_b, eps, y, stream=None):
    B, T, H, V = o.shape
    shape = make_shape(B, T, H, 0, V, o.dtype)
    _check(lib().gla_out_gate(ctypes.byref(shape), _ptr(o), _ptr(z), _ptr(ln_w), _ptr(ln_b), float(eps), _ptr(y),
                              _stream(stream)))


def gla_out_gate(o, z, ln_w, ln_b=None, eps=1e-5, stream=None) -> torch.Tensor:
    """y = Swish(z) * (LayerNorm_V(o) * ln_w + ln_b), per head row (GLA layer output, Section 4.4).

    o, z: [B,T,H,V] (bf16 or fp32); ln_w, ln_b: [V] float32 shared by the heads."""
    B, T, H, V, dev, dt = _gate_args(o, z, ln_w, ln_b)
    y = torch.empty(B, T, H, V, dtype=dt, device=dev)
    gla_out_gate_into(o, z, ln_w, ln_b, eps, y, stream)
    return y


def gla_out_gate_bwd_into(o, z, ln_w, ln_b, eps, dy, d_o, dz, dln_w, dln_b, ws, stream=None):
    B, T, H, V = o.shape
    shape = make_shape(B, T, H, 0, V, o.dtype)
    _check(lib().gla_out_gate_bwd(ctypes.byref(shape), _ptr(o), _ptr(z), _ptr(ln_w), _ptr(ln_b), float(eps),
                                  _ptr(dy), _ptr(d_o), _ptr(dz), _ptr(dln_w), _ptr(dln_b), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(stream)))


def gla_out_gate_bwd(o, z, ln_w, ln_b, eps, dy, stream=None):
    """Gradients of <y, dy> for gla_out_gate: (d_o, dz, dln_w, dln_b); dln_b is None when ln_b is."""
    B, T, H, V, dev, dt = _gate_args(o, z, ln_w, ln_b)
    _need(dy, "dy", (B, T, H, V), dt, dev)
    d_o = torch.empty_like(o); dz = torch.empty_like(z)
    dln_w = torch.empty(V, dtype=torch.float32, device=dev)
    dln_b = torch.empty(V, dtype=torch.float32, device=dev) if ln_b is not None else None
    ws = workspace(gla_out_gate_bwd_workspace_size(B, T, H, V, dt), dev)
    gla_out_gate_bwd_into(o, z, ln_w, ln_b, eps, dy, d_o, dz, dln_w, dln_b, ws, stream)
    return d_o, dz, dln_w, dln_b


class KernelTimer:
    """Per-kernel HIP-event times of the library launches this thread makes
    inside ``with timer:`` (gla_set_launch_recorder).  The events are torch
    events with timing enabled, owned here; ``read()`` waits for them and
    returns {kernel: (launches, total_ms)}."""

    def __init__(self, capacity: int = 4096):
        self.capacity = capacity
        self.ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        self.ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        for e in self.ev0 + self.ev1:
            e.record()  # creates the underlying hipEvent_t
        torch.cuda.synchronize()
        self._start = (ctypes.c_void_p * capacity)(*[e.cuda_event for e in self.ev0])
        self._stop = (ctypes.c_void_p * capacity)(*[e.cuda_event for e in self.ev1])
        self._name = (ctypes.c_char_p * capacity)()
        self.rec = LaunchRecorder(capacity, 0, 0, 0, self._start, self._stop, self._name)

    def __enter__(self):
        self.rec.count = 0
        self.rec.failed = 0
        lib().gla_set_launch_recorder(ctypes.byref(self.rec))
        return self

    def __exit__(self, *exc):
        lib().gla_set_launch_recorder(None)
        return False

    def read(self) -> dict:
        torch.cuda.synchronize()
        if self.rec.failed:
            raise RuntimeError("gla launch recorder: hipEventRecord failed")
        if self.rec.count > self.capacity:
            raise RuntimeError("gla launch recorder: %d launches for %d event pairs" % (self.rec.count,
                                                                                     self.capacity))
        out = {}
        for i in range(self.rec.count):
            name = self._name[i].decode()
            c, t = out.get(name, (0, 0.0))
            out[name] = (c + 1, t + self.ev0[i].elapsed_time(self.ev1[i]))
        return out
