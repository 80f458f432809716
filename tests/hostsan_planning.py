"""Launch planning under the host-sanitizer build (CPU, no GPU).  Not collected
by default (no test_ prefix): tests/test_sanitize.py names it explicitly.

Only meaningful with GLA_LIBRARY pointing at the sanitizer build of the ABI
layer (``build.build_host_sanitized()``), whose kernel launchers are stubs that
report hipErrorNoDevice: every valid call then runs validation, the launch
plan, the workspace partition and the launcher dispatch, and must end in
GLA_ERR_HIP at the first launch.  tests/test_sanitize.py runs this file in a
process that preloads the AddressSanitizer and UndefinedBehaviorSanitizer
runtimes; a stray access or an arithmetic overflow in that host code aborts it.
"""
import ctypes

import pytest

import chunkwise_linear_rnn_amd as gla

if "hostsan" not in gla.LIB_PATH:
    pytest.skip("needs the host-sanitizer build (GLA_LIBRARY); run by tests/test_sanitize.py", allow_module_level=True)

ERR_HIP = 6
P = ctypes.c_void_p(0x10000)


def _shape(B, T, H, K, V, dtype=gla.GLA_DTYPE_BF16):
    return gla.GlaShape(B, T, H, K, V, 64, dtype, 0)


SHAPES = [(1, 256, 1, 64, 64, gla.GLA_DTYPE_FP32), (4, 1024, 8, 64, 64, gla.GLA_DTYPE_BF16),
          (8, 2048, 4, 128, 256, gla.GLA_DTYPE_BF16), (2, 8192, 4, 128, 256, gla.GLA_DTYPE_BF16),
          (2, 8192, 4, 256, 512, gla.GLA_DTYPE_BF16), (4, 16384, 16, 128, 128, gla.GLA_DTYPE_BF16),
          (2, 64 * 21, 16, 128, 256, gla.GLA_DTYPE_BF16), (1, 64, 1, 128, 128, gla.GLA_DTYPE_FP32),
          # heads run as key and value slices, or (general gates) padded to 128
          (1, 256, 2, 512, 512, gla.GLA_DTYPE_BF16), (1, 256, 2, 512, 256, gla.GLA_DTYPE_FP32),
          (1, 128, 2, 256, 512, gla.GLA_DTYPE_FP32), (1, 320, 2, 64, 512, gla.GLA_DTYPE_BF16)]


@pytest.mark.parametrize("B,T,H,K,V,dt", SHAPES)
def test_every_entry_point_plans_to_a_launch(B, T, H, K, V, dt):
    L = gla.lib()
    s = _shape(B, T, H, K, V, dt)
    big = 1 << 40
    assert L.gla_fwd(ctypes.byref(s), P, P, P, P, P, P, P, P, big, None) == ERR_HIP
    assert L.gla_bwd(ctypes.byref(s), P, P, P, P, P, P, P, P, P, P, P, P, P, big, None) == ERR_HIP
    ck = P if L.gla_ckpt_size(ctypes.byref(s)) else None
    for f, b in ((L.gla_fwd_ckpt, L.gla_bwd_ckpt), (L.gla_fwd_scalar_ckpt, L.gla_bwd_scalar_ckpt)):
        assert f(ctypes.byref(s), P, P, P, P, P, P, P, ck, P, big, None) == ERR_HIP
        assert b(ctypes.byref(s), P, P, P, P, P, ck, P, P, P, P, P, P, P, P, big, None) == ERR_HIP
    assert L.gla_fwd_scalar(ctypes.byref(s), P, P, P, P, P, P, P, P, big, None) == ERR_HIP
    assert L.gla_bwd_scalar(ctypes.byref(s), P, P, P, P, P, P, P, P, P, P, P, P, P, big, None) == ERR_HIP
    assert L.gla_decode(ctypes.byref(s), P, P, P, P, P, P, None) == ERR_HIP
    assert L.gla_decode_scalar(ctypes.byref(s), P, P, P, P, P, P, None) == ERR_HIP
    assert L.gla_decode_general(ctypes.byref(s), P, P, P, P, P, P, P, None) == ERR_HIP
    assert L.gla_out_gate(ctypes.byref(s), P, P, P, P, ctypes.c_float(1e-5), P, None) == ERR_HIP
    if dt == gla.GLA_DTYPE_BF16:
        assert L.gla_fwd_general(ctypes.byref(s), P, P, P, P, P, P, P, P, P, big, None) == ERR_HIP
        assert L.gla_bwd_general(ctypes.byref(s), *([P] * 15), big, None) == ERR_HIP
        gck = P if L.gla_general_ckpt_size(ctypes.byref(s)) else None
        assert L.gla_fwd_general_ckpt(ctypes.byref(s), P, P, P, P, P, P, P, P, gck, P, big, None) == ERR_HIP
        assert L.gla_bwd_general_ckpt(ctypes.byref(s), P, P, P, P, P, P, P, gck, P, P, *([P] * 6), P, big,
                                      None) == ERR_HIP
    if L.gla_fwd_workspace_size(ctypes.byref(s)) <= 32 << 20:
        assert L.gla_fwd_noalloc(ctypes.byref(s), P, P, P, P, P, P, P, None) == ERR_HIP


def test_launch_recorder_counts_without_events():
    # a recorder with capacity 0 only counts the launches the calls reach
    L = gla.lib()
    rec = gla.LaunchRecorder(0, 0, 0, 0, None, None, None)
    L.gla_set_launch_recorder(ctypes.byref(rec))
    try:
        s = _shape(2, 8192, 4, 128, 256)
        assert L.gla_fwd(ctypes.byref(s), P, P, P, P, None, P, None, P, 1 << 40, None) == ERR_HIP
    finally:
        L.gla_set_launch_recorder(None)
    assert rec.failed == 0
