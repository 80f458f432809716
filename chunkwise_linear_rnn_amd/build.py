"""Build ``libgla.so`` (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m chunkwise_linear_rnn_amd.build`` (or ``build()`` from Python).
Objects go to ``_build/`` at the repository root; the shared library is written
next to this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgla.so")

SOURCES = ["gla_api.cpp", "gla_timing.cpp", "gla_fwd.hip", "gla_fwd_wide.hip", "gla_bwd.hip", "gla_decode.hip",
           "gla_gate.hip", "gla_bwd_general.hip", "gla_noalloc.hip", "gla_split.hip"]
ARCH = os.environ.get("GLA_OFFLOAD_ARCH", "gfx950")

# Packed-fp32 VALU forms are kept out of the generated code on purpose.  The
# register tiles that carry the next chunk's prefetch are private arrays; LLVM's
# promote-alloca pass would otherwise move them into LDS (a global load, a wait
# and an LDS write at the prefetch point), which defeats the prefetch.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-disable-promote-alloca-to-lds",
          "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


# Per-file additions.  The wide-head forward keeps its MFMA accumulators (the
# state) in VGPRs: it decays the state with vector multiplies every chunk.
EXTRA = {"gla_fwd_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + COMMON + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source and link libgla.so.  Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(BUILD, "libgla_hostsan.so")


def build_host_sanitized(verbose: bool = False) -> str:
    """The ABI layer (validation, launch plans, workspace sizes, launch recorder)
    built by the host compiler with AddressSanitizer and UndefinedBehaviorSanitizer,
    its kernel launchers replaced by host stubs that report hipErrorNoDevice
    (``csrc/gla_host_stubs.cpp``).  No GPU code is compiled.  Load it in place
    of libgla.so by setting GLA_LIBRARY to the returned path, in a process that
    preloads the sanitizer runtime."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = [os.path.join(CSRC, f) for f in ("gla_api.cpp", "gla_timing.cpp", "gla_host_stubs.cpp")]
    tmp = SAN_LIB + ".tmp%d" % os.getpid()
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
            "-I", os.path.join(ROOT, "include")] + SANITIZE + srcs +
           ["-L", "/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", tmp])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitizer build failed:\n%s" % r.stderr)
    os.replace(tmp, SAN_LIB)
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
