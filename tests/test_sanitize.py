"""Host sanitizer run (CPU only): the ABI layer's validation and launch
planning and the fp64 oracle, built with AddressSanitizer and
UndefinedBehaviorSanitizer, under the ABI tests, the planning tests and every
oracle pin.  The kernels are not part of this build (the launchers are stubs);
GPU code is never built with a sanitizer."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["g++", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc/g++")
def test_host_code_under_asan_ubsan():
    from chunkwise_linear_rnn_amd import build
    import oracle
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    lib = build.build_host_sanitized()
    olib = oracle.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=asan + ":" + ubsan, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1", GLA_LIBRARY=lib, GLA_ORACLE_LIBRARY=olib)
    tests = ["tests/test_abi.py", "tests/hostsan_planning.py"] + sorted(
        os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests")) if f.startswith("test_oracle_"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + tests,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out and "skipped" not in out, out[-2000:]
