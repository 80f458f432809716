"""Host check of the paired column layout of 16-bit LDS tiles (no GPU needed).

The dk walk's value tile and the dv walk's Kt tile are stored with the columns
of each 32-column block interleaved (``paired_col`` in gla_device.hpp), so that
an MFMA k-step that pairs two stacked accumulator tiles (k slots 0-3 from one
16-row tile, 4-7 from the next) reads its LDS operand as one 16-byte piece.
This compiles the header's host side with hipcc and checks, for the function as
written there: a permutation of every 32-column block, 4-column groups kept
whole (8-byte accesses of 4 columns stay contiguous), and lane group g's eight
k slots at positions 8g .. 8g+7.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SRC = r"""
#include "gla_device.hpp"
#include <cstdio>
int main() {
    using gla::paired_col;
    int bad = 0;
    for (int b = 0; b < 4; ++b) {
        bool seen[32] = {};
        for (int c = 0; c < 32; ++c) {
            const int p = paired_col(32 * b + c) - 32 * b;
            if (p < 0 || p >= 32 || seen[p]) ++bad; else seen[p] = true;
            if ((c & 3) && paired_col(32 * b + c) != paired_col(32 * b + c - 1) + 1) ++bad;
        }
    }
    for (int g = 0; g < 4; ++g)
        for (int e = 0; e < 8; ++e) {
            const int logical = e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
            if (paired_col(logical) != 8 * g + e) ++bad;
        }
    std::printf("%s\n", bad ? "bad" : "ok");
    return bad ? 1 : 0;
}
"""


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_paired_column_layout():
    d = tempfile.mkdtemp(prefix="gla_paired_")
    try:
        src = os.path.join(d, "paired.hip")
        exe = os.path.join(d, "paired")
        with open(src, "w") as f:
            f.write(SRC)
        cmd = [HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950", "-I",
               os.path.join(ROOT, "chunkwise_linear_rnn_amd", "csrc"), src, "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
        assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
    finally:
        shutil.rmtree(d, ignore_errors=True)
