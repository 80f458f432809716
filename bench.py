"""Throughput benchmark of the GLA forward + backward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload metric_8k]
    python bench.py --decode            (the recurrent decode step, its own JSON line)

A step is one gla_fwd followed by one gla_bwd (all hot-path steps: chunk
cumsum, intra-chunk attention, state scan, output, state recompute, dS scan,
chunk gradients, gate gradient) over one batch of seeded synthetic inputs that
are resident in HBM before timing starts.  Prints one JSON line.

Timing: the headline is cold, the median of the K timed steps with every step
behind a read of a 512 MiB buffer (so the inputs do not sit in L2 or the
Infinity Cache); p10/p90 and the warm mean of K back-to-back steps are beside
it.  The box's attainable copy bandwidth and bf16 GEMM rate are measured too.

Roofline: the dominant kernel (largest share of step time, timed with HIP
events on the launch stream through the library's launch recorder) is
compared with the HBM peak using its algorithmic bytes (each input it needs read
once, each output written once; workspace traffic excluded).  The CPU baseline
is the fp64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2516.6
FP32_MFMA_PEAK_TFLOPS = 157.3
METRIC = "GLA fwd(+bwd) tokens/sec at T=8K, dk=128, dv=256; % of bf16 MFMA peak"
METRIC_SCALAR = "GLA scalar-gate fwd+bwd tokens/sec at T=8K, dk=128, dv=256"


def alg_bytes_per_token_head(kernel: str, K: int, V: int, e: int, P: int, P_bwd: int, dv_split: bool = False,
                             G: int = None, ckpt: bool = False, T: int = 0, final_state: bool = True):
    """Algorithmic HBM bytes per (token, head) of one launch of `kernel`.

    G is the number of log-gate values per token and head (K for per-column
    gates, 1 for a scalar gate; g and dg have G elements).  The backward's
    segment-state pass reads q, g, d_o of every segment instead of all but the
    first when the dv walk takes segments in halves (it then also needs each
    segment's midpoint state); with a checkpoint (ckpt) it runs only that
    backward direction, and with a checkpoint, 16-bit inputs and the dv walk
    in halves (`fused`) the dq walk forms it: it then also reads q and
    writes the 2 P_bwd half-segment states of K x V per head (T tokens).  The
    forward's segment pass skips the last segment unless the final state is
    asked for (16-bit inputs: the combine then forms S_T from every segment)."""
    G = K if G is None else G
    seg_frac = (1.0 if final_state and e == 2 else (P - 1) / P) if P > 1 else 0.0
    seg_frac_bwd = (P_bwd - 1) / P_bwd if P_bwd > 1 else 0.0
    fused = ckpt and dv_split and e == 2 and T > 0
    table = {
        "fwd_walk": e * (2 * K + G + 2 * V),            # q, k, g, v read; o written
        # k, g, v, d_o read; dq written (fused: q read, the half segments' dS* written)
        "bwd_dq_walk": e * (2 * K + G + 2 * V) + (e * K + 2 * P_bwd * K * V * e / T if fused else 0),
        "bwd_dk_walk": e * (4 * K + 2 * G + 2 * V),     # q, k, g, dq, v, d_o read; dk, dg written
        "bwd_dv_walk": e * (2 * K + G + 2 * V),         # q, k, g, d_o read; dv written
        "fwd_seg_state": e * (K + G + V) * seg_frac,    # k, g, v of the segments (above)
        # k, g, v of all but the last segment and q, g, d_o of all but the first (or all)
        "bwd_seg_states": None if fused else
        e * (K + G + V) * ((0.0 if ckpt else seg_frac_bwd) + (1.0 if dv_split else seg_frac_bwd)),
    }
    return table.get(kernel)


def fwd_flops_per_token_head(K, V, C=64):
    # 4KV for Q S and K^T V, plus the causal halves of the 64x64 intra-chunk products
    return 4 * K * V + (C + 1) * (K + V)


def bwd_flops_per_token_head(K, V, C=64):
    return 10 * K * V + (C + 1) * (3 * K + 2 * V)


def _segments(bh, n, blocks):
    P = max(1, 256 // (bh * blocks)) if bh * blocks > 0 else 1
    P = min(P, max(n, 1))
    seg_len = -(-n // P)
    return -(-n // seg_len)


def plan_segments(B, H, T, K, V, bf16):
    """Forward segments per head chosen by the library's launch plan (mirrors gla_plan.hpp)."""
    if bf16:
        cap = 256 if K <= 128 else 64
    else:
        cap = 128
    bv = min(V, cap)
    return _segments(B * H, T // 64, V // bv)


def plan_segments_bwd(B, H, T, K, V, bf16):
    """Backward segments per head (gla_plan.hpp's make_bwd_plan)."""
    bk = 64 if (not bf16 or V >= 128) else min(K, 128)
    nkb = K // bk
    cap = (256 if K <= 128 else 64) if bf16 else 128
    bv = min(V, cap)
    if nkb > 1 and V // nkb < bv:
        bv = V // nkb
    if bv < 64:
        bv = V if V < 64 else 64
    nvb = V // bv
    return _segments(B * H, T // 64, max(nvb, nkb))


def plan_dv_split(B, H, T, K, V, bf16):
    """Whether the dv walk covers each segment in two halves (gla_plan.hpp's dv_split)."""
    bk = 64 if (not bf16 or V >= 128) else min(K, 128)
    nkb = K // bk
    cap = (256 if K <= 128 else 64) if bf16 else 128
    bvs = min(V, cap)
    bv = bvs
    if nkb > 1 and V // nkb < bv:
        bv = V // nkb
    if bv < 64:
        bv = V if V < 64 else 64
    return bool(bf16) and plan_segments_bwd(B, H, T, K, V, bf16) > 1 and bvs == 2 * bv


# sources of the forward and backward step kernels (the recorded traffic is theirs)
STEP_SOURCES = ["gla_bwd.hip", "gla_chunk.hpp", "gla_device.hpp", "gla_fwd.hip", "gla_plan.hpp"]


def source_digest() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "chunkwise_linear_rnn_amd", "csrc")
    for name in STEP_SOURCES:
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str, units: int):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE counters,
    or None if none were taken for this kernel/workload or the sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None
    return k.get("bytes_per_launch")


# Kernel function (as rocprofv3 names it) -> the launch name the library's
# launch recorder reports for it (the keys of the bench line's "kernels").
LAUNCH_LABEL = {
    "gla_fwd_walk_pipe": "fwd_walk", "gla_fwd_walk": "fwd_walk", "gla_seg_state": "fwd_seg_state",
    "gla_seg_combine_fwd_split": "combine_fwd", "gla_seg_combine_fwd": "combine_fwd",
    "gla_seg_state_pair": "bwd_seg_states", "gla_seg_combine_bwd_split": "combine_bwd",
    "gla_seg_combine_bwd": "combine_bwd", "gla_bwd_dq_pipe": "bwd_dq_walk", "gla_bwd_dq": "bwd_dq_walk",
    "gla_bwd_dk_pipe": "bwd_dk_walk", "gla_bwd_dk": "bwd_dk_walk", "gla_bwd_dv_pipe": "bwd_dv_walk",
    "gla_bwd_dv": "bwd_dv_walk", "gla_fwd_wide_prep": "fwd_prep", "gla_fwd_wide_walk": "fwd_walk",
    "gla_fwd_general_vprep": "fwd_general_vprep", "gla_seg_combine_fwd_general": "combine_fwd_general",
    "gla_gate_anchor": "bwdg_gate_anchor", "gla_gate_grad_out": "bwdg_gate_out", "gla_scale_ds0": "bwdg_scale_ds0",
    "gla_state_copy": "state_copy", "gla_decode_kernel": "decode",
}


def _is_lib(name: str) -> bool:
    """A kernel of this library (rocprofv3 prints some names mangled, some demangled)."""
    return "3gla" in name or "gla::" in name


def _kernel_base(mangled: str) -> str:
    """The kernel's function name inside namespace gla, e.g. gla_bwd_dq_pipe."""
    import re
    m = re.search(r"3gla(?:12_GLOBAL__N_1)?(\d+)", mangled)  # also inside an anonymous namespace
    if m:
        n = int(m.group(1))
        return mangled[m.end():m.end() + n]
    m = re.search(r"(gla_[a-z0-9_]+)", mangled)
    return m.group(1) if m else mangled


def _demangle(names):
    import subprocess
    try:
        # GNU c++filt does not know the bfloat16 code DF16b: spell it as a vendor type
        fixed = [n.replace("DF16b", "u4bf16") for n in names]
        r = subprocess.run(["c++filt"], input="\n".join(fixed), capture_output=True, text=True, timeout=30)
        out = r.stdout.splitlines()
        if len(out) == len(names):
            return [x.replace("__hip_bfloat16", "bf16").replace("(anonymous namespace)::", "") for x in out]
    except (OSError, subprocess.SubprocessError):
        pass
    return list(names)


def _cxa_demangle(name: str):
    """libstdc++'s own demangling of `name` (what rocprofv3 prints), or None."""
    import ctypes
    try:
        lib = ctypes.CDLL("libstdc++.so.6")
        f = lib.__cxa_demangle
        f.restype = ctypes.c_void_p
        f.argtypes = [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
        st = ctypes.c_int()
        r = f(name.encode(), None, None, ctypes.byref(st))
        return ctypes.cast(r, ctypes.c_char_p).value.decode() if r else None
    except (OSError, AttributeError):
        return None


def _resolve_names(names, lib_path=None):
    """{name: display name}.  rocprofv3 writes most kernel names mangled, but
    demangles some itself, and libstdc++ misreads a bfloat16 template argument
    followed by a literal 1 (an `_Accum` type appears).  Such a name is mapped
    back to the library's kernel symbol whose libstdc++ demangling it is (the
    kernels' host-side launch stubs carry the same mangled names)."""
    import subprocess
    dem = dict(zip(names, _demangle(names)))
    bad = [n for n in names if "_Accum" in n]
    if not bad:
        return dem
    lib_path = lib_path or os.path.join(ROOT, "chunkwise_linear_rnn_amd", "libgla.so")
    try:
        out = subprocess.run(["nm", lib_path], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return dem
    syms = sorted(set(t.split()[-1] for t in out.splitlines() if "_ZN3gla" in t))
    back = {}
    for m in syms:
        d = _cxa_demangle(m)
        if d and "_Accum" in d:
            back[d] = m
    hits = [n for n in bad if n in back]
    for n, d in zip(hits, _demangle([back[n] for n in hits])):
        dem[n] = d
    return dem


def _short(demangled: str) -> str:
    """'void gla::f<a, b>(args)' -> 'f<a,b>'."""
    s = demangled
    if s.startswith("void "):
        s = s[5:]
    s = s.split("(")[0].replace("gla::", "").replace(" ", "")
    return s


def summarize_trace(csv_path, out_md, title, command):
    """Markdown table from a rocprofv3 --kernel-trace --stats kernel_stats.csv."""
    import csv
    rows = [r for r in csv.DictReader(open(csv_path)) if _is_lib(r["Name"])]  # the library's kernels
    dem = _resolve_names([r["Name"] for r in rows])
    names = [dem[r["Name"]] for r in rows]
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = ["# Kernel times: %s (MI355X, rocprofv3 kernel trace)" % title, "",
             "Command (from the repository root, `cd /tmp && export TMPDIR=/tmp` first):", "",
             "    " + command, "", "Source: `%s` (every dispatch of the library's kernels in the run; torch's cache "
             "scrub and fills are left out of the table and of the shares)." % os.path.basename(csv_path), "",
             "| kernel | launch name | calls | avg us | min us | max us | share of GPU time |",
             "|---|---|---|---|---|---|---|"]
    for r, n in sorted(zip(rows, names), key=lambda x: -float(x[0]["TotalDurationNs"])):
        base = _kernel_base(r["Name"])
        lines.append("| %s | %s | %s | %.1f | %.1f | %.1f | %.1f %% |" % (
            _short(n), LAUNCH_LABEL.get(base, "-"), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, 100.0 * float(r["TotalDurationNs"]) / total))
    open(out_md, "w").write("\n".join(lines) + "\n")


def _counter_rows(csv_path):
    """{(dispatch, kernel name): {counter: value}} from a counter_collection.csv."""
    import csv
    out = {}
    for r in csv.DictReader(open(csv_path)):
        key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        d = out.setdefault(key, {"_scratch": int(r["Scratch_Size"]), "_ns": int(r["End_Timestamp"]) -
                                 int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _per_kernel_means(rows):
    acc = {}
    for (_, name), d in rows.items():
        a = acc.setdefault(name, {"_n": 0})
        a["_n"] += 1
        for k, v in d.items():
            a[k] = a.get(k, 0.0) + v
    return {name: {k: (v / a["_n"] if k != "_n" else v) for k, v in a.items()} for name, a in acc.items()}


def summarize_traffic(fetch_csv, write_csv, cfetch_csv, cwrite_csv, workload, commands, out_json, out_md,
                      alg_mb=None):
    """HBM bytes per launch from FETCH_SIZE and WRITE_SIZE runs (KiB per dispatch),
    each scaled by what the same counter reads for a 1 GiB device copy."""
    copy_kib = 1 << 20
    cf = [d for (_, n), d in _counter_rows(cfetch_csv).items() if "copyBuffer" in n]
    cw = [d for (_, n), d in _counter_rows(cwrite_csv).items() if "copyBuffer" in n]
    fscale = copy_kib / max(d["FETCH_SIZE"] for d in cf)
    wscale = copy_kib / max(d["WRITE_SIZE"] for d in cw)
    fm = _per_kernel_means(_counter_rows(fetch_csv))
    wm = _per_kernel_means(_counter_rows(write_csv))
    kernels = {}
    for name in fm:
        if name not in wm or not _is_lib(name):  # the library's kernels only (not torch's scrub or fills)
            continue
        base = _kernel_base(name)
        label = LAUNCH_LABEL.get(base, base)
        f, w = fm[name]["FETCH_SIZE"] * fscale, wm[name]["WRITE_SIZE"] * wscale
        kernels[label] = {"kernel": name, "bytes_per_launch": (f + w) * 1024.0, "fetch_kib": f, "write_kib": w,
                          "dispatches": fm[name]["_n"]}
    rec = {"workload": workload, "source_digest": source_digest(), "fetch_scale": fscale, "write_scale": wscale,
           "kernels": kernels, "commands": commands}
    json.dump(rec, open(out_json, "w"), indent=1)
    lines = ["# HBM traffic per launch: %s (MI355X, rocprofv3 FETCH_SIZE / WRITE_SIZE)" % workload, "",
             "Each counter in its own run (from the repository root, `cd /tmp && export TMPDIR=/tmp` first):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", "Calibration: a 1 GiB device copy reads and writes 1048576 KiB; FETCH_SIZE is scaled x%.4f and "
              "WRITE_SIZE x%.4f to match." % (fscale, wscale),
              "Per-launch bytes = mean over dispatches of (FETCH_SIZE x fetch scale + WRITE_SIZE x write scale)"
              " x 1024.", "",
              "| kernel | fetch MB | write MB | HBM MB per launch | algorithmic MB | ratio |", "|---|---|---|---|---|---|"]
    total = 0.0
    for label, k in sorted(kernels.items(), key=lambda kv: -kv[1]["bytes_per_launch"]):
        alg = (alg_mb or {}).get(label)
        total += k["bytes_per_launch"]
        lines.append("| %s | %.1f | %.1f | %.1f | %s | %s |" % (
            label, k["fetch_kib"] * 1024 / 1e6, k["write_kib"] * 1024 / 1e6, k["bytes_per_launch"] / 1e6,
            "%.1f" % alg if alg else "-", "%.2f" % (k["bytes_per_launch"] / 1e6 / alg) if alg else "-"))
    lines += ["", "Sum over the kernels listed: %.1f MB." % (total / 1e6),
              "`%s` holds the same figures with the digest of the kernel sources they were taken from; bench.py "
              "reports them only while those sources are unchanged." % os.path.basename(out_json)]
    open(out_md, "w").write("\n".join(lines) + "\n")


def summarize_pmc(csv_path, trace_csv, out_md, title, command):
    """Per-kernel MFMA and LDS counters (means per dispatch) beside the
    kernel-trace durations: MfmaUtil = busy MFMA cycles over (GPU active cycles x
    1024 SIMDs); bf16 flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512."""
    import csv
    means = {n: m for n, m in _per_kernel_means(_counter_rows(csv_path)).items() if _is_lib(n)}
    dur = {r["Name"]: float(r["AverageNs"]) for r in csv.DictReader(open(trace_csv))}
    names = list(means)
    dem = _resolve_names(names)
    lines = ["# MFMA and LDS counters: %s (MI355X, rocprofv3 --pmc)" % title, "",
             "Command (from the repository root, `cd /tmp && export TMPDIR=/tmp` first):", "", "    " + command, "",
             "Durations from the kernel trace of the same workload (`%s`)." % os.path.basename(trace_csv),
             "MfmaUtil is rocprofv3's derived metric (MFMA busy cycles summed over the SIMDs / (GPU active cycles x "
             "1024 SIMDs) x 100).  MFMA TFLOP/s = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / trace duration; "
             "LDS conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.", "",
             "| kernel | launch name | MfmaUtil % | bf16 MFMA TFLOP/s | % of 2516.6 | MFMA insts | VALU insts | "
             "LDS insts | LDS conflict | scratch B/lane |", "|---|---|---|---|---|---|---|---|---|---|"]
    for n in sorted(names, key=lambda x: -dur.get(x, 0.0)):
        m = means[n]
        ns = dur.get(n)
        fl = m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        tf = fl / (ns * 1e-9) / 1e12 if ns else float("nan")
        conf = m.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(1.0, m.get("SQ_LDS_IDX_ACTIVE", 0.0))
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %.3g | %.3g | %.3g | %.2f | %d |" % (
            _short(dem[n]), LAUNCH_LABEL.get(_kernel_base(n), "-"), m.get("MfmaUtil", float("nan")), tf,
            100 * tf / BF16_MFMA_PEAK_TFLOPS, m.get("SQ_INSTS_MFMA", 0.0), m.get("SQ_INSTS_VALU", 0.0),
            m.get("SQ_INSTS_LDS", 0.0), conf, m["_scratch"]))
    open(out_md, "w").write("\n".join(lines) + "\n")


def summarize_stalls(csv_path, out_md, title, command):
    """Where the waves of each kernel spend their time, from one rocprofv3 pass
    of SQ counters (all per-SE sums; the ratios divide like units): the share
    of wave cycles spent waiting (SQ_WAIT_ANY) and waiting on LDS issue
    (SQ_WAIT_INST_LDS), LDS-active cycles per CU-busy cycle, and the bank
    conflict share of LDS-active cycles."""
    acc = {}
    for (_, name), d in _counter_rows(csv_path).items():
        if not _is_lib(name):
            continue
        a = acc.setdefault(name, {})
        for k, v in d.items():
            a[k] = a.get(k, 0.0) + v
    names = list(acc)
    dem = _resolve_names(names)
    lines = ["# Wave stalls and LDS use: %s (MI355X, rocprofv3 --pmc)" % title, "",
             "Command (from the repository root, `cd /tmp && export TMPDIR=/tmp` first):", "", "    " + command, "",
             "wait = SQ_WAIT_ANY / SQ_WAVE_CYCLES (both in quad-cycles); wait on LDS = SQ_WAIT_INST_LDS / "
             "SQ_WAVE_CYCLES; LDS busy = SQ_LDS_IDX_ACTIVE / (4 x SQ_BUSY_CU_CYCLES); conflicts = "
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; VALU = SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES (quad-cycles "
             "both).", "",
             "| kernel | launch name | wait | wait on LDS | LDS busy | LDS conflicts | VALU |", "|---|---|---|---|---|---|---|"]
    for n in names:
        d = acc[n]
        wave = max(1.0, d.get("SQ_WAVE_CYCLES", 0.0))
        busy = max(1.0, 4 * d.get("SQ_BUSY_CU_CYCLES", 0.0))
        lds = d.get("SQ_LDS_IDX_ACTIVE", 0.0)
        lines.append("| %s | %s | %.2f | %.2f | %.2f | %.2f | %.2f |" % (
            _short(dem[n]), LAUNCH_LABEL.get(_kernel_base(n), "-"), d.get("SQ_WAIT_ANY", 0.0) / wave,
            d.get("SQ_WAIT_INST_LDS", 0.0) / wave, lds / busy, d.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(1.0, lds),
            d.get("SQ_ACTIVE_INST_VALU", 0.0) / wave))
    open(out_md, "w").write("\n".join(lines) + "\n")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def attainable_peaks(torch, dev):
    """What this GPU reaches on plain library work, for scale: a 1 GiB
    device-to-device copy (read + write bytes per second) and an 8192^3 bf16
    matrix product (hipBLASLt through torch.matmul), each the best of 5 runs
    after one warm-up run, timed with HIP events."""
    def best(fn, reps=5):
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        fn()
        torch.cuda.synchronize()
        for a, b in e:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return min(a.elapsed_time(b) for a, b in e)
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms_copy = best(lambda: dst.copy_(src))
    del src, dst
    m = 8192
    a = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    b = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    c = torch.empty(m, m, device=dev, dtype=torch.bfloat16)
    ms_mm = best(lambda: torch.matmul(a, b, out=c))
    del a, b, c
    return {"copy_GBps": 2 * n / (ms_copy * 1e-3) / 1e9, "copy_frac_of_peak": 2 * n / (ms_copy * 1e-3) / 1e9 /
            HBM_PEAK_GBS, "gemm_bf16_TFLOPs": 2 * m ** 3 / (ms_mm * 1e-3) / 1e12,
            "gemm_frac_of_peak": 2 * m ** 3 / (ms_mm * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "what": "1 GiB device copy; 8192^3 bf16 torch.matmul; best of 5"}


def cpu_baseline(inputs, w, n_heads, scalar_gate=False):
    """fp64 oracle forward + backward on n_heads full-length heads of the workload."""
    import numpy as np
    import oracle

    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:n_heads]
    f64 = lambda t: t.detach().cpu().double().numpy()
    pick = lambda a: (np.stack([a[b, :, h] for b, h in heads])[:, :, None] if a.ndim == 3 else
                      np.stack([a[b, :, h, :] for b, h in heads])[:, :, None, :])
    q, k, v, g, do = (pick(f64(inputs[n])) for n in ("q", "k", "v", "g", "do"))
    threads = min(oracle.num_threads(), len(heads))
    os.environ["OMP_NUM_THREADS"] = str(threads)
    t0 = time.perf_counter()
    if scalar_gate:
        oracle.gla_fwd_scalar(q, k, v, g, None)
        oracle.gla_bwd_scalar(q, k, v, g, do, None, None)
    else:
        oracle.gla_fwd(q, k, v, g, None)
        oracle.gla_bwd(q, k, v, g, do, None, None)
    dt = time.perf_counter() - t0
    tokens_equiv = len(heads) * w.T / w.H  # a token of the workload carries H heads
    return {
        "value": tokens_equiv / dt,
        "unit": "tokens/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "host_cpus_available": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": "fp64 oracle fwd+bwd on %d of %d heads, full T=%d (%.1f s wall)" % (len(heads), w.B * w.H,
                                                                                  w.T, dt),
    }


def device_info(torch, dev):
    """The GPU and software the line was measured on."""
    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1), "hip": torch.version.hip, "torch": torch.__version__}


def decode_bench(args, torch, gla, gi):
    """gla_decode at serving shape: B sequences, one new token each per call.

    The state round-trips through HBM every call (fp32 read and write), so the
    kernel is HBM-bound: algorithmic bytes per call = B*H*(8*K*V + e*(3K + 2V))
    with a log gate per key column, e*(2K + 2V + 1) for the scalar gate and
    e*(3K + 3V) with the value-side gate h of the general form."""
    B, H, K, V = 64, 4, 128, 256
    sg, gen = args.scalar_gate, args.general_gate
    w = gi.custom(B, H, 1, K, V, dtype="bf16", gate="scalar" if sg else "lowrank", s0="normal0.1", backward=False,
                  seed=6)
    cpu = gi.make_inputs(w)
    if gen:
        cpu["h"] = gi.make_value_gate(B, 1, H, V, seed=7)
    dev = "cuda:0"
    d = {k: (v.to(dev) if v is not None else None) for k, v in cpu.items()}
    state = d["s0"].clone()
    o = torch.empty(B, 1, H, V, dtype=torch.bfloat16, device=dev)
    call = lambda: gla.gla_decode_into(d["q"], d["k"], d["v"], d["g"], state, o, h=d.get("h"), scalar_gate=sg)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(args.steps, 1) * 10
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    timer = gla.KernelTimer(n)
    with timer:
        for _ in range(n):
            call()
    kt = timer.read()
    kern_ms = kt["decode"][1] / kt["decode"][0]
    # cold: each call behind a 512 MiB read, so the 64 MiB state comes from HBM
    # (back to back, the state stays in the 256 MB Infinity Cache)
    scrub = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b_ in evs:
        scrub.sum()
        a.record()
        call()
        b_.record()
    torch.cuda.synchronize()
    cold = sorted(a.elapsed_time(b_) for a, b_ in evs)
    cold_ms = cold[len(cold) // 2]
    del scrub
    alg = B * H * (8 * K * V + 2 * ((2 * K + 2 * V + 1) if sg else (3 * K + 3 * V) if gen else (3 * K + 2 * V)))
    form = " scalar gate [B,T,H]," if sg else " general gate (g and h [B,T,H,V])," if gen else ""
    achieved = alg / (cold_ms * 1e-3) / 1e9
    line = {"metric": "GLA decode tokens/sec (recurrent form, one token per sequence per call)",
            "value": B / (cold_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "calls": n, "ms_per_call": cold_ms,
            "timing": "cold: median call behind a 512 MiB read; warm: mean of back-to-back calls",
            "ms_per_call_warm": ms, "kernel_us_warm": kern_ms * 1e3, "warm_tokens_per_s": B / (ms * 1e-3),
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "decode: B=64 H=4 dk=128 dv=256 bf16,%s fp32 state, 1 token per call" % form},
            "roofline": {"bound": "hbm", "kernel": "decode", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "alg_bytes_per_launch": alg,
                         "time": "cold call (HIP events around the single launch)"}}
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 2.0:
            f64 = lambda x: cpu[x].to(torch.float64).numpy()
            if gen:
                oracle.gla_fwd_general(*(f64(x) for x in ("q", "k", "v", "g", "h", "s0")))
            elif sg:
                oracle.gla_fwd_scalar(*(f64(x) for x in ("q", "k", "v", "g", "s0")))
            else:
                oracle.gla_fwd(*(f64(x) for x in ("q", "k", "v", "g", "s0")))
            reps += 1
        sec = (time.perf_counter() - t0) / reps
        line["cpu_baseline"] = {"value": B / sec, "unit": "tokens/s", "cores": oracle.num_threads(),
                                "kind": "oracle", "sample": "fp64 oracle, the full call (%d repetitions)" % reps}
    line["device"] = device_info(torch, "cuda:0")
    print(json.dumps(line), flush=True)


def out_gate_bench(args, torch, gla, gi):
    """gla_out_gate and gla_out_gate_bwd on the metric workload's output rows
    (B=2, T=8192, H=4, V=256, bf16: 65536 rows of one head each).

    Both are HBM-bound.  Algorithmic bytes per call: forward e*V*R*3 (o, z read,
    y written); backward e*V*R*5 (o, z, dy read, d_o, dz written)."""
    B, T, H, V = 2, 8192, 4, 256
    R = B * T * H
    cpu = gi.make_gate_inputs(B, T, H, V, "bf16", seed=6)
    dev = "cuda:0"
    d = {k: (v.to(dev) if v is not None else None) for k, v in cpu.items()}
    eps = 1e-5
    y = torch.empty_like(d["o"]); dx = torch.empty_like(d["o"]); dz = torch.empty_like(d["o"])
    dw = torch.empty(V, device=dev); db = torch.empty(V, device=dev)
    ws = gla.workspace(gla.gla_out_gate_bwd_workspace_size(B, T, H, V, torch.bfloat16), dev)
    fwd = lambda: gla.gla_out_gate_into(d["o"], d["z"], d["ln_w"], d["ln_b"], eps, y)
    bwd = lambda: gla.gla_out_gate_bwd_into(d["o"], d["z"], d["ln_w"], d["ln_b"], eps, d["dy"], dx, dz, dw, db, ws)
    step = lambda: (fwd(), bwd())
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n = max(args.steps, 1) * 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    timer = gla.KernelTimer(3 * n)
    with timer:
        for _ in range(n):
            step()
    kt = timer.read()
    kern = {k: {"launches": c, "avg_us": 1e3 * t / c} for k, (c, t) in kt.items()}
    alg_f, alg_b = 2 * V * R * 3, 2 * V * R * 5
    bwd_us = kern["out_gate_bwd"]["avg_us"]
    achieved = alg_b / (bwd_us * 1e-6) / 1e9
    line = {"metric": "GLA output epilogue rows/sec (per-head LayerNorm + Swish gate, forward + backward)",
            "value": R / (ms * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": n, "ms_per_step": ms,
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "out_gate: B=2 T=8192 H=4 V=256 bf16 (the metric workload's output), eps 1e-5"},
            "kernels": kern,
            "fwd_GBps": alg_f / (kern["out_gate_fwd"]["avg_us"] * 1e-6) / 1e9,
            "roofline": {"bound": "hbm", "kernel": "out_gate_bwd", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "alg_bytes_per_launch": alg_b}}
    if not args.no_cpu_baseline:
        import oracle
        rows = 4096  # a bounded sample of the rows (they are independent)
        f64 = lambda t: t.reshape(R, V)[:rows].to(torch.float64).numpy()
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 2.0:
            oracle.out_gate(f64(cpu["o"]), f64(cpu["z"]), cpu["ln_w"].double().numpy(), cpu["ln_b"].double().numpy(),
                            eps)
            oracle.out_gate_bwd(f64(cpu["o"]), f64(cpu["z"]), cpu["ln_w"].double().numpy(),
                                cpu["ln_b"].double().numpy(), eps, f64(cpu["dy"]))
            reps += 1
        sec = (time.perf_counter() - t0) / reps
        line["cpu_baseline"] = {"value": rows / sec, "unit": "rows/s", "cores": 1, "kind": "oracle",
                                "sample": "fp64 oracle forward + backward on %d of %d rows (%d repetitions)" % (
                                    rows, R, reps)}
    line["device"] = device_info(torch, "cuda:0")
    print(json.dumps(line), flush=True)


def fwd_only_bench(args, torch, gla, gi):
    """gla_fwd alone on any named workload (including those without backward
    inputs), reported as tokens/s, % of bf16 MFMA peak (algorithmic flops at
    C = 64) and % of HBM peak (compulsory bytes e(3K+2V) per token-head)."""
    w = gi.WORKLOADS[args.workload]
    if args.dims:
        # another head shape with the workload's recipe: "B,H,T,K,V"
        B_, H_, T_, K_, V_ = (int(x) for x in args.dims.split(","))
        w = gi.Workload("%s@%s" % (w.name, args.dims), B_, H_, T_, K_, V_, w.dtype, w.gate, w.v_scale, w.s0,
                        w.backward, w.seed)
    dev = "cuda:0"
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    dt = w.torch_dtype
    e = 2 if w.dtype == "bf16" else 4
    cpu = gi.make_inputs(w)
    d = {k: (v.to(dev) if v is not None else None) for k, v in cpu.items()}
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    sf = torch.empty(B, H, K, V, dtype=torch.float32, device=dev)
    general = args.general_gate
    if general:
        # general gates: a value-side log gate h [B,T,H,V] as well (gla_fwd_general)
        hv = gi.make_value_gate(B, T, H, V, dtype=w.dtype, seed=w.seed + 1).to(dev)
        ws = gla.workspace(gla.gla_fwd_general_workspace_size(B, T, H, K, V, dt), dev)
        fwd = lambda: gla.gla_fwd_general_into(d["q"], d["k"], d["v"], d["g"], hv, d["s0"], o, sf, ws)
    else:
        ws = gla.workspace(gla.gla_fwd_workspace_size(B, T, H, K, V, dt), dev)
        fwd = lambda: gla.gla_fwd_into(d["q"], d["k"], d["v"], d["g"], d["s0"], o, sf, ws)
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    n = max(args.steps, 1) * 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fwd()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    timer = gla.KernelTimer(16 * args.steps)
    with timer:
        for _ in range(args.steps):
            fwd()
    kt = timer.read()
    units = B * T * H
    peak_tf = BF16_MFMA_PEAK_TFLOPS if w.dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS
    flops = fwd_flops_per_token_head(K, V) * units
    op = "gla_fwd_general" if general else "gla_fwd"
    line = {"metric": "%s forward tokens/sec and %% of MFMA peak (%s)" % ("General GLA" if general else "GLA", w.name),
            "value": B * T / (ms * 1e-3),
            "unit": "tokens/s", "n_gpus": 1, "steps": n, "ms_per_step": ms, "higher_is_better": True,
            "dtype": w.dtype, "data": "synthetic",
            "config": {"workload": "%s: B=%d H=%d T=%d dk=%d dv=%d %s, %s per step" % (
                w.name, B, H, T, K, V, w.dtype, op)},
            "mfma_frac": flops / (ms * 1e-3) / (peak_tf * 1e12),
            "hbm_frac": e * (3 * K + (3 if general else 2) * V) * units / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "kernels": {k: {"launches": c, "avg_us": 1e3 * t / c} for k, (c, t) in kt.items()}}
    line["device"] = device_info(torch, "cuda:0")
    print(json.dumps(line), flush=True)


def general_step_bench(args, torch, gla, gi):
    """The general-gate (alpha^T beta) training pair gla_fwd_general_ckpt +
    gla_bwd_general_ckpt per step on --workload (K and V in {128, 256}), h drawn
    like g; tokens/s (warm mean of back-to-back steps), the recompute pair
    gla_fwd_general + gla_bwd_general beside it, and per-kernel times of the
    pair.  A measurement of that operator, not the headline metric."""
    w = gi.WORKLOADS[args.workload]
    dev = "cuda:0"
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    dt = w.torch_dtype
    cpu = gi.make_inputs(w, dht=True)
    d = {k: (v.to(dev) if v is not None else None) for k, v in cpu.items()}
    hv = gi.make_value_gate(B, T, H, V, dtype=w.dtype, seed=w.seed + 1).to(dev)
    do = d.get("do")
    if do is None:
        do = torch.randn(B, T, H, V, generator=torch.Generator().manual_seed(w.seed + 2)).to(dt).to(dev)
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    sf = torch.empty(B, H, K, V, dtype=torch.float32, device=dev)
    grads = [torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]), torch.empty_like(d["g"]),
             torch.empty_like(hv), torch.empty(B, H, K, V, dtype=torch.float32, device=dev)]
    wsf = gla.workspace(gla.gla_fwd_general_workspace_size(B, T, H, K, V, dt), dev)
    wsb = gla.workspace(gla.gla_bwd_general_workspace_size(B, T, H, K, V, dt), dev)
    ck = gla.workspace(gla.gla_general_ckpt_size(B, T, H, K, V, dt), dev)

    def step():
        gla.gla_fwd_general_ckpt_into(d["q"], d["k"], d["v"], d["g"], hv, d["s0"], o, sf, ck, wsf)
        gla.gla_bwd_general_ckpt_into(d["q"], d["k"], d["v"], d["g"], hv, d["s0"], o, ck, do, d["dht"], *grads, wsb)

    def step_recompute():
        gla.gla_fwd_general_into(d["q"], d["k"], d["v"], d["g"], hv, d["s0"], o, sf, wsf)
        gla.gla_bwd_general_into(d["q"], d["k"], d["v"], d["g"], hv, d["s0"], do, d["dht"], *grads, wsb)

    n = max(args.steps, 1)

    def mean_ms(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n
    ms = mean_ms(step)
    ms_re = mean_ms(step_recompute)
    timer = gla.KernelTimer(64 * args.steps)
    with timer:
        for _ in range(args.steps):
            step()
    kt = timer.read()
    line = {"metric": "General GLA fwd+bwd tokens/sec (%s)" % w.name, "value": B * T / (ms * 1e-3),
            "unit": "tokens/s", "n_gpus": 1, "steps": n, "ms_per_step": ms, "ms_per_step_recompute": ms_re,
            "timing": "warm: mean of back-to-back steps", "higher_is_better": True,
            "dtype": w.dtype, "data": "synthetic",
            "config": {"workload": "%s: B=%d H=%d T=%d dk=%d dv=%d %s, gla_fwd_general_ckpt + gla_bwd_general_ckpt "
                                   "per step" % (w.name, B, H, T, K, V, w.dtype)},
            "kernels": {k: {"launches": c, "avg_us": 1e3 * t / c} for k, (c, t) in kt.items()}}
    line["device"] = device_info(torch, "cuda:0")
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="metric_8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--recompute", action="store_true",
                    help="time gla_fwd + gla_bwd as the step (no checkpoint handed from forward to backward)")
    ap.add_argument("--no-attainable", action="store_true",
                    help="skip measuring the box's attainable copy bandwidth and bf16 GEMM rate")
    ap.add_argument("--cpu-heads", type=int, default=8)
    ap.add_argument("--decode", action="store_true",
                    help="measure gla_decode (one token per call, B=64 H=4 dk=128 dv=256 bf16) instead; with "
                         "--scalar-gate or --general-gate gla_decode_scalar or gla_decode_general")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time gla_fwd alone on --workload (also those without backward inputs)")
    ap.add_argument("--dims", default="",
                    help="with --fwd-only: B,H,T,K,V instead of the workload's head shape (same input recipe)")
    ap.add_argument("--general-gate", action="store_true",
                    help="time gla_fwd_general_ckpt + gla_bwd_general_ckpt on --workload (alpha^T beta gates, h drawn "
                         "like g); with --fwd-only the forward alone")
    ap.add_argument("--scalar-gate", action="store_true",
                    help="the workload with one log gate per token and head (gla_fwd_scalar / gla_bwd_scalar)")
    ap.add_argument("--out-gate", action="store_true",
                    help="measure the output epilogue (LayerNorm + Swish gate, fwd + bwd) on the metric "
                         "workload's output rows instead")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("KERNEL_STATS_CSV", "OUT_MD"),
                    help="write a profiles/ summary of a rocprofv3 kernel trace (no GPU needed)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                              "COPY_WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json/.md from FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("COUNTER_CSV", "KERNEL_STATS_CSV", "OUT_MD"),
                    help="write a profiles/ summary of MFMA / LDS counters")
    ap.add_argument("--summarize-stalls", nargs=2, metavar=("COUNTER_CSV", "OUT_MD"),
                    help="write a profiles/ summary of wave-stall and LDS counters")
    ap.add_argument("--step-only", action="store_true",
                    help="run no recompute pair beside the step (so that counter runs see the step's kernels only)")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", action="append", default=[],
                    help="the command(s) that produced the input files, quoted in the summary")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (to calibrate rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.title or args.workload,
                        " && ".join(args.command))
        return
    if args.summarize_stalls:
        summarize_stalls(args.summarize_stalls[0], args.summarize_stalls[1], args.title or args.workload,
                         " && ".join(args.command))
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.summarize_pmc[2],
                      args.title or args.workload, " && ".join(args.command))
        return
    if args.summarize_traffic:
        w = __import__("gla_inputs").WORKLOADS[args.workload]
        e = 2 if w.dtype == "bf16" else 4
        P = plan_segments(w.B, w.H, w.T, w.K, w.V, e == 2)
        Pb = plan_segments_bwd(w.B, w.H, w.T, w.K, w.V, e == 2)
        split = plan_dv_split(w.B, w.H, w.T, w.K, w.V, e == 2)
        alg = {}
        for k in ("fwd_walk", "bwd_dq_walk", "bwd_dk_walk", "bwd_dv_walk", "fwd_seg_state", "bwd_seg_states"):
            b = alg_bytes_per_token_head(k, w.K, w.V, e, P, Pb, split, T=w.T,
                                         ckpt=not args.recompute and w.dtype == "bf16" and w.K <= 128)
            if b:
                alg[k] = b * w.B * w.T * w.H / 1e6
        base = os.path.join(ROOT, "profiles", "traffic_%s" % args.workload)
        summarize_traffic(*args.summarize_traffic, args.workload, args.command, base + ".json", base + ".md", alg)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the path is sharded across GPUs by heads and by sequence "
              "segments, which this benchmark does not run (requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return

    import chunkwise_linear_rnn_amd as gla
    import gla_inputs as gi

    if args.decode:
        decode_bench(args, torch, gla, gi)
        return
    if args.out_gate:
        out_gate_bench(args, torch, gla, gi)
        return
    if args.general_gate and not args.fwd_only:
        general_step_bench(args, torch, gla, gi)
        return
    if args.fwd_only:
        fwd_only_bench(args, torch, gla, gi)
        return

    w = gi.WORKLOADS[args.workload]
    sg = args.scalar_gate
    if sg:  # same shape, seed and draws, with the scalar gate recipe
        w = gi.Workload(w.name, w.B, w.H, w.T, w.K, w.V, w.dtype, "scalar", w.v_scale, w.s0, w.backward, w.seed)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    dt = w.torch_dtype
    e = 2 if w.dtype == "bf16" else 4
    cpu_inputs = gi.make_inputs(w)
    if "do" not in cpu_inputs:
        raise SystemExit("workload %s has no backward inputs" % w.name)
    d = {k: (v.to(dev) if v is not None else None) for k, v in cpu_inputs.items()}
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    sf = torch.empty(B, H, K, V, dtype=torch.float32, device=dev)
    dq, dk = (torch.empty(B, T, H, K, dtype=dt, device=dev) for _ in range(2))
    dg = torch.empty(*d["g"].shape, dtype=dt, device=dev)
    dv = torch.empty(B, T, H, V, dtype=dt, device=dev)
    ds0 = torch.empty(B, H, K, V, dtype=torch.float32, device=dev)
    wsf = gla.workspace((gla.gla_fwd_scalar_workspace_size if sg else gla.gla_fwd_workspace_size)(
        B, T, H, K, V, dt), dev)
    wsb = gla.workspace((gla.gla_bwd_scalar_workspace_size if sg else gla.gla_bwd_workspace_size)(
        B, T, H, K, V, dt), dev)

    # The step is the checkpointed training pair when the shape has one (the
    # forward keeps each backward segment's starting state, the backward
    # starts from it); the recompute pair gla_fwd + gla_bwd is timed beside it.
    ck_bytes = 0 if args.recompute else gla.gla_ckpt_size(B, T, H, K, V, dt)
    ck = gla.workspace(ck_bytes, dev)

    def fwd_rc():
        gla.gla_fwd_into(d["q"], d["k"], d["v"], d["g"], d["s0"], o, sf, wsf, scalar_gate=sg)

    def bwd_rc():
        gla.gla_bwd_into(d["q"], d["k"], d["v"], d["g"], d["s0"], d["do"], None, dq, dk, dv, dg, ds0, wsb,
                         scalar_gate=sg)

    def fwd():
        if ck_bytes:
            gla.gla_fwd_ckpt_into(d["q"], d["k"], d["v"], d["g"], d["s0"], o, sf, ck, wsf, scalar_gate=sg)
        else:
            fwd_rc()

    def bwd():
        if ck_bytes:
            gla.gla_bwd_ckpt_into(d["q"], d["k"], d["v"], d["g"], d["s0"], ck, d["do"], None, dq, dk, dv, dg, ds0,
                                  wsb, scalar_gate=sg)
        else:
            bwd_rc()

    def step():
        fwd()
        bwd()

    def step_rc():
        fwd_rc()
        bwd_rc()

    def timed(fn, n):
        # warm: n back-to-back calls, inputs left in the caches by the previous call
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # cold: before every timed call a 512 MiB buffer is read, which evicts the
    # inputs from L2 and from the 256 MB Infinity Cache (a read leaves no dirty
    # lines to be written back during the timed call).  The read is enqueued
    # ahead of the call's start event, so the call's launches are queued while
    # it runs and the interval holds no host launch gap.
    scrub = torch.ones(128 << 20, dtype=torch.float32, device=dev)

    def cold_times(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            scrub.sum()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)

    def pct(xs, p):
        return xs[min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: exactly K steps (each behind a cache scrub)
    wall0 = time.perf_counter()
    cold = cold_times(step, args.steps)
    wall = time.perf_counter() - wall0
    ms_step = pct(cold, 50)
    ms_warm = timed(step, args.steps)
    cold_fwd = cold_times(fwd, args.steps)
    cold_bwd = cold_times(bwd, args.steps)
    ms_fwd, ms_bwd = pct(cold_fwd, 50), pct(cold_bwd, 50)
    ms_fwd_warm, ms_bwd_warm = timed(fwd, args.steps), timed(bwd, args.steps)
    cold_rc = cold_times(step_rc, args.steps) if (ck_bytes and not args.step_only) else cold
    del scrub

    # per-kernel HIP-event timing over another K steps (each kernel bracketed on
    # its launch stream by the library's launch recorder)
    timer = gla.KernelTimer(32 * args.steps)
    with timer:
        for _ in range(args.steps):
            step()
    kt = timer.read()
    kern = {n: {"launches": c, "avg_us": 1e3 * ms / c, "share": ms / max(1e-9, sum(x[1] for x in kt.values()))}
            for n, (c, ms) in kt.items()}
    dom = max(kern, key=lambda n: kern[n]["avg_us"] * kern[n]["launches"])
    P = plan_segments(B, H, T, K, V, w.dtype == "bf16")
    P_bwd = plan_segments_bwd(B, H, T, K, V, w.dtype == "bf16")
    units = B * T * H
    bpt = alg_bytes_per_token_head(dom, K, V, e, P, P_bwd, plan_dv_split(B, H, T, K, V, w.dtype == "bf16"),
                                   G=1 if sg else K, ckpt=bool(ck_bytes), T=T)
    roofline = None
    if bpt is not None:
        ach = bpt * units / (kern[dom]["avg_us"] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": ach / HBM_PEAK_GBS, "traffic": None if sg else load_traffic(w.name, dom, units),
                    "alg_bytes_per_launch": bpt * units}

    tokens = B * T
    value = tokens / (ms_step * 1e-3)
    fwd_flops = fwd_flops_per_token_head(K, V) * units
    peak_tf = BF16_MFMA_PEAK_TFLOPS if w.dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS
    out = {
        "metric": METRIC_SCALAR if sg else METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "timing": "cold: median over the K timed steps, each behind a 512 MiB cache scrub; warm: mean of K "
                  "back-to-back steps",
        "ms_per_step_p10": pct(cold, 10),
        "ms_per_step_p90": pct(cold, 90),
        "ms_per_step_warm": ms_warm,
        "warm_tokens_per_s": tokens / (ms_warm * 1e-3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": "%s: B=%d H=%d T=%d dk=%d dv=%d %s, %s per step" % (
            w.name, B, H, T, K, V, w.dtype,
            ("scalar gate [B,T,H], " if sg else "") +
            (("gla_fwd_scalar_ckpt + gla_bwd_scalar_ckpt" if sg else "gla_fwd_ckpt + gla_bwd_ckpt") +
             " (the backward starts its segments from the forward's states)" if ck_bytes else
             ("gla_fwd_scalar + gla_bwd_scalar" if sg else "gla_fwd + gla_bwd"))), "global_batch": B, "seq_len": T, "heads": H, "dk": K, "dv": V,
            "chunk": 64, "segments": P},
        "ms_per_step_recompute": pct(cold_rc, 50) if (ck_bytes and not args.step_only) else None,
        "recompute_step": ("gla_fwd_scalar + gla_bwd_scalar" if sg else "gla_fwd + gla_bwd") +
                          " (every state recomputed in the backward), cold median",
        "fwd_tokens_per_s": tokens / (ms_fwd * 1e-3),
        "bwd_tokens_per_s": tokens / (ms_bwd * 1e-3),
        "ms_fwd": ms_fwd,
        "ms_bwd": ms_bwd,
        "ms_fwd_p10_p90": [pct(cold_fwd, 10), pct(cold_fwd, 90)],
        "ms_bwd_p10_p90": [pct(cold_bwd, 10), pct(cold_bwd, 90)],
        "ms_fwd_warm": ms_fwd_warm,
        "ms_bwd_warm": ms_bwd_warm,
        "fwd_mfma_frac": fwd_flops / (ms_fwd * 1e-3) / (peak_tf * 1e12),
        "fwdbwd_mfma_frac": (fwd_flops + bwd_flops_per_token_head(K, V) * units) / (ms_step * 1e-3) /
                            (peak_tf * 1e12),
        "fwd_hbm_frac": e * (2 * K + (1 if sg else K) + 2 * V) * units / (ms_fwd * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "step_hbm_frac": e * (2 * K + (1 if sg else K) + 2 * V + 2 * K + (1 if sg else K) + 2 * V +
                              2 * K + (1 if sg else K) + V) * units / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "kernels": kern,
        "roofline": roofline,
        "wall_s_timed": wall,
        "device": device_info(torch, dev),
    }
    if not args.no_attainable:
        out["attainable"] = attainable_peaks(torch, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cpu_inputs, w, args.cpu_heads, scalar_gate=sg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
