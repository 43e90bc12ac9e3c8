#!/usr/bin/env python3
"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one attn_fwd launch over the whole workload (default: B1 h16
Tq=Tk=16384 d128 bf16, unmasked: the non-causal long-sequence case the
throughput target is quoted on).  Inputs are generated once, seeded, and are
resident in device memory before the timed region.  Prints ONE JSON line:

  value      attention TFLOP/s, 4*B*h*Tq*Tk*d flops per step (halved for causal)
  roofline   matrix-core roofline of the kernel: achieved TFLOP/s from HIP
             events on the launch stream vs the 2.5 PFLOP/s dense-bf16 peak;
             traffic = HBM bytes per launch from the committed rocprofv3
             counter summary when it matches the current kernel source
  hbm        compulsory bytes (read Q, K, V once, write O once) / time vs 8 TB/s
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
             workload on this host's cores (reported, not a target)
  decode     single-row decode (attn_decode) on its own workload (default B8 h16,
             one query row per head against a 16384-entry K/V cache, d128):
             compulsory bytes (the valid K/V rows, q, out) / HIP-event time vs
             8 TB/s -- the decode step is bound by HBM
  weights    attn_fwd_weights on the decoder-causal workload (B16 h16 T1024
             d64): the fp32 weight matrix written per second; the weights
             kernel's time is the call's minus attn_fwd_lse's (both HIP events)
  mha        the multi-head wrapper (attn_mha_fwd) on B32 T1024 d_model 512 h8:
             weight transpose + projection GEMM + strided attention + W^O GEMM;
             TFLOP/s counts 2*B*d_model^2*(2 Tq + 2 Tk) projection flops plus the
             attention's 4*B*h*Tq*Tk*d
  backward   (bf16 workloads) the gradient pass on the same inputs: attn_bwd
             timed with HIP events after one attn_fwd_lse; TFLOP/s counts the
             algorithmic 10*B*h*Tq*Tk*d flops (halved for causal): recomputed
             scores, dP, dV, dQ, dK
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MFMA bf16 peak (B*h*T^2*d shapes), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix/vector peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
PROFILES = os.path.join(ROOT, "profiles")


# what the forward kernel is compiled from: its source, the device helpers it
# includes and its argument struct (the rest of attn_launch.h declares other kernels)
KERNEL_SOURCES = ["attn_fwd_kernel.hip", "attn_device.h"]
BWD_KERNEL_SOURCES = ["attn_bwd_kernel.hip", "attn_device.h"]
# kernels with committed counter summaries: the forward, and the two backward kernels
PROFILE_KERNELS = ("fwd", "bwd_dq", "bwd_dkdv")

# the forward workloads timed one by one in the `workloads` object (decode workloads are
# measured by their own kernels)
FORWARD_WORKLOADS = ["sdpa_f32_b1h8t64d64", "enc_self_bf16_b32h8t256d64_keypad",
                     "dec_causal_bf16_b16h16t1024d64", "cross_bf16_b16h16q512k1024d64_keypad",
                     "long_bf16_b1h16t16384d128", "long_causal_bf16_b1h16t16384d128"]


def code_only(src: bytes) -> bytes:
    """C++ source with comments removed and whitespace collapsed: edits to comments
    leave the compiled kernel, and so the digest, unchanged."""
    text = src.decode()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split()).encode()


def kernel_source_digest(kind: str = "fwd") -> str:
    """Short hash of the code of the forward kernel (kind "fwd") or of the two backward kernels
    ("bwd"): keys the committed counter data."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "transformer_scaled_dot_03_amd", "csrc")
    for name in (KERNEL_SOURCES if kind == "fwd" else BWD_KERNEL_SOURCES):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + code_only(f.read()))
    launch = open(os.path.join(csrc, "attn_launch.h"), "rb").read()
    struct = b"Params" if kind == "fwd" else b"BwdParams"
    m = re.search(rb"struct " + struct + rb" \{.*?\};", launch, flags=re.S)
    h.update(struct + b"\0" + code_only(m.group(0) if m else launch))
    return h.hexdigest()[:16]


def digest_kind(kernel: str) -> str:
    return "fwd" if kernel == "fwd" else "bwd"


def mfma_ceiling(torch, dev, blocks=512, iters=5000, reps=3):
    """What the bf16 matrix cores sustain here with random operands and no
    memory traffic (libmfma_probe.so), and the shader clock meanwhile."""
    import ctypes
    path = os.path.join(ROOT, "transformer_scaled_dot_03_amd", "libmfma_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.mfma_probe_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p]
    lib.mfma_probe_launch.restype = ctypes.c_int
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = None
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = lib.mfma_probe_launch(sink.data_ptr(), clocks.data_ptr(), blocks, iters, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if rc != 0:
            return None
        ms = e0.elapsed_time(e1)
        c = clocks.view(-1, 2).double()
        ghz = float((c[:, 0] / (c[:, 1] / 100e6)).mean()) / 1e9
        tflops = blocks * 4 * iters * 16 * 32768.0 / (ms * 1e-3) / 1e12
        if best is None or tflops > best["tflops"]:
            best = {"tflops": round(tflops, 1), "clock_ghz": round(ghz, 3)}
    best["what"] = ("v_mfma_f32_32x32x16_bf16 loop, random bf16 operands, no memory traffic, "
                    f"{blocks} work-groups x 4 waves, best of {reps}")
    return best


def counters_path(workload: str, kernel: str = "fwd") -> str:
    prefix = {"fwd": "attn_fwd", "bwd_dq": "attn_bwd_dq", "bwd_dkdv": "attn_bwd_dkdv"}[kernel]
    return os.path.join(PROFILES, f"{prefix}_{workload}_counters.md")


def committed_counters(workload: str, digest: str, kernel: str = "fwd"):
    """The machine-readable figures of the committed counter summary of `kernel` on `workload`
    (written by --summarize-profile), or None if it is missing or was taken on other
    kernel code (its digest differs)."""
    path = counters_path(workload, kernel)
    if not os.path.exists(path):
        return None
    vals = dict(re.findall(r"^([a-z_]+):\s*(\S+)\s*$", open(path).read(), flags=re.M))
    if vals.get("kernel_source_digest") != digest:
        return None
    out = {}
    for key in ("mfma_util", "hbm_bytes_per_launch", "hbm_read_bytes_per_launch", "hbm_write_bytes_per_launch",
                "valu_per_mfma", "lds_per_mfma", "kernel_clock_ghz", "kernel_us"):
        if key in vals:
            out[key] = float(vals[key])
    return out


def committed_traffic(workload: str, digest: str):
    """HBM bytes per launch from the committed counter summary, if it matches this kernel."""
    c = committed_counters(workload, digest)
    return None if c is None or "hbm_bytes_per_launch" not in c else c["hbm_bytes_per_launch"]


# ---------------------------------------------------------------------------
# rocprofv3 counter passes and their summaries
# ---------------------------------------------------------------------------

# one pass each (rocprofv3 does not split counters over passes): matrix-core and instruction counters, then
# the two HBM byte counters on their own
PMC_MFMA = ["SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
            "SQ_INSTS_SALU", "SQ_WAVES", "SQ_LDS_BANK_CONFLICT"]
PROFILE_ARGS = ["--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-mfma-probe", "--no-backward",
                "--no-decode", "--no-weights", "--no-mha", "--no-workloads"]
CALIBRATION_BYTES = 256 << 20   # --copy-calibration: a device copy reading and writing this many bytes


def profile_commands(workload: str, out_dir: str, backward: bool = False):
    """(name, argv) of the rocprofv3 runs behind one counter summary: the program itself after `--`.
    With backward=True the runs also time attn_bwd (both backward kernels) after the forward."""
    bench = [sys.executable, os.path.abspath(__file__), "--workload", workload]
    args = [a for a in PROFILE_ARGS if not (backward and a == "--no-backward")]
    runs = [("mfma", ["--pmc", *PMC_MFMA]), ("fetch", ["--pmc", "FETCH_SIZE"]), ("write", ["--pmc", "WRITE_SIZE"])]
    cmds = []
    for name, pmc in runs:
        cmds.append((name, ["rocprofv3", *pmc, "--output-format", "csv", "-d", os.path.join(out_dir, name), "-o", "run",
                            "--", *bench, *args, "--copy-calibration"]))
    # kernel time: the default warm-up and timed launches, nothing else
    cmds.append(("trace", ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
                           os.path.join(out_dir, "trace"), "-o", "run", "--", *bench, *args[4:]]))
    return cmds


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find_csv(d, name):
    for root, _dirs, files in os.walk(d):
        if name in files:
            return os.path.join(root, name)
    raise FileNotFoundError(f"{name} under {d}")


def forward_kernel_name(w) -> str:
    kind = "attn_fwd_bf16_kernel" if w.dtype == "bf16" else "attn_fwd_f32_kernel"
    return f"attn::{kind}<{w.d}, {str(w.causal).lower()}, {str(w.keypad).lower()}>"


def profiled_kernel_name(w, kernel: str) -> str:
    if kernel == "fwd":
        return forward_kernel_name(w)
    kind = {"bwd_dq": "attn_bwd_dq_kernel", "bwd_dkdv": "attn_bwd_dkdv_kernel"}[kernel]
    return f"attn::{kind}<{w.d}, {str(w.causal).lower()}, {str(w.keypad).lower()}>"


def kernel_bytes_and_flops(w, kernel: str):
    """(compulsory HBM bytes, what they are, flops per launch, what they count) of one launch of
    the profiled kernel on workload w (bf16 tensors, fp32 lse / D)."""
    rows, keys = w.B * w.h * w.Tq, w.B * w.h * w.Tk
    if kernel == "fwd":
        return (compulsory_bytes(w), "read Q, K, V, write O once", flops_per_step(w),
                "metric flops: 4 d per allowed pair")
    if kernel == "bwd_dq":
        return (2 * w.d * (3 * rows + 2 * keys) + 4 * rows + 2 * w.d * rows + 8 * rows,
                "read Q, dO, O, K, V and lse, write dQ and the per-row D and lse log2(e) once",
                1.5 * flops_per_step(w), "executed flops: S, dP and dQ, 6 d per allowed pair")
    return (2 * w.d * (2 * rows + 2 * keys) + 8 * rows + 2 * w.d * 2 * keys,
            "read Q, dO, K, V and the per-row D and lse log2(e), write dK and dV once",
            2.0 * flops_per_step(w), "executed flops: S, dP, dV and dK, 8 d per allowed pair")


def _per_dispatch(rows, kernel_substr):
    """{dispatch id: {counter: value}} for the dispatches of one kernel (values summed over dimensions)."""
    out = {}
    for r in rows:
        if kernel_substr in r["Kernel_Name"]:
            d = out.setdefault(int(r["Dispatch_Id"]), {"_grid": int(r["Grid_Size"])})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _mean(xs):
    xs = list(xs)
    return sum(xs) / len(xs)


def summarize_profile(workload: str, prof_dir: str, digest: str | None = None, commands=None,
                      kernel: str = "fwd") -> str:
    """Markdown summary of the counter passes under prof_dir (mfma/, fetch/, write/) for the forward
    kernel of `workload`, ending in machine-readable `key: value` lines that bench.py reads back
    (committed_counters).  HBM bytes: FETCH_SIZE and WRITE_SIZE per dispatch (KiB), each scaled by the
    factor that makes the same counter read the known bytes of the calibration copy in the same run."""
    from transformer_scaled_dot_03_amd.workloads import WORKLOADS
    w = WORKLOADS[workload]
    kname = profiled_kernel_name(w, kernel)
    agent = next(a for a in _read_csv(_find_csv(os.path.join(prof_dir, "mfma"), "run_agent_info.csv"))
                 if a["Agent_Type"] == "GPU")
    simds, xcds = int(agent["Simd_Count"]), int(agent["Num_Xcc"])
    rows = _read_csv(_find_csv(os.path.join(prof_dir, "mfma"), "run_counter_collection.csv"))
    disp = _per_dispatch(rows, kname)
    if not disp:
        raise ValueError(f"no dispatch of {kname} in {prof_dir}/mfma")
    missing = [k for k in PMC_MFMA if any(k not in d for d in disp.values())]
    if missing:
        raise ValueError(f"counters {missing} missing from {prof_dir}/mfma")
    c = {k: _mean(d[k] for d in disp.values()) for k in PMC_MFMA}
    dur_ns = _mean(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]) for r in rows
                   if kname in r["Kernel_Name"] and r["Counter_Name"] == "GRBM_GUI_ACTIVE")
    long_dispatch = dur_ns > 100e3
    busy_per_simd = c["SQ_VALU_MFMA_BUSY_CYCLES"] / simds
    cycles_per_xcd = c["GRBM_GUI_ACTIVE"] / xcds
    util = busy_per_simd / cycles_per_xcd
    valu_other = c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]   # SQ_INSTS_VALU counts the MFMAs too

    def scaled(sub, counter):
        rs = _read_csv(_find_csv(os.path.join(prof_dir, sub), "run_counter_collection.csv"))
        kern = [v[counter] for v in _per_dispatch(rs, kname).values()]
        copies = _per_dispatch(rs, "copyBuffer")
        big = max(v["_grid"] for v in copies.values())
        cal = [v[counter] for v in copies.values() if v["_grid"] == big]
        factor = (CALIBRATION_BYTES / 1024.0) / _mean(cal)
        return _mean(kern), factor, _mean(cal)

    # kernel time from the trace pass (when present): every dispatch of the kernel, and the timed ones
    trace_rows = []
    tdir = os.path.join(prof_dir, "trace")
    if os.path.isdir(tdir):
        trace_rows = [float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                      for r in _read_csv(_find_csv(tdir, "run_kernel_trace.csv")) if kname in r["Kernel_Name"]]
    fetch_kib, f_fac, f_cal = scaled("fetch", "FETCH_SIZE")
    write_kib, w_fac, w_cal = scaled("write", "WRITE_SIZE")
    rd = fetch_kib * f_fac * 1024.0
    wr = write_kib * w_fac * 1024.0
    comp, comp_what, kflops, flops_what = kernel_bytes_and_flops(w, kernel)
    pk = "" if kernel == "fwd" else " --profile-kernel bwd"
    lines = [
        f"# Counters: {kname} on {workload}",
        "",
        f"{w.desc}: B{w.B} h{w.h} Tq={w.Tq} Tk={w.Tk} d={w.d} {w.dtype}, causal={w.causal}, "
        f"key padding={w.keypad}.  {len(disp)} dispatches of the kernel per pass; means per dispatch.",
        "",
        f"Commands: `python3 bench.py --workload {workload} --collect-profile <out>{pk}` on an MI355X host "
        "runs these passes, each from /tmp with `TMPDIR=/tmp` (bench.py is the repository's, by its "
        "absolute path); the summary is "
        f"`python3 bench.py --summarize-profile <out> --workload {workload}"
        + ("" if kernel == "fwd" else f" --profile-kernel {kernel}") + "`:",
        "",
    ]
    out_prefix = os.path.abspath(prof_dir)

    def show(a):
        if a == sys.executable:
            return "python3"
        if a == os.path.abspath(__file__):
            return "bench.py"
        if os.path.isabs(a) and (a == out_prefix or a.startswith(out_prefix + os.sep)):
            return "<out>" + a[len(out_prefix):]
        return a

    for name, argv in (commands or profile_commands(workload, "<out>", backward=kernel != "fwd")):
        shown = [show(a) for a in argv]
        lines.append("    " + " ".join(shown))
    lines += [
        "",
        "| Quantity | Value | Reading |",
        "|---|---|---|",
        f"| SQ_INSTS_MFMA | {c['SQ_INSTS_MFMA']:.0f} | {c['SQ_INSTS_MFMA'] / c['SQ_WAVES']:.1f} per wave |",
        f"| SQ_VALU_MFMA_BUSY_CYCLES | {c['SQ_VALU_MFMA_BUSY_CYCLES']:.0f} | "
        f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / c['SQ_INSTS_MFMA']:.1f} busy cycles per MFMA; {busy_per_simd:.0f} per SIMD "
        f"({simds} SIMDs) |",
        f"| GRBM_GUI_ACTIVE | {c['GRBM_GUI_ACTIVE']:.0f} | {cycles_per_xcd:.0f} GPU cycles per XCD ({xcds} XCDs)"
        + (f"; {cycles_per_xcd / dur_ns:.3f} GHz over the {dur_ns / 1e3:.1f} us dispatch |" if long_dispatch else
           f" over a {dur_ns / 1e3:.1f} us dispatch (too short for a clock figure: the counter also runs "
           "around the dispatch) |"),
        f"| MFMA utilisation | {util:.4f} | busy cycles per SIMD / GPU cycles per XCD |",
        f"| SQ_INSTS_VALU (less MFMA) | {valu_other:.0f} | {valu_other / c['SQ_INSTS_MFMA']:.2f} per MFMA |",
        f"| SQ_INSTS_LDS | {c['SQ_INSTS_LDS']:.0f} | {c['SQ_INSTS_LDS'] / c['SQ_INSTS_MFMA']:.2f} per MFMA |",
        f"| SQ_INSTS_SALU | {c['SQ_INSTS_SALU']:.0f} | |",
        f"| SQ_LDS_BANK_CONFLICT | {c['SQ_LDS_BANK_CONFLICT']:.0f} | cycles |",
        f"| SQ_WAVES | {c['SQ_WAVES']:.0f} | |",
        f"| FETCH_SIZE | {fetch_kib:.1f} KiB | x {f_fac:.5f} (the calibration copy reads {CALIBRATION_BYTES} bytes, "
        f"FETCH_SIZE {f_cal:.1f} KiB) = {rd:.0f} bytes read |",
        f"| WRITE_SIZE | {write_kib:.1f} KiB | x {w_fac:.5f} (calibration WRITE_SIZE {w_cal:.1f} KiB) = {wr:.0f} "
        f"bytes written |",
        f"| HBM traffic | {rd + wr:.0f} bytes | {(rd + wr) / comp:.3f} x the compulsory {comp:.0f} ({comp_what}) |",
    ]
    timed = trace_rows[30:] if len(trace_rows) > 30 else trace_rows
    if trace_rows:
        first = trace_rows[:20]
        lines += [
            f"| kernel time (trace pass) | {_mean(timed) / 1e3:.2f} us | mean of the {len(timed)} timed launches "
            f"(after the 30 warm-up ones, back to back); all {len(trace_rows)}: min {min(trace_rows) / 1e3:.2f}, "
            f"max {max(trace_rows) / 1e3:.2f} us; launches 1-{len(first)}: mean {_mean(first) / 1e3:.2f} us |",
            f"| {'metric' if kernel == 'fwd' else 'executed'} throughput at that time | "
            f"{kflops / (_mean(timed) * 1e-9) / 1e12:.1f} TFLOP/s | "
            f"{kflops / (_mean(timed) * 1e-9) / 1e12 / PEAK_BF16_TFLOPS:.4f} of the {PEAK_BF16_TFLOPS:.0f} "
            f"TFLOP/s dense-bf16 peak ({kflops:.4g} {flops_what}) |",
        ]
    lines += [
        "",
        f"kernel_source_digest: {digest or kernel_source_digest(digest_kind(kernel))}",
        f"workload: {workload}",
        f"kernel: {kernel}",
        f"mfma_util: {util:.4f}",
        f"valu_per_mfma: {valu_other / c['SQ_INSTS_MFMA']:.3f}",
        f"lds_per_mfma: {c['SQ_INSTS_LDS'] / c['SQ_INSTS_MFMA']:.3f}",
        f"hbm_read_bytes_per_launch: {rd:.0f}",
        f"hbm_write_bytes_per_launch: {wr:.0f}",
        f"hbm_bytes_per_launch: {rd + wr:.0f}",
    ]
    if long_dispatch:
        lines.append(f"kernel_clock_ghz: {cycles_per_xcd / dur_ns:.3f}")
    if trace_rows:
        lines.append(f"kernel_us: {_mean(timed) / 1e3:.3f}")
    lines.append("")
    return "\n".join(lines)


def collect_profile(workload: str, out_dir: str, backward: bool = False) -> dict:
    """Run the counter passes (each rocprofv3 with this program after `--`, under a time limit) and
    return {kernel: summary}: the forward's, or with backward=True the two backward kernels'.
    This process itself never touches the GPU."""
    import subprocess
    env = dict(os.environ, TMPDIR="/tmp")
    cmds = profile_commands(workload, out_dir, backward=backward)
    for name, argv in cmds:
        print(f"bench.py: counter pass {name} for {workload}", file=sys.stderr, flush=True)
        r = subprocess.run(["timeout", "-s", "KILL", "180", *argv], cwd="/tmp", env=env,
                           stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"counter pass {name} failed ({r.returncode}): {r.stderr[-2000:]}")
    kernels = ("bwd_dq", "bwd_dkdv") if backward else ("fwd",)
    return {k: summarize_profile(workload, out_dir, commands=cmds, kernel=k) for k in kernels}


def flops_per_step(w) -> float:
    f = 4.0 * w.B * w.h * w.Tq * w.Tk * w.d
    return f / 2 if w.causal else f


def bwd_flops_per_step(w) -> float:
    """Algorithmic backward flops: five products of B*h*Tq*Tk*d multiply-adds (S recomputed, dP,
    dV, dQ, dK), 2.5 x the forward's two."""
    return 2.5 * flops_per_step(w)


def bwd_executed_flops(w) -> float:
    """Matrix-core flops the two backward kernels issue: the dQ kernel computes S, dP, dQ and the
    dK/dV kernel S, dP, dV, dK (S and dP twice), 3.5 x the forward's."""
    return 3.5 * flops_per_step(w)


def time_backward(torch, tsd, w, qd, kd, vd, kld, steps, warmup):
    """HIP-event time of one attn_bwd call (both kernels) on the workload."""
    dev = qd.device
    stream = torch.cuda.current_stream(dev)
    st = stream.cuda_stream
    mask = (tsd.MASK_CAUSAL if w.causal else 0) | (tsd.MASK_KEYPAD if w.keypad else 0)
    klp = None if kld is None else kld.data_ptr()
    from transformer_scaled_dot_03_amd.workloads import grad_output
    dout = grad_output(w.B, w.h, w.Tq, w.d, seed=0).to(dev)
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.h, w.Tq), dtype=torch.float32, device=dev)
    delta = torch.empty((2, w.B, w.h, w.Tq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    rc = tsd.attn_fwd_lse(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          w.B, w.h, w.Tq, w.Tk, w.d, w.d, w.scale, mask, klp, st)
    if rc != tsd.OK:
        raise RuntimeError(f"attn_fwd_lse failed: {tsd.attn_status_str(rc)}")
    args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), w.B, w.h, w.Tq, w.Tk, w.d, w.d,
            w.scale, mask, klp, st)

    def bstep():
        rc = tsd.attn_bwd(*args)
        if rc != tsd.OK:
            raise RuntimeError(f"attn_bwd failed: {tsd.attn_status_str(rc)}")

    for _ in range(warmup):
        bstep()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        bstep()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fl = bwd_flops_per_step(w)
    return {
        "what": "attn_bwd (dQ kernel + dK/dV kernel) after one attn_fwd_lse, same inputs, seeded dO",
        "ms": round(ms, 4),
        "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "flops_per_step": fl,
        "frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "executed_tflops": round(bwd_executed_flops(w) / (ms * 1e-3) / 1e12, 2),
        "peak": PEAK_BF16_TFLOPS,
        "steps": steps,
    }


def decode_bytes(w, key_lens) -> float:
    """Compulsory bytes of one decode step: each (b, head) reads its L_b valid K and V rows and
    its query row and writes one output row (bf16)."""
    rows = w.B * w.Tk if key_lens is None else int(key_lens.clamp(0, w.Tk).sum())
    return float(2 * w.h * (2 * rows * w.d + 2 * w.B * w.d))


def time_decode(torch, tsd, name, steps, warmup):
    """HIP-event time of attn_decode (split + merge kernels) on a decode workload."""
    from transformer_scaled_dot_03_amd.workloads import WORKLOADS, make_inputs
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    q, k, v, kl = make_inputs(w, seed=0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    kld = None if kl is None else kl.to(dev)
    del q, k, v
    out = torch.empty_like(qd)
    nbytes = tsd.attn_decode_workspace_bytes(w.B, w.h, w.Tk, w.d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    mask = tsd.MASK_KEYPAD if w.keypad else 0
    args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), w.B, w.h, w.Tk, w.d, w.d, w.scale, mask,
            None if kld is None else kld.data_ptr(), ws.data_ptr(), nbytes, stream.cuda_stream)

    def dstep():
        rc = tsd.attn_decode(*args)
        if rc != tsd.OK:
            raise RuntimeError(f"attn_decode failed: {tsd.attn_status_str(rc)}")

    for _ in range(warmup):
        dstep()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        dstep()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nb = decode_bytes(w, kl)
    gbs = nb / (ms * 1e-3) / 1e9
    return {
        "workload": name,
        "what": "attn_decode (split + merge kernels), one query row per (b, head), seeded inputs",
        "ms": round(ms, 4),
        "compulsory_bytes": nb,
        "achieved_GBs": round(gbs, 1),
        "peak_GBs": PEAK_HBM_GBS,
        "frac": round(gbs / PEAK_HBM_GBS, 4),
        "steps": steps,
    }


def time_weights(torch, tsd, name, steps, warmup):
    """HIP-event times of attn_fwd_weights and attn_fwd_lse on one workload; the difference is the
    weights kernel, which writes B*h*Tq*Tk fp32 values."""
    from transformer_scaled_dot_03_amd.workloads import WORKLOADS, make_inputs
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    q, k, v, kl = make_inputs(w, seed=0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    kld = None if kl is None else kl.to(dev)
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.h, w.Tq), dtype=torch.float32, device=dev)
    wts = torch.empty((w.B, w.h, w.Tq, w.Tk), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    mask = (tsd.MASK_CAUSAL if w.causal else 0) | (tsd.MASK_KEYPAD if w.keypad else 0)
    klp = None if kld is None else kld.data_ptr()
    head = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), lse.data_ptr())
    tail = (w.B, w.h, w.Tq, w.Tk, w.d, w.d, w.scale, mask, klp, stream.cuda_stream)

    def run(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def call_w():
        if tsd.attn_fwd_weights(*head, wts.data_ptr(), *tail) != tsd.OK:
            raise RuntimeError("attn_fwd_weights failed")

    def call_f():
        if tsd.attn_fwd_lse(*head, *tail) != tsd.OK:
            raise RuntimeError("attn_fwd_lse failed")

    ms_w = run(call_w)
    ms_f = run(call_f)
    ms_fill = run(lambda: wts.fill_(0.5))     # a plain write of the same bytes: the write ceiling here
    nbytes = float(w.B * w.h * w.Tq * w.Tk * 4)
    ms_k = max(ms_w - ms_f, 1e-6)
    return {
        "workload": name,
        "what": "attn_fwd_weights (forward + weights kernel); weights kernel = call minus attn_fwd_lse",
        "ms_call": round(ms_w, 4),
        "ms_forward": round(ms_f, 4),
        "ms_weights_kernel": round(ms_k, 4),
        "weights_bytes": nbytes,
        "achieved_GBs": round(nbytes / (ms_k * 1e-3) / 1e9, 1),
        "peak_GBs": PEAK_HBM_GBS,
        "frac": round(nbytes / (ms_k * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "fill_GBs": round(nbytes / (ms_fill * 1e-3) / 1e9, 1),
        "steps": steps,
    }


def time_mha(torch, tsd, name, steps, warmup):
    """HIP-event time of attn_mha_fwd on a multi-head workload."""
    from transformer_scaled_dot_03_amd.workloads import MHA_WORKLOADS, mha_inputs
    c = MHA_WORKLOADS[name]
    dev = torch.device("cuda:0")
    xq, _, _, wq, wk, wv, wo = (t.to(dev) for t in mha_inputs(c["B"], c["Tq"], c["Tk"], c["d_model"], seed=0))
    B, Tq, Tk, dm, h = c["B"], c["Tq"], c["Tk"], c["d_model"], c["heads"]
    y = torch.empty_like(xq)
    nb = tsd.attn_mha_workspace_bytes(B, Tq, Tk, dm)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    d = dm // h
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    args = (xq.data_ptr(), xq.data_ptr(), xq.data_ptr(), wq.data_ptr(), wk.data_ptr(), wv.data_ptr(), wo.data_ptr(),
            y.data_ptr(), B, Tq, Tk, dm, h, scale, tsd.MASK_CAUSAL if c["causal"] else 0, None, ws.data_ptr(), nb,
            stream.cuda_stream)

    def mstep():
        rc = tsd.attn_mha_fwd(*args)
        if rc != tsd.OK:
            raise RuntimeError(f"attn_mha_fwd failed: {tsd.attn_status_str(rc)}")

    for _ in range(warmup):
        mstep()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        mstep()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    proj = 2.0 * B * dm * dm * (2 * Tq + 2 * Tk)
    att = 4.0 * B * h * Tq * Tk * d / (2 if c["causal"] else 1)
    return {
        "workload": name,
        "what": "attn_mha_fwd: weight transpose, fused QKV projection GEMM, strided attention, W^O projection GEMM",
        "ms": round(ms, 4),
        "flops_per_step": proj + att,
        "tflops": round((proj + att) / (ms * 1e-3) / 1e12, 2),
        "frac": round((proj + att) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "peak": PEAK_BF16_TFLOPS,
        "steps": steps,
    }


def algorithmic_flops(w, key_lens) -> float:
    """4*d flops per (query row, allowed key) pair, counting exactly the allowed pairs:
    sum_b L_b keys per row under key padding, min(i+1, Tk) keys for row i under the causal mask."""
    import numpy as np
    Tq, Tk = w.Tq, w.Tk
    if w.keypad:
        lens = np.clip(np.asarray(key_lens), 0, Tk).astype(np.float64)
    else:
        lens = np.full(w.B, float(Tk))
    per_b = []
    for L in lens:
        if w.causal:
            i = np.arange(Tq, dtype=np.float64)
            per_b.append(np.minimum(i + 1, L).sum())
        else:
            per_b.append(Tq * L)
    return 4.0 * w.h * w.d * float(sum(per_b))


def time_workloads(torch, tsd, names, min_calls=100, min_seconds=1.0, max_calls=5000, cold_calls=100):
    """Each forward workload on its own: 20 warm-up calls, then every call timed alone with a pair
    of HIP events on the launch stream, at least `min_calls` and `min_seconds` of calls (at most
    `max_calls`); median and minimum per call.  Workloads whose compulsory bytes fit in the
    256 MiB last-level cache are also timed "cold": a 512 MiB device write between calls.  The
    oracle is timed beside each one on the host: whole when it is small, else on the seeded
    256-row subset of every head."""
    import statistics

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attention_fp64
    from transformer_scaled_dot_03_amd.workloads import WORKLOADS, make_inputs, sample_rows

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    st = stream.cuda_stream
    cores = len(os.sched_getaffinity(0))
    flush = None
    res = {}
    for name in names:
        w = WORKLOADS[name]
        q, k, v, kl = make_inputs(w, seed=0)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        kld = None if kl is None else kl.to(dev)
        out = torch.empty((w.B, w.h, w.Tq, w.d), dtype=qd.dtype, device=dev)
        fn = tsd.attn_fwd if w.dtype == "bf16" else tsd.attn_fwd_f32
        mask = (tsd.MASK_CAUSAL if w.causal else 0) | (tsd.MASK_KEYPAD if w.keypad else 0)
        args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), w.B, w.h, w.Tq, w.Tk,
                w.d, w.d, w.scale, mask, None if kld is None else kld.data_ptr(), st)

        def call():
            rc = fn(*args)
            if rc != tsd.OK:
                raise RuntimeError(f"attn_fwd failed on {name}: {tsd.attn_status_str(rc)}")

        def timed(n, between=None):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(min(n, 200))]
            ms = []
            while len(ms) < n:
                batch = evs[:min(len(evs), n - len(ms))]
                for e0, e1 in batch:
                    if between is not None:
                        between()
                    e0.record(stream)
                    call()
                    e1.record(stream)
                torch.cuda.synchronize()
                ms.extend(e0.elapsed_time(e1) for e0, e1 in batch)
            return ms

        for _ in range(20):
            call()
        torch.cuda.synchronize()
        probe = statistics.median(timed(20))
        n = int(min(max(min_calls, min_seconds * 1e3 / max(probe, 1e-6)), max_calls))
        ms = timed(n)
        med, mn = statistics.median(ms), min(ms)
        fl = flops_per_step(w)
        alg = algorithmic_flops(w, kl)
        cb = compulsory_bytes(w)
        r = {"calls": n, "median_ms": round(med, 5), "min_ms": round(mn, 5),
             "tflops": round(fl / (med * 1e-3) / 1e12, 2),
             "frac": round(fl / (med * 1e-3) / 1e12 / (PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS), 4),
             "algorithmic_tflops": round(alg / (med * 1e-3) / 1e12, 2),
             "hbm_GBs": round(cb / (med * 1e-3) / 1e9, 1)}
        cnt = committed_counters(name, kernel_source_digest())
        if cnt:
            # counter figures of this kernel code on this workload (profiles/), rocprofv3 passes
            r["mfma_util"] = cnt.get("mfma_util")
            r["hbm_traffic_bytes"] = cnt.get("hbm_bytes_per_launch")
            if cnt.get("hbm_bytes_per_launch"):
                r["measured_hbm_GBs"] = round(cnt["hbm_bytes_per_launch"] / (med * 1e-3) / 1e9, 1)
        if cb <= (256 << 20):
            if flush is None:
                flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
            cms = timed(cold_calls, between=lambda: flush.fill_(1.0))
            r["cold_median_ms"] = round(statistics.median(cms), 5)
            r["cold_min_ms"] = round(min(cms), 5)
        del qd, kd, vd, kld, out

        # the oracle beside it, on the same inputs
        qn, kn, vn = (t.float().numpy() for t in (q, k, v))
        kln = None if kl is None else kl.numpy()
        small = fl <= 40e9
        rows = None if small else sample_rows(w.Tq, 256, seed=0).numpy()
        with threadpool_limits(limits=cores):
            t0 = time.perf_counter()
            attention_fp64(qn, kn, vn, w.scale, causal=w.causal, key_lens=kln, rows=rows)
            el = time.perf_counter() - t0
        orc = {"seconds": round(el, 3), "cores": cores,
               "sample": "whole workload" if small else f"{len(rows)} seeded query rows x {w.B * w.h} heads"}
        if rows is not None:
            orc["rows_per_s"] = round(len(rows) * w.B * w.h / el, 1)
        if w.Tq * w.Tk * w.B * w.h <= 1 << 20:
            with threadpool_limits(limits=1):
                t0 = time.perf_counter()
                attention_fp64(qn, kn, vn, w.scale, causal=w.causal, key_lens=kln)
                orc["seconds_1_thread"] = round(time.perf_counter() - t0, 4)
        r["oracle"] = orc
        res[name] = r
    return res


def compulsory_bytes(w) -> float:
    es = 2 if w.dtype == "bf16" else 4
    return float(es * w.B * w.h * (2 * w.Tq * w.d + 2 * w.Tk * w.d))


def cpu_baseline(w, q, k, v, key_lens, budget_s: float):
    """fp64 oracle on a bounded sample: blocks of 256 query rows (seeded order),
    all heads, until `budget_s` of CPU time is spent."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attention_fp64

    cores = len(os.sched_getaffinity(0))
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    kl = None if key_lens is None else key_lens.numpy()
    order = np.random.default_rng(0).permutation(w.Tq)  # every row, seeded order
    done_rows = 0
    flops = 0.0
    t0 = time.perf_counter()
    with threadpool_limits(limits=cores):
        while done_rows < w.Tq:
            rows = np.sort(order[done_rows:done_rows + 256])
            attention_fp64(qn, kn, vn, w.scale, causal=w.causal, key_lens=kl, rows=rows)
            done_rows += rows.shape[0]
            if w.causal:
                kk = np.minimum(rows + 1, w.Tk).sum()
            else:
                kk = rows.shape[0] * w.Tk
            flops += 4.0 * w.B * w.h * float(kk) * w.d
            if time.perf_counter() - t0 >= budget_s:
                break
    el = time.perf_counter() - t0
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{done_rows} of {w.Tq} query rows (blocks of 256, seeded order) x "
                   f"{w.B * w.h} heads, fp64 NumPy/OpenBLAS, {el:.1f} s"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed launches first: the board settles to its power-limited clock over ~20")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the pure-MFMA ceiling measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-weights", action="store_true", help="skip the weights-output measurement")
    ap.add_argument("--no-mha", action="store_true", help="skip the multi-head wrapper measurement")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the per-workload forward timings (median / min / cold, oracle beside)")
    ap.add_argument("--decode-workload", default=None)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    ap.add_argument("--collect-profile", metavar="DIR", default=None,
                    help="run the rocprofv3 counter passes of --workload into DIR and write the summary to "
                         "profiles/ (this process starts rocprofv3 runs and touches no GPU itself)")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="print the summary of counter passes already in DIR (mfma/, fetch/, write/)")
    ap.add_argument("--profile-kernel", default="fwd", choices=("fwd", "bwd", "bwd_dq", "bwd_dkdv"),
                    help="which kernel the counter passes cover: the forward, or the backward (collect: "
                         "bwd, writing both backward summaries; summarize: bwd_dq or bwd_dkdv)"),
    args = ap.parse_args()

    if args.summarize_profile or args.collect_profile:
        from transformer_scaled_dot_03_amd.workloads import HEADLINE
        name = args.workload or HEADLINE
        if args.collect_profile:
            if args.profile_kernel not in ("fwd", "bwd"):
                ap.error("--collect-profile takes --profile-kernel fwd or bwd")
            texts = collect_profile(name, os.path.abspath(args.collect_profile), backward=args.profile_kernel == "bwd")
            for kern, text in texts.items():
                with open(counters_path(name, kern), "w") as f:
                    f.write(text)
                print(text)
        else:
            if args.profile_kernel == "bwd":
                ap.error("--summarize-profile takes --profile-kernel fwd, bwd_dq or bwd_dkdv")
            print(summarize_profile(name, args.summarize_profile, kernel=args.profile_kernel))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU (--gpus 1); multi-GPU runs are not "
              "supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import transformer_scaled_dot_03_amd as tsd
    from transformer_scaled_dot_03_amd.workloads import HEADLINE, WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    tsd.raw_library()  # loud failure if the HIP library is missing

    name = args.workload or HEADLINE
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    q, k, v, kl = make_inputs(w, seed=0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    kld = None if kl is None else kl.to(dev)
    out = torch.empty((w.B, w.h, w.Tq, w.d), dtype=qd.dtype, device=dev)
    stream = torch.cuda.current_stream(dev)
    fn = tsd.attn_fwd if w.dtype == "bf16" else tsd.attn_fwd_f32
    mask = (tsd.MASK_CAUSAL if w.causal else 0) | (tsd.MASK_KEYPAD if w.keypad else 0)
    ptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr())
    klp = None if kld is None else kld.data_ptr()
    st = stream.cuda_stream

    def step():
        rc = fn(*ptrs, w.B, w.h, w.Tq, w.Tk, w.d, w.d, w.scale, mask, klp, st)
        if rc != tsd.OK:
            raise RuntimeError(f"attn_fwd failed: {tsd.attn_status_str(rc)}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1) / args.steps       # average per launch, HIP events

    if args.copy_calibration:
        nbytes = 256 << 20
        a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(f"copy calibration: {nbytes} bytes read + {nbytes} bytes written per copy kernel",
              file=sys.stderr)

    ms_per_step = wall * 1e3 / args.steps
    fl = flops_per_step(w)
    value = fl / (ms_per_step * 1e-3) / 1e12
    achieved = fl / (ev_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    digest = kernel_source_digest()
    counters = committed_counters(name, digest) or {}
    traffic = counters.get("hbm_bytes_per_launch")
    cb = compulsory_bytes(w)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, recipe in workloads.py)",
        "config": {"workload": name, "B": w.B, "h": w.h, "Tq": w.Tq, "Tk": w.Tk, "d": w.d,
                   "causal": w.causal, "key_padding": w.keypad, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel_ms": round(ev_ms, 4), "kernel_source_digest": digest,
                     "mfma_util": counters.get("mfma_util"),
                     "counters": ("profiles/" + os.path.basename(counters_path(name))) if counters else None},
        "hbm": {"compulsory_bytes": cb, "achieved_GBs": round(cb / (ev_ms * 1e-3) / 1e9, 1),
                "measured_GBs": round(traffic / (ev_ms * 1e-3) / 1e9, 1) if traffic else None,
                "peak_GBs": PEAK_HBM_GBS},
    }
    if not args.no_backward and w.dtype == "bf16":
        rec["backward"] = time_backward(torch, tsd, w, qd, kd, vd, kld, args.steps, args.warmup)
        bd = kernel_source_digest("bwd")
        for kern in ("bwd_dq", "bwd_dkdv"):
            cnt = committed_counters(name, bd, kern)
            rec["backward"][kern] = None if cnt is None else {
                "mfma_util": cnt.get("mfma_util"), "hbm_bytes_per_launch": cnt.get("hbm_bytes_per_launch"),
                "kernel_us": cnt.get("kernel_us"), "kernel_source_digest": bd,
                "counters": "profiles/" + os.path.basename(counters_path(name, kern))}
    if not args.no_decode:
        from transformer_scaled_dot_03_amd.workloads import DECODE_HEADLINE
        rec["decode"] = time_decode(torch, tsd, args.decode_workload or DECODE_HEADLINE, args.steps, args.warmup)
    if not args.no_weights:
        rec["weights"] = time_weights(torch, tsd, "dec_causal_bf16_b16h16t1024d64", args.steps, args.warmup)
    if not args.no_mha:
        rec["mha"] = time_mha(torch, tsd, "mha_self_bf16_b32t1024dm512h8", args.steps, args.warmup)
    if not args.no_workloads:
        rec["workloads"] = time_workloads(torch, tsd, FORWARD_WORKLOADS)
    if not args.no_mfma_probe and w.dtype == "bf16":
        rec["mfma_ceiling"] = mfma_ceiling(torch, dev)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, kl, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
