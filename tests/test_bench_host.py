"""Host-side checks of bench.py's contract (no GPU needed)."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_flop_and_byte_counts():
    sys.path.insert(0, ROOT)
    import bench
    from transformer_scaled_dot_03_amd.workloads import WORKLOADS
    w = WORKLOADS["long_bf16_b1h16t16384d128"]
    assert bench.flops_per_step(w) == 4.0 * 16 * 16384 * 16384 * 128
    assert bench.flops_per_step(WORKLOADS["long_causal_bf16_b1h16t16384d128"]) == bench.flops_per_step(w) / 2
    assert bench.bwd_flops_per_step(w) == 2.5 * bench.flops_per_step(w)
    assert bench.compulsory_bytes(w) == 2 * 16 * (2 * 16384 * 128 + 2 * 16384 * 128)
    d = WORKLOADS["decode_bf16_b8h16k16384d128"]
    assert bench.decode_bytes(d, None) == 2 * 16 * (2 * 8 * 16384 * 128 + 2 * 8 * 128)


def test_traffic_figure_is_keyed_to_the_kernel_source():
    sys.path.insert(0, ROOT)
    import bench
    digest = bench.kernel_source_digest()
    assert len(digest) == 16
    # a mismatching digest gives no figure rather than a stale one
    assert bench.committed_traffic("long_bf16_b1h16t16384d128", "0" * 16) is None
    assert bench.committed_traffic("no_such_workload", digest) is None


def test_algorithmic_flops_count_exactly_the_allowed_pairs():
    sys.path.insert(0, ROOT)
    import bench
    from transformer_scaled_dot_03_amd.workloads import MASK_CAUSAL, MASK_KEYPAD, Workload
    # brute-force pair count on small shapes, every mask combination, Tq != Tk included
    for Tq, Tk in ((5, 7), (7, 5), (6, 6)):
        for mask in (0, MASK_CAUSAL, MASK_KEYPAD, MASK_CAUSAL | MASK_KEYPAD):
            w = Workload("t", 3, 2, Tq, Tk, 4, "bf16", mask, 0.5)
            lens = [0, 3, Tk + 4]   # clamped to [0, Tk] as the kernels do
            pairs = 0
            for b in range(w.B):
                L = min(max(lens[b], 0), Tk) if w.keypad else Tk
                pairs += sum(1 for i in range(Tq) for j in range(Tk) if j < L and (not w.causal or j <= i))
            assert bench.algorithmic_flops(w, lens) == 4.0 * w.h * w.d * pairs


def test_digest_ignores_comments_but_not_code():
    sys.path.insert(0, ROOT)
    import bench
    a = b"int f(int x) {  // doubles\n  return 2 * x; /* no\n overflow check */ }\n"
    b = b"int f(int x) {\n\n  return 2 * x;   }  // reworded note\n"
    c = b"int f(int x) { return 3 * x; }\n"
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(a) != bench.code_only(c)


FIXTURE = os.path.join(ROOT, "tests", "golden", "rocprof_enc_self_b32h8t256d64")
FIX_WORKLOAD = "enc_self_bf16_b32h8t256d64_keypad"


def _fixture_rows(sub):
    import csv
    with open(os.path.join(FIXTURE, sub, "run_counter_collection.csv"), newline="") as f:
        return list(csv.DictReader(f))


def _machine_lines(text):
    import re
    return dict(re.findall(r"^([a-z_]+):\s*(\S+)\s*$", text, flags=re.M))


def test_profile_summary_of_a_recorded_rocprofv3_run():
    """tests/golden/rocprof_enc_self_b32h8t256d64: rocprofv3 CSVs of the encoder key-padding forward
    (two kernel dispatches per counter pass, the calibration copies, a kernel trace), trimmed from a
    run of `bench.py --collect-profile` on an MI355X.  The summary must reproduce the figures computed
    here directly from the rows."""
    sys.path.insert(0, ROOT)
    import bench
    text = bench.summarize_profile(FIX_WORKLOAD, FIXTURE, digest="f" * 16)
    vals = _machine_lines(text)
    assert vals["kernel_source_digest"] == "f" * 16 and vals["workload"] == FIX_WORKLOAD

    kern = "attn_fwd_bf16_kernel<64, false, true>"
    rows = _fixture_rows("mfma")

    def per_dispatch(rs, counter, name):
        vals_ = {}
        for r in rs:
            if name in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals_[r["Dispatch_Id"]] = vals_.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        return list(vals_.values())

    busy = per_dispatch(rows, "SQ_VALU_MFMA_BUSY_CYCLES", kern)
    grbm = per_dispatch(rows, "GRBM_GUI_ACTIVE", kern)
    assert len(busy) == 2 and len(grbm) == 2
    # 1024 SIMDs and 8 XCDs, as the agent table of the run says
    util = (sum(busy) / 2 / 1024) / (sum(grbm) / 2 / 8)
    assert abs(float(vals["mfma_util"]) - util) < 1e-4

    def scaled(sub, counter):
        rs = _fixture_rows(sub)
        k = per_dispatch(rs, counter, kern)
        grids = {}
        for r in rs:
            if "copyBuffer" in r["Kernel_Name"]:
                grids.setdefault(int(r["Grid_Size"]), []).append(float(r["Counter_Value"]))
        cal = grids[max(grids)]        # the 256 MiB calibration copies, not the small input copy
        return (sum(k) / len(k)) * (256 * 1024 / (sum(cal) / len(cal))) * 1024

    rd, wr = scaled("fetch", "FETCH_SIZE"), scaled("write", "WRITE_SIZE")
    assert abs(float(vals["hbm_read_bytes_per_launch"]) - rd) <= 1.0
    assert abs(float(vals["hbm_write_bytes_per_launch"]) - wr) <= 1.0
    assert abs(float(vals["hbm_bytes_per_launch"]) - (rd + wr)) <= 2.0
    # the output is written once: 2 bytes per element of [32, 8, 256, 64]
    assert abs(wr - 32 * 8 * 256 * 64 * 2) / wr < 0.01
    # kernel time from the trace pass: the dispatches after the 30 warm-up launches
    import csv
    with open(os.path.join(FIXTURE, "trace", "run_kernel_trace.csv"), newline="") as f:
        durs = [float(r["End_Timestamp"]) - float(r["Start_Timestamp"]) for r in csv.DictReader(f)]
    assert abs(float(vals["kernel_us"]) - sum(durs[30:]) / len(durs[30:]) / 1e3) < 1e-3


def test_counter_summary_round_trip_is_keyed_to_the_kernel_source(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    digest = bench.kernel_source_digest()
    with open(bench.counters_path(FIX_WORKLOAD), "w") as f:
        f.write(bench.summarize_profile(FIX_WORKLOAD, FIXTURE, digest=digest))
    got = bench.committed_counters(FIX_WORKLOAD, digest)
    vals = _machine_lines(open(bench.counters_path(FIX_WORKLOAD)).read())
    assert got["mfma_util"] == float(vals["mfma_util"])
    assert bench.committed_traffic(FIX_WORKLOAD, digest) == float(vals["hbm_bytes_per_launch"])
    # figures taken on other kernel code are not reported
    assert bench.committed_counters(FIX_WORKLOAD, "0" * 16) is None


def test_profile_commands_put_the_program_right_after_the_double_dash():
    sys.path.insert(0, ROOT)
    import bench
    cmds = bench.profile_commands(FIX_WORKLOAD, "/tmp/x")
    assert [n for n, _ in cmds] == ["mfma", "fetch", "write", "trace"]
    for name, argv in cmds:
        assert argv[0] == "rocprofv3"
        i = argv.index("--")
        assert argv[i + 1] == sys.executable and argv[i + 2].endswith("bench.py")
        if name == "trace":
            assert "--kernel-trace" in argv and "--pmc" not in argv
        else:
            assert "--pmc" in argv and not any(a in argv for a in ("-s", "--sys-trace", "-r", "--runtime-trace"))


def test_summary_shows_the_output_directory_as_a_placeholder():
    """The passes write under an absolute directory of the host that ran them; the committed summary
    names it `<out>`, the argument given to --collect-profile."""
    sys.path.insert(0, ROOT)
    import bench
    text = bench.summarize_profile(FIX_WORKLOAD, FIXTURE, digest="f" * 16,
                                   commands=bench.profile_commands(FIX_WORKLOAD, FIXTURE))
    assert FIXTURE not in text and os.path.abspath(FIXTURE) not in text
    for sub in ("mfma", "fetch", "write", "trace"):
        assert f"-d <out>/{sub} " in text
    assert "-- python3 bench.py --workload " + FIX_WORKLOAD in text


BWD_FIXTURE = os.path.join(ROOT, "tests", "golden", "rocprof_bwd_enc_self_b32h8t256d64")


def _rows(fixture, sub, name):
    import csv
    with open(os.path.join(fixture, sub, name), newline="") as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, counter, name):
    vals = {}
    for r in rows:
        if name in r["Kernel_Name"] and r["Counter_Name"] == counter:
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(vals.values())


@pytest.mark.parametrize("kernel,kname", [("bwd_dq", "attn_bwd_dq_kernel<64, false, true>"),
                                          ("bwd_dkdv", "attn_bwd_dkdv_kernel<64, false, true>")])
def test_backward_profile_summary_of_a_recorded_rocprofv3_run(kernel, kname):
    """tests/golden/rocprof_bwd_enc_self_b32h8t256d64: rocprofv3 CSVs of `bench.py --collect-profile
    --profile-kernel bwd` on the encoder key-padding workload (attn_fwd_lse, then attn_bwd: the dQ and
    the dK/dV kernel), trimmed to two dispatches of each kernel per counter pass, the calibration
    copies and 34 traced launches of each.  Each kernel's summary must reproduce the figures computed
    here from its own rows only."""
    sys.path.insert(0, ROOT)
    import bench
    text = bench.summarize_profile(FIX_WORKLOAD, BWD_FIXTURE, digest="e" * 16, kernel=kernel)
    vals = _machine_lines(text)
    assert vals["kernel"] == kernel and vals["kernel_source_digest"] == "e" * 16
    assert text.startswith(f"# Counters: attn::{kname} on {FIX_WORKLOAD}")
    rows = _rows(BWD_FIXTURE, "mfma", "run_counter_collection.csv")
    busy = _per_dispatch(rows, "SQ_VALU_MFMA_BUSY_CYCLES", kname)
    grbm = _per_dispatch(rows, "GRBM_GUI_ACTIVE", kname)
    assert len(busy) == 2 and len(grbm) == 2
    util = (sum(busy) / 2 / 1024) / (sum(grbm) / 2 / 8)
    assert abs(float(vals["mfma_util"]) - util) < 1e-4

    def scaled(sub, counter):
        rs = _rows(BWD_FIXTURE, sub, "run_counter_collection.csv")
        k = _per_dispatch(rs, counter, kname)
        grids = {}
        for r in rs:
            if "copyBuffer" in r["Kernel_Name"]:
                grids.setdefault(int(r["Grid_Size"]), []).append(float(r["Counter_Value"]))
        cal = grids[max(grids)]
        return (sum(k) / len(k)) * (256 * 1024 / (sum(cal) / len(cal))) * 1024

    rd, wr = scaled("fetch", "FETCH_SIZE"), scaled("write", "WRITE_SIZE")
    assert abs(float(vals["hbm_bytes_per_launch"]) - (rd + wr)) <= 2.0
    # the dQ kernel writes dQ (bf16) plus two fp32 values per row; the dK/dV kernel dK and dV
    B, h, T, d = 32, 8, 256, 64
    want_wr = 2 * B * h * T * d + 8 * B * h * T if kernel == "bwd_dq" else 2 * 2 * B * h * T * d
    assert abs(wr - want_wr) / want_wr < 0.02
    durs = [float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            for r in _rows(BWD_FIXTURE, "trace", "run_kernel_trace.csv") if kname in r["Kernel_Name"]]
    assert len(durs) == 34
    assert abs(float(vals["kernel_us"]) - sum(durs[30:]) / 4 / 1e3) < 1e-3


def test_backward_summaries_are_keyed_to_the_backward_source(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    fwd, bwd = bench.kernel_source_digest("fwd"), bench.kernel_source_digest("bwd")
    assert fwd != bwd and fwd == bench.kernel_source_digest()
    for kern in ("bwd_dq", "bwd_dkdv"):
        with open(bench.counters_path(FIX_WORKLOAD, kern), "w") as f:
            f.write(bench.summarize_profile(FIX_WORKLOAD, BWD_FIXTURE, kernel=kern))
        assert os.path.basename(bench.counters_path(FIX_WORKLOAD, kern)).startswith(f"attn_{kern}_")
        got = bench.committed_counters(FIX_WORKLOAD, bwd, kern)
        assert got is not None and 0 < got["mfma_util"] < 1 and got["kernel_us"] > 0
        # figures taken on other code, or asked for under the forward's digest, are not reported
        assert bench.committed_counters(FIX_WORKLOAD, fwd, kern) is None
    assert bench.committed_counters(FIX_WORKLOAD, fwd, "fwd") is None   # no forward summary written here


def test_backward_profile_runs_keep_the_backward_leg():
    sys.path.insert(0, ROOT)
    import bench
    for name, argv in bench.profile_commands(FIX_WORKLOAD, "/tmp/x", backward=True):
        assert "--no-backward" not in argv and argv[argv.index("--") + 1] == sys.executable
    for name, argv in bench.profile_commands(FIX_WORKLOAD, "/tmp/x"):
        assert "--no-backward" in argv
