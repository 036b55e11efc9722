"""bench.py's host-side logic (CPU): the command-line contract for more than
one GPU, and the kernel-code hash that decides whether the committed HBM
counter summary still describes the kernels."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_hash_ignores_comments_and_whitespace_only(tmp_path):
    src = open(bench.KERNEL_SOURCE).read()
    base = bench.kernel_source_hash()
    edited = tmp_path / "k.hip"
    edited.write_text("// a new leading comment\n" + src.replace("\n", "\n\n", 5) + "\n/* tail */\n")
    assert bench.kernel_source_hash(str(edited)) == base
    changed = tmp_path / "k2.hip"
    changed.write_text(src.replace("kThreads = 256", "kThreads = 512", 1))
    assert "kThreads = 256" in src
    assert bench.kernel_source_hash(str(changed)) != base


def test_committed_counter_summary_is_plausible():
    # null when the kernels changed since the counters were taken; otherwise
    # the combine's HBM bytes sit near its algorithmic bytes
    import synth
    traffic = bench.measured_traffic()
    if traffic is not None:
        wl = synth.BY_NAME["prefill"]
        algo = wl.T * (2 * wl.H * (wl.k + 1) + 8 * wl.k)
        assert 0.9 * algo < traffic < 1.5 * algo


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def test_shape_workloads_parse():
    wl = bench.shape_workload("shape:T=4096,H=2048,E=128,k=8,ep=8")
    assert (wl.T, wl.H, wl.E, wl.k, wl.ep, wl.R, wl.cap) == (4096, 2048, 128, 8, 8, 4096, None)
    assert wl.routing == "uniform" and wl.combine == "unweighted" and wl.expert == "identity"
    wl = bench.shape_workload("shape:T=64,H=128,E=8,k=2,ep=4,routing=zipf1.2,combine=weighted")
    assert wl.routing == "zipf1.2" and wl.combine == "weighted"
    for bad in ("shape:T=64,H=128", "shape:T=64,H=128,E=8,k=2,ep=4,colour=blue"):
        try:
            bench.shape_workload(bad)
        except SystemExit:
            continue
        raise AssertionError(f"{bad} accepted")


def test_cpu_baseline_suite_on_small_workloads():
    # one thread and two threads, median of 3 runs per op; the fused
    # workload also times its fused epilogue, and its step is dispatch + fused
    one = bench.cpu_baseline_suite(names=("tiny", "decode"), runs=3, threads=1)
    many = bench.cpu_baseline_suite(names=("tiny",), runs=3, threads=2)
    for res, threads in ((one, 1), (many, 2)):
        for name, r in res.items():
            assert r["threads"] == threads and r["tokens_per_s"] > 0
            assert r["dispatch_ms_p50"] > 0 and r["combine_ms_p50"] > 0
            assert r["step"] == "dispatch + combine"
    assert 1 <= bench.host_cores() <= 16


def test_summary_lists_every_workload():
    res = {"tokens_per_s": 1e6, "ms_per_step": 0.1, "step_hbm_frac": 0.7, "dispatch_gbs": 5000.0,
           "combine_gbs": 6000.0, "cold": {"hbm_frac_p50": 0.65}, "graph_ms_per_step": 0.01}
    ladder = {"rungs": {"1": {"roundtrip_us_p50": 7.5, "gbs_p50": 40.0}}}
    s = bench.summary(res, "prefill", {"decode": res, "ladder": ladder})
    assert list(s) == ["prefill", "decode", "ladder"]
    assert s["prefill"]["hbm_pct"] == 70.0 and s["prefill"]["cold_hbm_pct"] == 65.0
    assert s["decode"]["graph_ms_per_step"] == 0.01 and s["ladder"]["1"]["hbm_pct"] == 0.5


def test_unknown_workload_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "partials",
                          "--extras="], capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "unknown workload" in (res.stdout + res.stderr)


def test_dispatch_kernels_follow_the_library_thresholds():
    """The roofline's kernel label names the path the library takes: one
    launch up to 4096 copies, the single-pass kernel for the per-copy layout
    (bf16 or fp8) up to 65536, the routing + copy kernels otherwise."""
    assert bench.dispatch_kernels(1024, "copy", "bf16") == "dispatch_small_kernel"
    assert bench.dispatch_kernels(4096, "region", "fp8") == "dispatch_small_kernel"
    assert bench.dispatch_kernels(32768, "copy", "bf16").startswith("dispatch_onepass_kernel")
    assert bench.dispatch_kernels(65536, "copy", "bf16").startswith("dispatch_onepass_kernel")
    assert bench.dispatch_kernels(65544, "copy", "bf16") == "route_rank_kernel + dispatch_copy_kernel"
    assert bench.dispatch_kernels(32768, "region", "bf16") == "route_rank_kernel + dispatch_copy_kernel"
    assert bench.dispatch_kernels(16384, "copy", "fp8").startswith("dispatch_onepass_kernel")
    assert bench.dispatch_kernels(65544, "copy", "fp8") == "route_rank_kernel + dispatch_copy_kernel"
    assert bench.dispatch_kernels(16384, "region", "fp8") == "route_rank_kernel + dispatch_copy_kernel"


def _launch_constant(name):
    import re
    src = open(os.path.join(ROOT, "combine_moe_dispatch_03_amd", "csrc", "launch.h")).read()
    m = re.search(r"constexpr\s+\w+\s+" + name + r"\s*=\s*(\w+);", src)
    assert m, name
    v = m.group(1)
    return int(v) if v.isdigit() else _launch_constant(v)


def test_dispatch_kernels_match_the_library_constants():
    """The thresholds bench.py names kernels by are the library's own
    (launch.h), read from the source so that the two cannot drift apart."""
    small, onepass = _launch_constant("kSmallItems"), _launch_constant("kOnePassItems")
    assert bench.dispatch_kernels(small, "copy", "bf16") == "dispatch_small_kernel"
    assert bench.dispatch_kernels(small + 1, "copy", "bf16").startswith("dispatch_onepass_kernel")
    assert bench.dispatch_kernels(small + 1, "copy", "fp8").startswith("dispatch_onepass_kernel")
    assert bench.dispatch_kernels(onepass, "copy", "bf16").startswith("dispatch_onepass_kernel")
    assert bench.dispatch_kernels(onepass + 1, "copy", "bf16") == "route_rank_kernel + dispatch_copy_kernel"
    assert bench.dispatch_kernels(small + 1, "region", "bf16") == "route_rank_kernel + dispatch_copy_kernel"
    # the single pass's row-first window lies inside its range
    lo, hi = _launch_constant("kOnePassRowFirstFrom"), _launch_constant("kOnePassRowFirstItems")
    assert small < lo < hi <= onepass

