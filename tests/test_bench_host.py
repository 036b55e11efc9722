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


def test_cpu_baselines_on_the_tiny_workload():
    # both CPU legs run the oracle on the same batch; the all-cores one
    # counts every thread's batches over the wall time
    import synth
    wl = synth.BY_NAME["tiny"]
    one = bench.cpu_baseline(wl, seconds=0.2)
    many = bench.cpu_baseline_all_cores(wl, threads=2, seconds=0.2)
    assert one["cores"] == 1 and many["cores"] == 2
    for res in (one, many):
        assert res["kind"] == "oracle" and res["unit"] == "tokens/s" and res["value"] > 0
    assert 1 <= bench.host_cores() <= 16


def test_unknown_workload_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "partials",
                          "--extras="], capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "unknown workload" in (res.stdout + res.stderr)
