"""Benchmark of the MoE dispatch + combine hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]

A step is one pass of the hot path over one batch of synthetic input already
resident in HBM: dispatch (route + stable scan + row copies) -> identity
expert stage (the expert outputs are the dispatched rows, in place) ->
combine (reduce once).  On the fused workload the combine is the fused
combine + residual add + RMSNorm.  W untimed steps, then K timed steps
bracketed by device synchronisation (``value``, ``ms_per_step``), then K more
steps with HIP events recorded around every launch (the per-kernel
durations; ``ms_per_step_instrumented`` shows what the events themselves
cost).  One JSON line is printed.

``value`` is tokens/s of the headline workload (prefill: 4096 tokens,
hidden 7168, top-8 of 256 experts over 8 regions, unweighted combine).  The
line also carries:
  roofline      the phase that takes longer of the two: the dispatch call
                (one C call, timed as one, whichever kernels it launches:
                dispatch_small_kernel, dispatch_onepass_kernel, or
                route_rank_kernel + dispatch_copy_kernel) or the combine
                (combine_kernel), with HIP
                events on the launch stream in the instrumented steps,
                against MI355X's 8 TB/s HBM peak: algorithmic bytes per call
                / mean call time; ``traffic`` is the measured HBM bytes per
                call from the committed rocprofv3 counter summary, or null
                if the kernel source has changed since those counters were
                taken
  cpu_baseline  the CPU oracle (plain scalar C, its -O3 -march=native build
                compiled on this host) on the headline workload, one thread:
                dispatch + combine, each the median of 5 runs; with the
                per-workload medians (prefill, skewed, fused; dispatch,
                combine, fused epilogue) behind it, and the headline
                workload on every core this process may use (at most 16:
                cpu_baseline_all_cores)
  cold          per-kernel p50 / mean over --cold-iters launches, each after
                an untimed 1 GiB read that evicts the 256 MB Infinity Cache
  workloads     the same step on the skewed, decode and fused workloads (decode
                also replayed from a captured HIP graph, ``graph_*``), and
                on prefill and skewed under the per-region layout (one row per
                token and destination region, the form the FlashInfer pages
                measure; unweighted combine of per-region messages), and with
                the fp8 dispatch payload (e4m3 codes + one scale per row; the
                combine reads the experts' bf16 outputs); decode and the
                ladder run at least 100 timed steps whatever --steps is
  summary       last in the line: tokens/s and % of the HBM peak of every
                workload, warm and cold, and of each phase
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
GRAPH_STEPS = 10               # decode steps per captured graph
SMALL_STEPS = 100              # timed steps of the launch-bound workloads (decode, ladder), at least
PROFILES = {"combine": os.path.join(ROOT, "profiles", "combine_prefill_counters.txt"),
            "dispatch": os.path.join(ROOT, "profiles", "dispatch_prefill_counters.txt")}
KERNEL_SOURCE = os.path.join(ROOT, "combine_moe_dispatch_03_amd", "csrc", "kernels.hip")


def kernel_source_hash(path: str = KERNEL_SOURCE) -> str:
    """SHA-256 of the kernel source with comments removed and whitespace
    collapsed: a counter summary stays valid across comment edits, and no
    longer matches after any change to the code itself."""
    with open(path) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def measured_traffic(phase: str = "combine"):
    """HBM bytes per launch of the combine, or per dispatch call (routing +
    copy kernels), from the committed counter summary of the prefill
    workload, if the kernels are unchanged since it was taken."""
    path = PROFILES[phase]
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_code_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


class HipEvents:
    """HIP events on the runtime torch already loaded, created with
    hipEventDisableSystemFence: recording one then writes a timestamp without
    the system-scope cache writeback a default event performs, which would
    otherwise stall the queue for several microseconds at every record."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        path = next(line.split()[-1] for line in open("/proc/self/maps")
                    if "libamdhip64" in line.split()[-1])
        lib = ctypes.CDLL(path)
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib = lib

    def create(self) -> ctypes.c_void_p:
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return ev

    def record(self, ev, stream_handle: int) -> None:
        rc = self.lib.hipEventRecord(ev, ctypes.c_void_p(stream_handle))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, ev) -> None:
        self.lib.hipEventDestroy(ev)


def dispatch_kernels(items: int, layout: str, payload: str) -> str:
    """The kernels one dispatch call launches for `items` routed copies
    (the library's size thresholds: single launch up to 4096 copies; the
    single-pass kernel for the per-copy layout, either payload, up to 65536)."""
    if items <= 4096:
        return "dispatch_small_kernel"
    if layout == "copy" and items <= 65536:
        return "dispatch_onepass_kernel (routing blocks + copy blocks, one launch)"
    return "route_rank_kernel + dispatch_copy_kernel"


def describe(wl, cap) -> str:
    mode = {"weighted": "weighted combine", "unweighted": "unweighted combine",
            "both": "weighted combine", "fused": "weighted combine + residual + RMSNorm"}[wl.combine]
    return (f"{wl.name}: T={wl.T} H={wl.H} E={wl.E} top-{wl.k} ep={wl.ep} cap={cap} "
            f"rung={wl.R} {wl.routing} routing, {mode}")


def measure(wl, steps: int, warmup: int, cold_iters: int = 100, seed: int = 0,
            layout: str = "copy", payload: str = "bf16", graph: bool = False) -> dict:
    import numpy as np
    import torch

    import combine_moe_dispatch_03_amd as moe
    import synth

    dev = torch.device("cuda:0")
    inp = synth.make_inputs(wl, seed)
    x = torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.bfloat16)
    ids = torch.from_numpy(inp.ids).to(dev)
    # the per-region layout's combine is an unweighted sum of per-region messages
    weighted = wl.combine in ("weighted", "both", "fused") and layout == "copy"
    w = torch.from_numpy(inp.weights).to(dev) if weighted else None
    cap = wl.cap if layout == "copy" else wl.R   # a token has at most one row per region
    if cap is None:                              # size the regions from the routing itself
        probe = moe.MoeA2A(wl.T, wl.H, wl.k, wl.E, wl.ep, 1, device=dev)
        cap = int(moe.moe_route_counts(probe, ids).max().item())
        del probe
    h = moe.MoeA2A(wl.R, wl.H, wl.k, wl.E, wl.ep, cap, device=dev, layout=layout)
    ws = h.new_workspace()
    fp8 = payload == "fp8"
    if fp8:
        # the experts' bf16 outputs (here the dispatched rows themselves) sit in
        # ws; each step dispatches the fp8 payload into ws8 / scales
        moe.moe_dispatch(h, x, ids, wl.R, ws)
        moe.moe_reset(h)
        ws8 = h.new_workspace_fp8()
        scales = h.new_scales()
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
    fused = wl.combine == "fused"
    if fused:
        res = torch.from_numpy(inp.residual.view(np.int16)).to(dev).view(torch.bfloat16)
        gamma = torch.from_numpy(inp.gamma.view(np.int16)).to(dev).view(torch.bfloat16)
        res_out = torch.empty_like(res)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    hev = HipEvents()

    def dispatch(st=stream):
        if fp8:
            moe.moe_dispatch_fp8(h, x, ids, wl.R, ws8, scales, stream=st)
        else:
            moe.moe_dispatch(h, x, ids, wl.R, ws, stream=st)

    def combine(st=stream):
        if fused:
            moe.moe_combine_residual_rmsnorm(h, ws, w, weighted, res, gamma, wl.eps,
                                             residual_out=res_out, normed=out, stream=st)
        else:
            moe.moe_combine(h, ws, w, weighted, out=out, stream=st)

    def step(ev=None, st=stream):
        if ev is not None:
            hev.record(ev[0], sh)
        dispatch(st)
        if ev is not None:
            hev.record(ev[1], sh)
        combine(st)
        if ev is not None:
            hev.record(ev[2], sh)

    def check_status(when):
        code, bits = moe.moe_sync_status(h, stream)
        if code != moe.MOE_OK:
            raise RuntimeError(f"device status {bits} {when}: {moe.moe_strerror(code)}")

    for _ in range(warmup):
        step()
    check_status("after warmup")
    graph_ms = None
    if graph:
        # the same step captured in a HIP graph and replayed: no host launch
        # overhead between steps (the decode step is launch-bound).  A graph
        # holds GRAPH_STEPS steps, as a step sits inside a larger captured
        # forward pass in practice; a graph of one step mostly measures the
        # runtime's per-graph launch cost.
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(st=side)
        stream.wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(GRAPH_STEPS):
                step(st=torch.cuda.current_stream(dev))     # the capturing stream
        if h.handle.phase != 0:
            raise RuntimeError("capture left the handle dispatched")
        eager = out.clone()
        out.zero_()
        g.replay()
        torch.cuda.synchronize(dev)
        if not torch.equal(out.view(torch.int16), eager.view(torch.int16)):
            raise RuntimeError("graph replay does not reproduce the eager step")
        replays = max(steps // GRAPH_STEPS, 5)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for _ in range(replays):
            g.replay()
        torch.cuda.synchronize(dev)
        graph_ms = (time.perf_counter() - t0) * 1e3 / (replays * GRAPH_STEPS)
        check_status("after the graph replays")
        del g
    # timed steps (the headline figure): nothing but the path itself is enqueued
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    check_status("after timing")
    # the same number of steps again with HIP events around each launch, for
    # the per-kernel durations
    events = [[hev.create() for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for s in range(steps):
        step(events[s])
    torch.cuda.synchronize(dev)
    elapsed_ev = time.perf_counter() - t0
    check_status("after the instrumented steps")
    d_ms = [hev.elapsed_ms(e[0], e[1]) for e in events]
    c_ms = [hev.elapsed_ms(e[1], e[2]) for e in events]
    for e in events:
        for ev in e:
            hev.destroy(ev)
    # cold launches: an untimed read of a 1 GiB buffer before every dispatch
    # and every combine, so MI355X's 256 MB Infinity Cache holds none of the
    # working set.  The flush reads rather than writes: a written buffer would
    # leave dirty lines whose write-back then lands inside the timed kernel.
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev) if cold_iters > 0 else None
    cold = [[hev.create() for _ in range(4)] for _ in range(cold_iters)]
    for ev in cold:
        flush.max()
        hev.record(ev[0], sh)
        dispatch()
        hev.record(ev[1], sh)
        flush.max()
        hev.record(ev[2], sh)
        combine()
        hev.record(ev[3], sh)
    torch.cuda.synchronize(dev)
    check_status("after the cold launches")
    cd_ms = [hev.elapsed_ms(e[0], e[1]) for e in cold]
    cc_ms = [hev.elapsed_ms(e[2], e[3]) for e in cold]
    for e in cold:
        for ev in e:
            hev.destroy(ev)
    del flush
    if layout == "copy":
        b = wl.algorithmic_bytes()
    else:
        b = region_bytes(wl, int(h.counts.sum().item()))
    if fp8:   # the dispatch writes H code bytes and a 4-byte scale per row instead of 2H
        rows = int(h.counts.sum().item())
        b["dispatch"] -= rows * (wl.H - 4)
    comb_bytes = b["fused"] if fused else b["combine"]
    ms = elapsed * 1e3 / steps
    res_d = {
        "workload": describe(wl, cap) + ("" if layout == "copy" else
                                         ", per-region layout (one row per token and region)")
                    + (", fp8 e4m3 dispatch payload with a per-row scale" if fp8 else ""),
        "ms_per_step": ms,
        "ms_per_step_instrumented": elapsed_ev * 1e3 / steps,
        "tokens_per_s": wl.T / (ms / 1e3),
        "step_gbs": (b["dispatch"] + comb_bytes) / (ms / 1e3) / 1e9,
        "dispatch_ms_mean": float(np.mean(d_ms)), "dispatch_ms_p50": float(np.median(d_ms)),
        "combine_ms_mean": float(np.mean(c_ms)), "combine_ms_p50": float(np.median(c_ms)),
        "dispatch_bytes": b["dispatch"], "combine_bytes": comb_bytes,
    }
    res_d["dispatch_gbs"] = b["dispatch"] / (res_d["dispatch_ms_mean"] / 1e3) / 1e9
    res_d["combine_gbs"] = comb_bytes / (res_d["combine_ms_mean"] / 1e3) / 1e9
    res_d["step_hbm_frac"] = res_d["step_gbs"] / HBM_PEAK_GBS
    if graph_ms is not None:
        res_d["graph_ms_per_step"] = graph_ms
        res_d["graph_tokens_per_s"] = wl.T / (graph_ms / 1e3)
        res_d["graph_step_gbs"] = (b["dispatch"] + comb_bytes) / (graph_ms / 1e3) / 1e9
    res_d["cold"] = None
    if cold_iters > 0:
        res_d["cold"] = cold_stats(cd_ms, cc_ms, cold_iters, wl.T, b["dispatch"], comb_bytes)
    del ws, h
    torch.cuda.empty_cache()
    return res_d


def measure_partials(pw, steps: int, warmup: int, cold_iters: int = 100, seed: int = 0) -> dict:
    """The partials reduction fused with residual + RMSNorm (the local half of
    a tensor-parallel all-reduce and the norm after it, one kernel), and the
    plain reduction, at one shape: warm steps back to back, per-launch HIP
    events, and cold launches after a cache-evicting read."""
    import numpy as np
    import torch

    import combine_moe_dispatch_03_amd as moe
    import synth

    dev = torch.device("cuda:0")
    partials, residual, gamma = synth.make_partials(pw, seed)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    pd, rd, gd = up(partials), up(residual), up(gamma)
    ro, nd, od = torch.empty_like(rd), torch.empty_like(rd), torch.empty_like(rd)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    hev = HipEvents()

    def fused():
        moe.moe_partials_reduce_residual_rmsnorm(pd, rd, gd, pw.eps, residual_out=ro, normed=nd,
                                                 stream=stream)

    def plain():
        moe.moe_partials_reduce(pd, out=od, stream=stream)

    for _ in range(warmup):
        fused()
        plain()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(steps):
        fused()
    torch.cuda.synchronize(dev)
    ms = (time.perf_counter() - t0) * 1e3 / steps

    def timed(fn, n, flush=None):
        evs = [[hev.create() for _ in range(2)] for _ in range(n)]
        for e in evs:
            if flush is not None:
                flush.max()
            hev.record(e[0], sh)
            fn()
            hev.record(e[1], sh)
        torch.cuda.synchronize(dev)
        out = [hev.elapsed_ms(e[0], e[1]) for e in evs]
        for e in evs:
            for ev in e:
                hev.destroy(ev)
        return out

    f_ms = timed(fused, steps)
    r_ms = timed(plain, steps)
    b = pw.algorithmic_bytes()
    res = {
        "workload": f"partials: P={pw.P} tensor-parallel partials of T={pw.T} H={pw.H}, summed "
                    f"once + residual + RMSNorm (eps {pw.eps:g}) in one kernel",
        "ms_per_step": ms,
        "tokens_per_s": pw.T / (ms / 1e3),
        "step_gbs": b["fused"] / (ms / 1e3) / 1e9,
        "step_hbm_frac": b["fused"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "fused_ms_mean": float(np.mean(f_ms)), "fused_ms_p50": float(np.median(f_ms)),
        "fused_bytes": b["fused"],
        "fused_gbs": b["fused"] / (float(np.mean(f_ms)) / 1e3) / 1e9,
        "reduce_ms_mean": float(np.mean(r_ms)), "reduce_ms_p50": float(np.median(r_ms)),
        "reduce_bytes": b["reduce"],
        "reduce_gbs": b["reduce"] / (float(np.mean(r_ms)) / 1e3) / 1e9,
        "cold": None,
    }
    if cold_iters > 0:
        flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        c_ms = timed(fused, cold_iters, flush)
        del flush
        c50 = float(np.median(c_ms))
        res["cold"] = {"iters": cold_iters, "flush_bytes": 1 << 30, "fused_ms_p50": c50,
                       "fused_ms_mean": float(np.mean(c_ms)),
                       "fused_gbs_p50": b["fused"] / (c50 / 1e3) / 1e9,
                       "hbm_frac_p50": b["fused"] / (c50 / 1e3) / 1e9 / HBM_PEAK_GBS}
    del pd, rd, gd, ro, nd, od
    torch.cuda.empty_cache()
    return res


LADDER_RUNGS = (1, 16, 32, 512, 8192)


def measure_ladder(iters: int, warmup: int, rungs=LADDER_RUNGS, seed: int = 0) -> dict:
    """The pages' decode ladder protocol: one handle and one workspace sized
    once for the largest rung, each call passing its own rung (T tokens, the
    first T of one seeded batch at H = 7168, top-8 of 256 experts over 8
    regions, unweighted combine); per rung the dispatch -> combine roundtrip
    (identity expert stage) timed with HIP events, p50 and mean."""
    import numpy as np
    import torch

    import combine_moe_dispatch_03_amd as moe
    import synth

    dev = torch.device("cuda:0")
    T_max = max(rungs)
    wl = synth.Workload("ladder", T=T_max, H=7168, E=256, k=8, ep=8, cap=None, R=T_max,
                        routing="uniform", expert="identity", combine="unweighted")
    inp = synth.make_inputs(wl, seed)
    x = torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.bfloat16)
    ids = torch.from_numpy(inp.ids).to(dev)
    probe = moe.MoeA2A(T_max, wl.H, wl.k, wl.E, wl.ep, 1, device=dev)
    cap = int(moe.moe_route_counts(probe, ids).max().item())   # the largest rung fills most
    del probe
    h = moe.MoeA2A(T_max, wl.H, wl.k, wl.E, wl.ep, cap, device=dev)
    ws = h.new_workspace()
    out = torch.empty((T_max, wl.H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    hev = HipEvents()
    res = {"workload": f"ladder: T in {list(rungs)} of one batch, H=7168 E=256 top-8 ep=8, "
                       f"workspace sized once (cap={cap} rows per region), each call passing its "
                       f"rung; dispatch -> identity expert stage -> unweighted combine",
           "rungs": {}}
    for T in rungs:
        xs, ids_t, o = x[:T], ids[:T], out[:T]

        def step():
            moe.moe_dispatch(h, xs, ids_t, T, ws, stream=stream)
            moe.moe_combine(h, ws, None, False, out=o, stream=stream)

        for _ in range(warmup):
            step()
        code, bits = moe.moe_sync_status(h, stream)
        if code != moe.MOE_OK:
            raise RuntimeError(f"ladder rung {T}: device status {bits}")
        evs = [(hev.create(), hev.create()) for _ in range(iters)]
        for a, b in evs:
            hev.record(a, sh)
            step()
            hev.record(b, sh)
        torch.cuda.synchronize(dev)
        ms = [hev.elapsed_ms(a, b) for a, b in evs]
        for a, b in evs:
            hev.destroy(a)
            hev.destroy(b)
        b_ = wl.algorithmic_bytes()
        per_tok = (b_["dispatch"] + b_["combine"]) / wl.T
        p50 = float(np.median(ms))
        res["rungs"][str(T)] = {"roundtrip_us_p50": p50 * 1e3, "roundtrip_us_mean": float(np.mean(ms)) * 1e3,
                                "tokens_per_s_p50": T / (p50 / 1e3),
                                "gbs_p50": per_tok * T / (p50 / 1e3) / 1e9}
    del ws, h
    torch.cuda.empty_cache()
    return res


def summary(main_res: dict, main_name: str, extras: dict) -> dict:
    """A compact view of every workload: tokens/s and % of the HBM peak for the
    warm step, the step after a cache-evicting read (cold), and each phase."""
    def pct(v):
        return None if v is None else round(100.0 * v, 1)

    def one(r):
        if "rungs" in r:                             # the ladder
            return {t: {"roundtrip_us_p50": round(x["roundtrip_us_p50"], 2),
                        "hbm_pct": pct(x["gbs_p50"] / HBM_PEAK_GBS)} for t, x in r["rungs"].items()}
        if "fused_bytes" in r:                       # the partials reduction
            c = r.get("cold") or {}
            return {"tokens_per_s": round(r["tokens_per_s"]), "hbm_pct": pct(r["step_hbm_frac"]),
                    "cold_hbm_pct": pct(c.get("hbm_frac_p50"))}
        c = r.get("cold") or {}
        d = {"tokens_per_s": round(r["tokens_per_s"]), "ms_per_step": round(r["ms_per_step"], 4),
             "hbm_pct": pct(r["step_hbm_frac"]), "cold_hbm_pct": pct(c.get("hbm_frac_p50")),
             "dispatch_pct": pct(r["dispatch_gbs"] / HBM_PEAK_GBS),
             "combine_pct": pct(r["combine_gbs"] / HBM_PEAK_GBS)}
        if "graph_ms_per_step" in r:
            d["graph_ms_per_step"] = round(r["graph_ms_per_step"], 4)
        return d

    out = {main_name: one(main_res)}
    out.update({k: one(v) for k, v in extras.items()})
    return out


def region_bytes(wl, rows: int) -> dict:
    """Algorithmic bytes under the per-region layout with ``rows`` rows sent:
    dispatch reads x and ids, writes the rows, slot_index and src_index;
    combine reads slot_index and the rows, writes out (fused: + residual in,
    residual and normed out, gamma once)."""
    T, H, k = wl.T, wl.H, wl.k
    row = 2 * H
    return {
        "dispatch": T * (row + 8 * k) + rows * (row + 4),
        "combine": T * (row + 4 * k) + rows * row,
        "fused": T * (3 * row + 4 * k) + rows * row + row,
    }


def cold_stats(cd_ms, cc_ms, iters, T, disp_bytes, comb_bytes) -> dict:
    import numpy as np
    d50, c50 = float(np.median(cd_ms)), float(np.median(cc_ms))
    return {
        "iters": iters, "flush_bytes": 1 << 30,
        "dispatch_ms_p50": d50, "dispatch_ms_mean": float(np.mean(cd_ms)),
        "combine_ms_p50": c50, "combine_ms_mean": float(np.mean(cc_ms)),
        "dispatch_gbs_p50": disp_bytes / (d50 / 1e3) / 1e9,
        "combine_gbs_p50": comb_bytes / (c50 / 1e3) / 1e9,
        "tokens_per_s_p50": T / ((d50 + c50) / 1e3),
        "hbm_frac_p50": (disp_bytes + comb_bytes) / ((d50 + c50) / 1e3) / 1e9 / HBM_PEAK_GBS,
    }


def _cpu_ops(orc, wl, seed: int = 0):
    """One batch of ``wl`` on the CPU oracle: callables running dispatch, and
    on its result the combine (and, for the fused workload, the fused
    epilogue).  The workspace is kept across runs, so a timed run does not
    pay for first-touch page faults."""
    import numpy as np

    import synth

    inp = synth.make_inputs(wl, seed)
    weighted = wl.combine in ("weighted", "both", "fused")
    cap = wl.cap
    if cap is None:
        cap = int(orc.dispatch(np.zeros((wl.T, 1), np.uint16), inp.ids, wl.ep, wl.epr,
                               wl.T * wl.k).counts.max())
    x, ids, w = inp.x.copy(), inp.ids.copy(), inp.weights.copy()
    state = {}

    def dispatch():
        state["d"] = orc.dispatch(x, ids, wl.ep, wl.epr, cap, ws=state.get("ws"))
        state["ws"] = state["d"].ws

    def combine():
        d = state["d"]
        orc.combine(d.ws, d.slot_index, w, weighted, wl.H)

    ops = {"dispatch": dispatch, "combine": combine}
    if wl.combine == "fused":
        res, gamma = inp.residual.copy(), inp.gamma.copy()

        def fused():
            d = state["d"]
            orc.combine_residual_rmsnorm(d.ws, d.slot_index, w, True, res, gamma, wl.eps)

        ops["fused"] = fused
    return ops


def cpu_baseline_suite(names=("prefill", "skewed", "fused"), runs: int = 5,
                       threads: int = 1, seed: int = 0) -> dict:
    """The CPU oracle (its -O3 -march=native build, compiled here for this
    host) timed per workload and op: one untimed run, then the median of
    ``runs`` timed runs of each op.  With ``threads`` > 1, each thread runs
    the op on its own copy of the batch at the same time (independent batches
    in parallel: the oracle's code is unchanged and single-threaded), and a
    run's time is the wall time until every thread is done."""
    import threading

    import numpy as np

    import oracle
    import synth

    orc = oracle.load_timing(rebuild=True)
    out = {}
    for name in names:
        wl = synth.BY_NAME[name]
        workers = [_cpu_ops(orc, wl, seed) for _ in range(threads)]
        times = {op: [] for op in workers[0]}
        for op in workers[0]:
            if threads == 1:
                fn = workers[0][op]
                fn()                                       # untimed: first touch
                for _ in range(runs):
                    t0 = time.perf_counter()
                    fn()
                    times[op].append(time.perf_counter() - t0)
                continue
            start, done = threading.Barrier(threads + 1), threading.Barrier(threads + 1)

            def work(ops, op=op):
                for _ in range(runs + 1):
                    start.wait()
                    ops[op]()
                    done.wait()

            pool = [threading.Thread(target=work, args=(ops,)) for ops in workers]
            for th in pool:
                th.start()
            for r in range(runs + 1):
                start.wait()
                t0 = time.perf_counter()
                done.wait()
                if r > 0:                                  # run 0: first touch, untimed
                    times[op].append(time.perf_counter() - t0)
            for th in pool:
                th.join()
        med = {op: float(np.median(v)) for op, v in times.items()}
        second = "fused" if "fused" in med else "combine"
        step = med["dispatch"] + med[second]
        out[name] = {"tokens": wl.T, "threads": threads,
                     **{f"{op}_ms_p50": v * 1e3 for op, v in med.items()},
                     "step": f"dispatch + {second}",
                     "tokens_per_s": threads * wl.T / step}
        del workers
    return out


def cpu_baseline_lines(threads: int, runs: int = 5) -> tuple:
    """The bench line's cpu_baseline (one core, the headline workload) and
    cpu_baseline_all_cores, with the per-workload medians behind them."""
    build = "gcc " + " ".join(__import__("oracle").TIMING_CFLAGS[:2]) + " -ffp-contract=off"
    one = cpu_baseline_suite(threads=1, runs=runs)
    line = {"value": one["prefill"]["tokens_per_s"], "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"the full prefill workload (4096 tokens): dispatch + combine, each the "
                      f"median of {runs} runs after one untimed run, single-threaded scalar C "
                      f"({build})",
            "cpu_model": _cpu_model(), "host_cpus_visible": os.cpu_count(),
            "per_workload": one}
    all_cores = None
    if threads > 1:
        many = cpu_baseline_suite(names=("prefill",), threads=threads, runs=runs)
        all_cores = {"value": many["prefill"]["tokens_per_s"], "unit": "tokens/s",
                     "cores": threads, "kind": "oracle",
                     "sample": f"the full prefill workload on {threads} threads at once, each "
                               f"running its own copy of the batch; per op the median of {runs} "
                               f"runs of the wall time until every thread is done ({build})",
                     "cpu_model": _cpu_model(), "per_workload": many}
    return line, all_cores


def host_cores() -> int:
    """Cores this process may run on, at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


PROBE_KINDS = {"read": 0, "copy": 1, "write": 2, "rows": 3, "oneshot_write": 4, "oneshot_copy": 5,
               "empty": 6}


def _probe_library():
    from combine_moe_dispatch_03_amd import build as pkg_build
    if not os.path.exists(pkg_build.PROBE_LIBRARY):
        raise SystemExit(f"{pkg_build.PROBE_LIBRARY} is not built (python -m combine_moe_dispatch_03_amd.build)")
    lib = ctypes.CDLL(pkg_build.PROBE_LIBRARY)
    lib.moe_probe_stream.restype = ctypes.c_int
    lib.moe_probe_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_void_p]
    return lib


def ceilings(nbytes: int = 1 << 30, reps: int = 20) -> dict:
    """Reference bandwidths on this GPU, for comparing the path's kernels
    with what plain streaming reaches on the same device: the reference
    kernels of libmoe_stream_probe.so (grid-stride read, copy and write, plain
    and non-temporal, over a grid sweep; rows written whole by one workgroup,
    one or eight per workgroup) and torch's fill, max reduction and copy, all
    over ``nbytes``.  Mean of ``reps`` launches after 3 warm-up launches, timed
    with HIP events; GB/s counts the bytes read plus written."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(1)
    b = torch.empty_like(a)
    hev = HipEvents()
    sh = torch.cuda.current_stream(dev).cuda_stream
    lib = _probe_library()

    def probe(kind, nt, grid=0, row_bytes=0, rpb=0):
        def run():
            rc = lib.moe_probe_stream(PROBE_KINDS[kind], nt, ctypes.c_void_p(b.data_ptr()),
                                      ctypes.c_void_p(a.data_ptr()), nbytes, grid, row_bytes, rpb,
                                      ctypes.c_void_p(sh))
            if rc != 0:
                raise RuntimeError(f"moe_probe_stream({kind}) returned {rc}")
        return run

    ops = {"torch fill": (lambda: b.fill_(2), nbytes),
           "torch max": (lambda: a.max(), nbytes),
           "torch copy": (lambda: b.copy_(a), 2 * nbytes)}
    for kind, moved in (("read", nbytes), ("copy", 2 * nbytes), ("write", nbytes)):
        for nt in (0, 1):
            for grid in (1024, 2048, 4096, 8192, 16384):
                ops[f"{kind} {'nt' if nt else 'plain'} grid={grid}"] = (probe(kind, nt, grid=grid), moved)
    for kind, moved in (("oneshot_write", nbytes), ("oneshot_copy", 2 * nbytes)):
        for nt in (0, 1):
            for v in (1, 2, 4, 8):
                ops[f"{kind} {'nt' if nt else 'plain'} {v} vec/lane"] = (probe(kind, nt, rpb=v), moved)
    for row_bytes, rpb in ((16384, 1), (65536, 1), (262144, 1), (14336, 1), (14336, 8)):
        for nt in (0, 1):
            written = nbytes // (row_bytes * rpb) * row_bytes * rpb
            ops[f"rows {'nt' if nt else 'plain'} {row_bytes} B x{rpb}/workgroup"] = (
                probe("rows", nt, row_bytes=row_bytes, rpb=rpb), written)
    out = {}
    for name, (fn, moved) in ops.items():
        for _ in range(3):
            fn()
        evs = [(hev.create(), hev.create()) for _ in range(reps)]
        for e0, e1 in evs:
            hev.record(e0, sh)
            fn()
            hev.record(e1, sh)
        torch.cuda.synchronize(dev)
        ms = sum(hev.elapsed_ms(e0, e1) for e0, e1 in evs) / reps
        for e0, e1 in evs:
            hev.destroy(e0)
            hev.destroy(e1)
        gbs = moved / (ms / 1e3) / 1e9
        out[name] = {"bytes": moved, "us_mean": round(ms * 1e3, 2), "gbs": round(gbs, 1),
                     "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 1)}
        print(f"# {name:40s} {ms * 1e3:9.1f} us {gbs:8.1f} GB/s", file=sys.stderr, flush=True)
    def graph_us(kind, nt, grid, rpb, nb):
        """Microseconds per launch of a probe kernel, from a HIP graph of 100
        launches replayed 20 times (the host's issue time stays out)."""
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            gs = torch.cuda.current_stream(dev).cuda_stream
            for _ in range(100):
                rc = lib.moe_probe_stream(PROBE_KINDS[kind], nt, ctypes.c_void_p(b.data_ptr()),
                                          ctypes.c_void_p(a.data_ptr()), nb, grid, 0, rpb,
                                          ctypes.c_void_p(gs))
                if rc != 0:
                    raise RuntimeError(f"moe_probe_stream({kind}) returned {rc}")
        graph.replay()
        torch.cuda.synchronize(dev)
        e0, e1 = hev.create(), hev.create()
        hev.record(e0, sh)
        for _ in range(20):
            graph.replay()
        hev.record(e1, sh)
        torch.cuda.synchronize(dev)
        us = hev.elapsed_ms(e0, e1) * 1e3 / 2000
        hev.destroy(e0)
        hev.destroy(e1)
        del graph
        return round(us, 2)

    # the launch floor: launches of a kernel whose workgroups each store one
    # word (the decode step's two kernels run near this floor)
    floors = {}
    for grid in (128, 512, 1024):
        floors[f"{grid} workgroups"] = graph_us("empty", 0, grid, 0, nbytes)
        print(f"# launch floor, {grid} workgroups: {floors[f'{grid} workgroups']:.2f} us per launch",
              file=sys.stderr, flush=True)
    # the decode dispatch's bytes written alone: the 14.7 MB of rows of 128
    # tokens x top-8 x 7168 written by a one-store-per-lane kernel (no loads),
    # the floor under a dispatch that must first load its rows
    decode_bytes = 128 * 8 * 7168 * 2
    decode_write = {f"{v} vec/lane": graph_us("oneshot_write", 1, 0, v, decode_bytes) for v in (1, 2)}
    for name, us in decode_write.items():
        print(f"# decode-size write ({decode_bytes} B, non-temporal), {name}: {us:.2f} us per launch",
              file=sys.stderr, flush=True)
    best = {}
    for name, rec in out.items():
        family = name.split(" grid=")[0].split(" vec/lane")[0].rsplit(" ", 1)[0] \
            if name.startswith("oneshot") else name.split(" grid=")[0]
        if family not in best or rec["gbs"] > best[family]["gbs"]:
            best[family] = {"variant": name, "gbs": rec["gbs"], "pct_of_peak": rec["pct_of_peak"]}
    return {"ceilings": out, "best": best, "launch_floor_us": floors,
            "decode_size_write_us": {"bytes": decode_bytes, **decode_write}, "nbytes": nbytes, "reps": reps}


def calibrate_copy(nbytes: int, reps: int) -> None:
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": nbytes, "reps": reps}), flush=True)


def shape_workload(spec: str):
    """A workload of any shape: ``shape:T=4096,H=2048,E=128,k=8,ep=8`` with
    optional ``routing=zipf1.2`` and ``combine=weighted|unweighted|fused``.
    Every region gets as many rows as the routing sends it (cap from the
    route counts), the rung is T, and the expert stage is the identity."""
    import synth
    fields = {}
    for item in spec.split(":", 1)[1].split(","):
        key, _, value = item.partition("=")
        fields[key.strip()] = value.strip()
    unknown = set(fields) - {"T", "H", "E", "k", "ep", "routing", "combine"}
    if unknown or not {"T", "H", "E", "k", "ep"} <= set(fields):
        raise SystemExit(f"bad shape {spec!r}: give T, H, E, k, ep (and optionally routing, combine)")
    T, H, E, k, ep = (int(fields[n]) for n in ("T", "H", "E", "k", "ep"))
    return synth.Workload(name="shape", T=T, H=H, E=E, k=k, ep=ep, cap=None, R=T,
                          routing=fields.get("routing", "uniform"), expert="identity",
                          combine=fields.get("combine", "unweighted"))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill",
                    help="headline workload: tiny, decode, prefill, skewed, fused, or "
                         "shape:T=..,H=..,E=..,k=..,ep=..[,routing=..][,combine=..]; a _region / "
                         "_fp8 suffix selects a variant")
    ap.add_argument("--extras",
                    default="skewed,decode,fused,prefill_region,skewed_region,prefill_fp8,"
                            "prefill_region_fp8,partials,ladder",
                    help="comma-separated workloads also measured (empty for none); a "
                         "_region suffix runs the per-region layout, _fp8 the fp8 payload; "
                         "partials is the tensor-parallel partials reduction fused with "
                         "residual + RMSNorm; ladder the roundtrip at T = 1 ... 8192 with the "
                         "workspace sized once")
    ap.add_argument("--cold-iters", type=int, default=100,
                    help="launches timed after an untimed 1 GiB cache-evicting read, per kernel")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-runs", type=int, default=5,
                    help="timed runs per op of the CPU baseline (the median is reported)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the all-cores CPU baseline (0: every core this process "
                         "may use, at most 16; 1 skips it)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES bytes (counter calibration)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only time plain 1 GiB fill / read / copy (reference bandwidths)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs the exchange on one GPU "
              "(the destination regions are partitions of local HBM); --gpus must be 1.",
              file=sys.stderr)
        return 2
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, max(args.steps, 1))
        return 0
    if args.ceilings:
        print(json.dumps(ceilings()), flush=True)
        return 0

    import synth

    def variant(name):
        """workload name with optional _region / _fp8 suffixes"""
        base, *mods = name.split("_")
        if not base.startswith("shape:") and base not in synth.BY_NAME:
            raise SystemExit(f"unknown workload {name!r}: the headline is one of "
                             f"{sorted(synth.BY_NAME)} or shape:..., with an optional _region / "
                             f"_fp8 suffix (partials and ladder are --extras entries)")
        wl = shape_workload(base) if base.startswith("shape:") else synth.BY_NAME[base]
        return wl, dict(layout="region" if "region" in mods else "copy",
                        payload="fp8" if "fp8" in mods else "bf16")

    wl, opts = variant(args.workload)
    main_res = measure(wl, args.steps, args.warmup, args.cold_iters, **opts)
    extras = {}
    # workload names are comma-separated; a shape spec has commas of its own,
    # so split only where the next workload's name begins
    names = re.split(r",(?=(?:tiny|decode|prefill|skewed|fused|partials|ladder|shape:))",
                     args.extras)
    for name in [n for n in names if n and n != args.workload]:
        if name == "ladder":                 # launch-bound: never fewer than 100 timed steps
            extras[name] = measure_ladder(max(args.steps, SMALL_STEPS), max(args.warmup, 10))
            continue
        if name == "partials":
            extras[name] = measure_partials(synth.PARTIALS, max(args.steps // 2, 5),
                                            max(args.warmup // 2, 2), args.cold_iters)
            continue
        ewl, eopts = variant(name)
        if ewl.name in ("decode", "tiny"):   # launch-bound: never fewer than 100 timed steps
            steps, warm = max(args.steps, SMALL_STEPS), max(args.warmup, 10)
        else:
            steps, warm = max(args.steps // 2, 5), max(args.warmup // 2, 2)
        extras[name] = measure(ewl, steps, warm, args.cold_iters, graph=ewl.name == "decode",
                               **eopts)

    # the roofline describes the phase that takes longer: the dispatch call
    # (routing + copy kernels, one C call, timed as one) or the combine
    phase = "dispatch" if main_res["dispatch_ms_mean"] > main_res["combine_ms_mean"] else "combine"
    phase_ms = main_res[f"{phase}_ms_mean"]
    phase_bytes = main_res[f"{phase}_bytes"]
    achieved = phase_bytes / (phase_ms / 1e3) / 1e9
    phase_kernels = {"dispatch": dispatch_kernels(wl.T * wl.k, opts["layout"], opts["payload"]),
                     "combine": "combine_kernel"}[phase]
    line = {
        "metric": "dispatch+combine tokens/s and achieved HBM GB/s (% of peak), H=7168 top-8",
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "ms_per_step_instrumented": main_res["ms_per_step_instrumented"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded N(0,1) bf16 tokens, {wl.routing} distinct top-{wl.k} routing)",
        "config": {"workload": main_res["workload"], "tokens": wl.T, "hidden": wl.H,
                   "top_k": wl.k, "experts": wl.E, "ep_size": wl.ep,
                   "step": "dispatch -> identity expert stage -> combine"},
        "achieved_gbs": main_res["step_gbs"],
        "hbm_frac": main_res["step_hbm_frac"],
        "roofline": {"bound": "hbm", "kernel": phase_kernels, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     # the committed counters describe the prefill workload only
                     "traffic": measured_traffic(phase) if (wl.name, opts["layout"],
                                                            opts["payload"])
                     == ("prefill", "copy", "bf16") else None,
                     "algorithmic_bytes_per_launch": phase_bytes,
                     "launch_ms_mean": phase_ms},
        "kernels": {"dispatch_ms_mean": main_res["dispatch_ms_mean"],
                    "dispatch_ms_p50": main_res["dispatch_ms_p50"],
                    "dispatch_gbs": main_res["dispatch_gbs"],
                    "combine_ms_mean": main_res["combine_ms_mean"],
                    "combine_ms_p50": main_res["combine_ms_p50"],
                    "combine_gbs": main_res["combine_gbs"]},
        "cold": main_res["cold"],
        "workloads": extras,
    }
    if not args.no_cpu_baseline:
        one, many = cpu_baseline_lines(args.cpu_threads or host_cores(), args.cpu_runs)
        line["cpu_baseline"] = one
        if many is not None:
            line["cpu_baseline_all_cores"] = many
    # last, so that a reader of the line's tail sees every workload
    line["summary"] = summary(main_res, wl.name, extras)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
