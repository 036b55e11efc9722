"""Parity of the HIP path with the CPU oracle on the five workloads.

Dispatch (counts, slot_index, src_index, every valid row) must match
bit-exactly; padding rows keep their NaN canary (never written) and, because
a read canary would poison the sum, the combine result also shows padding is
never read.  Combine and the fused epilogue must equal the oracle bit for bit
everywhere (the kernels take the oracle's fp32 operations in its order and
round once; the normalised output rounds its fp64 value through fp32 with
round-to-odd, so it too is rounded once), and the normalised output is also
checked against 1e-2 relative error
(0.02 magnitude floor).  All five workloads run at their full sizes, in the
same launch configuration the benchmark times.
"""
import functools

import numpy as np
import pytest
import torch

import combine_moe_dispatch_03_amd as moe
import oracle
import synth
from gpu_harness import (assert_bf16_close, check_dispatch, expert_stage_gpu, expert_stage_oracle,
                         gpu_dispatch, oracle_counts, say, to_dev, to_dev_bf16, to_u16)
from oracle import compare

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def prepared(name: str, staged: bool = False, seed: int = 0):
    """Inputs, capacity, oracle dispatch and per-copy expert outputs.

    With ``staged`` the oracle's workspace rows already hold the expert
    outputs (the input of the combine); otherwise they hold the dispatched
    token rows."""
    wl = synth.BY_NAME[name]
    orc = oracle.load()
    inp = synth.make_inputs(wl, seed)
    cap = wl.cap if wl.cap is not None else int(oracle_counts(orc, inp.ids, wl.ep, wl.epr).max())
    ref = orc.dispatch(inp.x, inp.ids, wl.ep, wl.epr, cap)
    y = synth.expert_outputs(wl, inp)
    if staged:
        expert_stage_oracle(ref, y)
    return wl, inp, cap, ref, y


@pytest.mark.parametrize("name", [w.name for w in synth.ALL])
def test_dispatch_bit_exact(name):
    wl, inp, cap, ref, _ = prepared(name)
    say("dispatch", name, "T", wl.T, "H", wl.H, "k", wl.k, "ep", wl.ep, "cap", cap)
    assert ref.status == 0
    run = gpu_dispatch(inp.x, inp.ids, wl.E, wl.ep, cap, R=wl.R)
    assert run.code == moe.MOE_OK and run.bits == 0
    check_dispatch(run, ref, inp.x, wl.k)


def combine_modes(wl):
    return {"both": [True, False], "weighted": [True], "unweighted": [False],
            "fused": [True]}[wl.combine]


@pytest.mark.parametrize("name", [w.name for w in synth.ALL])
def test_combine_within_one_ulp(name):
    wl, inp, cap, ref, y = prepared(name, staged=True)
    orc = oracle.load()
    for weighted in combine_modes(wl):
        say("combine", name, "weighted" if weighted else "unweighted")
        run = gpu_dispatch(inp.x, inp.ids, wl.E, wl.ep, cap, R=wl.R)
        expert_stage_gpu(run, y)
        w = to_dev(inp.weights)
        out = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.moe_combine(run.h, run.ws, w if weighted else None, weighted, out=out)
        got = to_u16(out)
        want = orc.combine(ref.ws, ref.slot_index, inp.weights, weighted, wl.H)
        inexact = assert_bf16_close(got, want, f"{name} combine")
        say(f"{name}: {inexact} of {got.size} elements differ from the oracle")
        assert run.h.handle.phase == 0


def test_fused_epilogue_within_one_ulp():
    wl, inp, cap, ref, y = prepared("fused", staged=True)
    orc = oracle.load()
    want_r, want_n = orc.combine_residual_rmsnorm(ref.ws, ref.slot_index, inp.weights, True,
                                                  inp.residual, inp.gamma, wl.eps)
    for in_place in (False, True):
        say("fused epilogue, residual updated in place" if in_place else "fused epilogue")
        run = gpu_dispatch(inp.x, inp.ids, wl.E, wl.ep, cap, R=wl.R)
        expert_stage_gpu(run, y)
        res = to_dev_bf16(inp.residual)
        res_out = res if in_place else torch.empty_like(res)
        r_out, normed = moe.moe_combine_residual_rmsnorm(
            run.h, run.ws, to_dev(inp.weights), True, res, to_dev_bf16(inp.gamma), wl.eps,
            residual_out=res_out)
        got_r, got_n = to_u16(r_out), to_u16(normed)
        assert_bf16_close(got_r, want_r, "residual_out")
        inexact = assert_bf16_close(got_n, want_n, "normed")
        assert compare.rel_err(got_n, want_n) <= 1e-2
        say(f"fused: {inexact} normed elements differ from the oracle, "
            f"rel err {compare.rel_err(got_n, want_n):.2e}")


def test_prefill_reduces_exactly_once():
    # the prefill expert stage applies the gates itself; an unweighted
    # rank-sum must then count every copy once (multiplicity 1), never twice
    wl, inp, cap, ref, y = prepared("prefill", staged=True)
    orc = oracle.load()
    once = orc.combine(ref.ws, ref.slot_index, None, False, wl.H)
    run = gpu_dispatch(inp.x, inp.ids, wl.E, wl.ep, cap, R=wl.R)
    expert_stage_gpu(run, y)
    got = to_u16(moe.moe_combine(run.h, run.ws, None, False))
    alpha = compare.reduce_multiplicity(got, once)
    assert np.abs(alpha - 1).max() < 1e-2
    assert not compare.reduced_more_than_once(got, once)
    assert moe.moe_output_is_reduced()


def test_route_counts_sizes_the_skewed_workspace():
    wl, inp, cap, ref, _ = prepared("skewed")
    say("route counts, skewed")
    h = moe.MoeA2A(wl.T, wl.H, wl.k, wl.E, wl.ep, 1)
    counts = moe.moe_route_counts(h, to_dev(inp.ids)).cpu().numpy()
    assert np.array_equal(counts, ref.counts)
    assert int(counts.max()) == cap
    assert h.handle.phase == 0


def test_determinism_from_first_invocation():
    wl, inp, cap, ref, y = prepared("decode")
    outs = []
    for rep in range(3):
        say("decode determinism run", rep)
        run = gpu_dispatch(inp.x, inp.ids, wl.E, wl.ep, cap, R=wl.R)
        slots = run.h.slot_index_view().cpu().numpy()
        expert_stage_gpu(run, y)
        out = to_u16(moe.moe_combine(run.h, run.ws, to_dev(inp.weights), True))
        outs.append((slots, out, to_u16(run.ws.view(-1, wl.H)[: 64])))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
