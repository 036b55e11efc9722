"""Seeded random shapes through the HIP path, each compared with the oracle.

Forty cases drawn from a fixed seed: 0-700 tokens (the single-launch
dispatch, the single pass and the two kernels), hidden sizes from 8 to 1024 in steps of 8, top-1 to
top-12, 1 to 16 regions of 1 to 8 experts, both layouts, unrouted copies and
repeated experts, and now and then a capacity too small for the routing (an
overflow: reported, the copies past capacity dropped).  Dispatch must match
bit for bit and the combine (weighted for the per-copy layout, the
per-region rank-sum otherwise) bit for bit.  Twenty more cases run
the fused residual + RMSNorm epilogue and twenty the FP8 payload (codes and
scales bit-exact).  Twenty more draw 3000-9000 tokens with rows of at most
128 elements, so that random shapes also reach the single pass with the row
loaded after the routing words (32769-65536 per-copy copies) and the routing
kernel + copy kernel above 65536.
"""
import numpy as np
import pytest

import combine_moe_dispatch_03_amd as moe
import oracle
import pins
import synth
from gpu_harness import (assert_bf16_close, check_dispatch, expert_stage_gpu, expert_stage_gpu_by_row,
                         expert_stage_oracle, fp8_check, gpu_dispatch, say, to_dev, to_dev_bf16,
                         to_u16)

pytestmark = pytest.mark.gpu


def draw_case(seed, t_range=(0, 700), h_steps=128):
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.integers(t_range[0], t_range[1] + 1))
    H = 8 * int(rng.integers(1, h_steps + 1))
    k = int(rng.integers(1, 13))
    ep = int(rng.integers(1, 17))
    epr = int(rng.integers(1, 9))
    E = ep * epr
    layout = "region" if rng.random() < 0.4 else "copy"
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)          # repeats allowed
    ids[rng.random((T, k)) < rng.choice([0.0, 0.1, 0.3])] = -1
    full = T if layout == "region" else T * k
    cap = max(1, full if rng.random() < 0.8 else int(full * rng.uniform(0.05, 0.5)) // max(ep, 1))
    x = pins.random_bf16(rng, (T, H))
    w = rng.random((T, k)).astype(np.float32)
    y = pins.random_bf16(rng, (T * k, H))
    return dict(T=T, H=H, k=k, E=E, ep=ep, epr=epr, layout=layout, cap=cap, ids=ids, x=x, w=w, y=y)


def dispatch_and_combine(c, seed):
    T, H, k, E, ep, epr, cap = c["T"], c["H"], c["k"], c["E"], c["ep"], c["epr"], c["cap"]
    say("random case", seed, {n: c[n] for n in ("T", "H", "k", "E", "ep", "layout", "cap")})
    orc = oracle.load()
    ref = orc.dispatch(c["x"], c["ids"], ep, epr, cap, layout=c["layout"])
    run = gpu_dispatch(c["x"], c["ids"], E, ep, cap, R=max(T, 1), max_tokens=max(T, 1),
                       layout=c["layout"])
    assert run.bits == ref.status, (run.bits, ref.status)
    check_dispatch(run, ref, c["x"], k)
    if c["layout"] == "copy":
        expert_stage_oracle(ref, c["y"])
        expert_stage_gpu(run, c["y"])
        got = moe.moe_combine(run.h, run.ws, to_dev(c["w"]), True)
        want = orc.combine(ref.ws, ref.slot_index, c["w"], True, H)
    else:
        msgs = synth.region_messages(c["ids"], c["w"], c["y"], epr)
        oracle.place_expert_outputs(ref.ws, ref.slot_index, msgs)
        expert_stage_gpu_by_row(run, msgs)
        got = moe.moe_combine(run.h, run.ws, None, False)
        want = orc.combine(ref.ws, ref.slot_index, None, False, H, layout="region")
    assert_bf16_close(to_u16(got), want, f"random case {seed} combine")
    assert run.h.handle.phase == 0


@pytest.mark.parametrize("seed", range(40))
def test_random_shape_against_oracle(seed):
    dispatch_and_combine(draw_case(seed), seed)


@pytest.mark.parametrize("seed", range(80, 100))
def test_random_large_batch_against_oracle(seed):
    dispatch_and_combine(draw_case(seed, t_range=(3000, 9000), h_steps=16), seed)


@pytest.mark.parametrize("seed", range(40, 60))
def test_random_shape_fused_epilogue(seed):
    c = draw_case(seed)
    T, H, k, E, ep, epr, cap = c["T"], c["H"], c["k"], c["E"], c["ep"], c["epr"], c["cap"]
    say("random fused case", seed, {n: c[n] for n in ("T", "H", "k", "E", "ep", "cap")})
    rng = np.random.default_rng(seed)
    res = pins.random_bf16(rng, (T, H))
    gamma = pins.torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    orc = oracle.load()
    ref = orc.dispatch(c["x"], c["ids"], ep, epr, cap)
    run = gpu_dispatch(c["x"], c["ids"], E, ep, cap, R=max(T, 1), max_tokens=max(T, 1))
    assert run.bits == ref.status
    expert_stage_oracle(ref, c["y"])
    expert_stage_gpu(run, c["y"])
    r_out, normed = moe.moe_combine_residual_rmsnorm(run.h, run.ws, to_dev(c["w"]), True,
                                                     to_dev_bf16(res), to_dev_bf16(gamma), 1e-6)
    want_r, want_n = orc.combine_residual_rmsnorm(ref.ws, ref.slot_index, c["w"], True, res,
                                                  gamma, 1e-6)
    assert_bf16_close(to_u16(r_out), want_r, "residual_out")
    assert_bf16_close(to_u16(normed), want_n, "normed")


@pytest.mark.parametrize("seed", range(60, 80))
def test_random_shape_fp8_dispatch(seed):
    c = draw_case(seed)
    say("random fp8 case", seed, {n: c[n] for n in ("T", "H", "k", "E", "ep", "layout", "cap")})
    fp8_check(c["x"], c["ids"], c["E"], c["ep"], c["cap"], R=max(c["T"], 1), layout=c["layout"])


@pytest.mark.parametrize("seed", range(100, 110))
def test_random_large_fp8_dispatch(seed):
    # 3,000-9,000 tokens: the fp8 single pass, or the two kernels, by size and layout
    c = draw_case(seed, t_range=(3000, 9000), h_steps=16)
    say("random large fp8 case", seed, {n: c[n] for n in ("T", "H", "k", "E", "ep", "layout", "cap")})
    fp8_check(c["x"], c["ids"], c["E"], c["ep"], c["cap"], R=max(c["T"], 1), layout=c["layout"])
