"""Seeded random shapes through the HIP path, each compared with the oracle.

Forty cases drawn from a fixed seed: 0-700 tokens (both the single-launch
and the routed dispatch), hidden sizes from 8 to 1024 in steps of 8, top-1 to
top-12, 1 to 16 regions of 1 to 8 experts, both layouts, unrouted copies and
repeated experts, and now and then a capacity too small for the routing (an
overflow: reported, the copies past capacity dropped).  Dispatch must match
bit for bit and the combine (weighted for the per-copy layout, the
per-region rank-sum otherwise) within 1 bf16 ulp.
"""
import numpy as np
import pytest
import torch

import combine_moe_dispatch_03_amd as moe
import oracle
import pins
import synth
from gpu_harness import (assert_bf16_close, check_dispatch, expert_stage_gpu, expert_stage_gpu_by_row,
                         expert_stage_oracle, gpu_dispatch, say, to_dev, to_u16)

pytestmark = pytest.mark.gpu


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.integers(0, 701))
    H = 8 * int(rng.integers(1, 129))
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


@pytest.mark.parametrize("seed", range(40))
def test_random_shape_against_oracle(seed):
    c = draw_case(seed)
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
