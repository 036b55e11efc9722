"""Parity of the per-region (rank-dedup) layout with the oracle on the GPU.

One workspace row per (token, destination region); the region's experts
return one message per token (synth.region_messages: the gated fp32 sum of
the token's local copies, narrowed once); the combine adds each region's
message once.  Dispatch, combine and fused epilogue bit for bit against the
oracle, at the full prefill / skewed / decode / fused shapes and on edge cases,
plus the pages' dedup probes through the GPU path.
"""
import numpy as np
import pytest
import torch

import combine_moe_dispatch_03_amd as moe
import oracle
import pins
import synth
from gpu_harness import (CANARY, assert_bf16_close, check_dispatch, expert_stage_gpu_by_row,
                         gpu_dispatch, say, to_dev_bf16, to_u16)
from oracle import compare

pytestmark = pytest.mark.gpu


def region_roundtrip(x, ids, w, y, E, ep, cap, R=None, fused=None, eps=1e-6):
    """Dispatch, per-region expert stage and combine (or fused) on both sides."""
    orc = oracle.load()
    T, H = x.shape
    k = ids.shape[1]
    ref = orc.dispatch(x, ids, ep, E // ep, cap, layout="region")
    run = gpu_dispatch(x, ids, E, ep, cap, R=R, layout="region")
    assert run.bits == ref.status, (run.bits, ref.status)
    check_dispatch(run, ref, x, k)
    msgs = synth.region_messages(ids, w, y, E // ep)
    oracle.place_expert_outputs(ref.ws, ref.slot_index, msgs)
    expert_stage_gpu_by_row(run, msgs)
    if fused is None:
        out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.moe_combine(run.h, run.ws, None, False, out=out)
        want = orc.combine(ref.ws, ref.slot_index, None, False, H, layout="region")
        n = assert_bf16_close(to_u16(out), want, "region combine")
    else:
        res, gamma = fused
        r_out, normed = moe.moe_combine_residual_rmsnorm(run.h, run.ws, None, False,
                                                         to_dev_bf16(res), to_dev_bf16(gamma), eps)
        want_r, want_n = orc.combine_residual_rmsnorm(ref.ws, ref.slot_index, None, False, res,
                                                      gamma, eps, layout="region")
        assert_bf16_close(to_u16(r_out), want_r, "region residual_out")
        n = assert_bf16_close(to_u16(normed), want_n, "region normed")
        assert compare.rel_err(to_u16(normed), want_n) <= 1e-2
    assert run.h.handle.phase == 0
    return ref, n


@pytest.mark.parametrize("name", ["prefill", "skewed", "decode", "fused"])
def test_region_layout_full_size(name):
    wl = synth.BY_NAME[name]
    say("region layout", name)
    inp = synth.make_inputs(wl, 0)
    y = synth.expert_outputs(wl, inp)
    fused = (inp.residual, inp.gamma) if wl.combine == "fused" else None
    ref, n = region_roundtrip(inp.x, inp.ids, inp.weights, y, wl.E, wl.ep, cap=wl.T, R=wl.R,
                              fused=fused)
    per_token = ref.counts.sum() / wl.T
    say(f"{name}: {per_token:.3f} rows per token, {n} elements differ from the oracle")
    if wl.routing == "uniform":
        assert abs(per_token - 5.2947) < 0.05


REGION_EDGE_CASES = [
    # (name, T, H, k, E, ep, p_missing)
    ("duplicates_and_gaps", 61, 136, 6, 12, 4, 0.15),
    ("one_region", 17, 64, 4, 8, 1, 0.0),
    ("top1", 33, 256, 1, 16, 8, 0.1),
    ("wide_rows", 5, 16384, 8, 32, 4, 0.1),
    ("two_kernel_path", 1200, 64, 8, 64, 8, 0.05),
    ("whole_token_blocks_last_size", 1024, 4096, 8, 64, 8, 0.05),   # 8192 copies
    ("pair_blocks_first_size", 1025, 4096, 8, 64, 8, 0.05),         # 8200 copies
    ("max_topk", 24, 64, 64, 512, 256, 0.0),
    ("tile_groups_wave_form", 9000, 16, 8, 64, 8, 0.05),     # k divides 64: ballot test
    ("tile_groups_k6", 12000, 16, 6, 36, 6, 0.05),           # k = 6: ids re-read
    # rows of 8 KB and more, above 8192 copies: two copies per copy-kernel block
    ("pairs_region_sums_16", 1100, 4096, 8, 64, 16, 0.05),   # regions = 2 x copies
    ("pairs_region_sums", 1200, 4104, 7, 28, 4, 0.1),        # fewer regions, ragged row
    ("pairs_copy_sums_32_regions", 1100, 4096, 8, 64, 32, 0.05),  # regions > 2 x copies
    ("copy_sums_small_rows", 1200, 64, 4, 128, 64, 0.05),    # whole-token blocks, per-copy sums
]


@pytest.mark.parametrize("case", REGION_EDGE_CASES, ids=[c[0] for c in REGION_EDGE_CASES])
def test_region_layout_edges(case):
    name, T, H, k, E, ep, pm = case
    say("region edge", name)
    rng = np.random.default_rng(T * 7 + k)
    x = pins.random_bf16(rng, (T, H))
    ids = np.stack([rng.integers(0, E, size=k) for _ in range(T)]).astype(np.int32)  # repeats allowed
    ids[rng.random(ids.shape) < pm] = -1
    w = rng.random((T, k)).astype(np.float32)
    y = pins.random_bf16(rng, (T * k, H))
    region_roundtrip(x, ids, w, y, E, ep, cap=T)
    res = pins.random_bf16(rng, (T, H))
    gamma = pins.torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    if H <= moe.MOE_MAX_FUSED_HIDDEN:
        region_roundtrip(x, ids, w, y, E, ep, cap=T, fused=(res, gamma))


def test_region_bad_ids_and_overflow():
    say("region bad ids / overflow")
    orc = oracle.load()
    rng = np.random.default_rng(5)
    T, H, k, E, ep = 40, 64, 4, 8, 2
    x = pins.random_bf16(rng, (T, H))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[3, 2], ids[7, 0] = E + 3, -9
    for cap in (T, 25):
        ref = orc.dispatch(x, ids, ep, E // ep, cap, layout="region")
        run = gpu_dispatch(x, ids, E, ep, cap, layout="region")
        assert run.bits == ref.status and ref.status & oracle.STATUS_BAD_ID
        assert bool(ref.status & oracle.STATUS_OVERFLOW) == (cap == 25)
        check_dispatch(run, ref, x, k)


def test_region_weighted_combine_is_rejected():
    rng = np.random.default_rng(1)
    x = pins.random_bf16(rng, (4, 64))
    run = gpu_dispatch(x, np.array([[0, 1]] * 4, np.int32), 4, 2, 4, layout="region")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_combine(run.h, run.ws, torch.ones(4, 2, device="cuda"), True)
    assert e.value.code == moe.MOE_ERR_ARG and run.h.handle.phase == 1


@pytest.mark.parametrize("probe", ["duplicates_read_once", "power_of_two", "staged_sum"])
def test_region_page_probes_on_gpu(probe):
    say("region page probe", probe)
    if probe == "duplicates_read_once":
        ids, msgs, want = [[0, 0]], [1.0], 1.0
    elif probe == "power_of_two":
        g = pins.read_golden("power_of_two_probe.txt")
        ids, msgs = [[3, 0, 1, 2, 4, 5, 7, 6, 0, 3]], [float(v) for v in g["contributions"][0]]
        want = float(g["expected"][0][0])
    else:
        g = pins.read_golden("staged_sum.txt")
        msgs = [0.0] * 8
        for r, v in g["contribution"]:
            msgs[int(r)] = float(v)
        ids, want = [[0, 1, 2, 4, 5, 6, 7, 0]], float(g["expected"][0][0])
    ids = np.array(ids, np.int32)
    ep, H = len(msgs), 64
    run = gpu_dispatch(np.zeros((1, H), np.uint16), ids, ep, ep, 1, layout="region")
    counts = run.h.counts.cpu().numpy()
    flat = run.ws.view(-1, H)
    for r in range(ep):
        if counts[r]:
            flat[r] = to_dev_bf16(np.full(H, pins.printed_bits(msgs[r]), np.uint16))
    out = to_u16(moe.moe_combine(run.h, run.ws, None, False))
    assert (out == pins.exact_bits(want)).all(), hex(out[0, 0])
    for r in range(ep):
        if not counts[r]:
            assert bool((run.ws[r].view(torch.int16) == CANARY).all())
