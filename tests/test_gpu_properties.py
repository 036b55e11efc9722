"""Properties of the HIP path that hold at any size, checked without the
oracle, and a seed sweep against it.

* Payload identity: every token row carries its own index in two columns as
  exact bf16 integers (t // 256, t % 256); after dispatch each valid row is
  decoded and must name the token that src_index says it came from.
* Region membership, order-agnostic: the copies in region r are exactly
  {f : ids[f] // epr == r} as a set (numpy's own routing of the ids), and,
  for the stable slot order, src_index is strictly increasing in a region.
* slot_index and src_index are inverse maps; unrouted copies have no slot;
  padding rows keep their canary.
* Exactly once at full size: copy j's row holds 2^j in every element, so an
  unweighted combine gives 2^k - 1 exactly (255 for top-8); a copy counted
  twice or missed changes the sum.
* Seeds 1-4 on the small workloads: dispatch bit-exact and combine (and the
  fused epilogue) bit for bit against the oracle.
* The combine reads expert outputs from a buffer other than the dispatch
  workspace and leaves the workspace as dispatched.
* Two handles driven on two streams at once give the same bytes as each
  driven alone (no state outside a handle).
"""
import numpy as np
import pytest
import torch

import combine_moe_dispatch_03_amd as moe
import oracle
import synth
from gpu_harness import (CANARY, assert_bf16_close, check_dispatch, expert_stage_gpu,
                         expert_stage_oracle, gpu_dispatch, say, to_dev, to_dev_bf16, to_u16)
from oracle import compare

pytestmark = pytest.mark.gpu

SEEDS = (1, 2, 3, 4)


def labelled_inputs(wl, seed):
    inp = synth.make_inputs(wl, seed)
    t = np.arange(wl.T)
    x = inp.x.copy()
    x[:, 0] = synth.f32_to_bf16_bits((t // 256).astype(np.float32))
    x[:, 1] = synth.f32_to_bf16_bits((t % 256).astype(np.float32))
    return inp, x


def region_counts(ids, epr, ep):
    dest = np.where(ids >= 0, ids // epr, -1).reshape(-1)
    return dest, np.bincount(dest[dest >= 0], minlength=ep)


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("name", ["decode", "prefill", "skewed"])
def test_payload_identity_and_region_membership(name, seed):
    wl = synth.BY_NAME[name]
    inp, x = labelled_inputs(wl, seed)
    dest, counts = region_counts(inp.ids, wl.epr, wl.ep)
    cap = wl.cap if wl.cap is not None else int(counts.max())
    say("properties", name, "seed", seed, "cap", cap)
    assert counts.max() <= cap
    run = gpu_dispatch(x, inp.ids, wl.E, wl.ep, cap, R=wl.R)
    assert run.code == moe.MOE_OK and run.bits == 0
    h = run.h
    assert np.array_equal(h.counts.cpu().numpy(), counts)
    slot = h.slot_index_view().cpu().numpy().reshape(-1)
    src = h.src_index_view().cpu().numpy()
    labels = to_u16(run.ws[:, :, :2])                          # [ep, cap, 2]
    tok = (synth.bf16_bits_to_f32(labels[..., 0]) * 256 + synth.bf16_bits_to_f32(labels[..., 1]))
    for r in range(wl.ep):
        n = int(counts[r])
        mine = np.flatnonzero(dest == r)
        got = src[r, :n]
        assert np.array_equal(np.sort(got), mine), f"region {r}: wrong set of copies"
        assert (np.diff(got) > 0).all(), f"region {r}: slots not in flat-index order"
        assert (src[r, n:] == -1).all()
        assert np.array_equal(tok[r, :n].astype(np.int64), got // wl.k), f"region {r}: payload rows"
        if n < cap:
            assert bool((run.ws[r, n:].view(torch.int16) == CANARY).all()), f"region {r}: padding"
    routed = dest >= 0
    assert (slot[~routed] == -1).all()
    assert np.array_equal(src.reshape(-1)[slot[routed]], np.flatnonzero(routed))
    assert np.array_equal(slot[routed] // cap, dest[routed])


@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_every_copy_reduced_exactly_once_at_full_size(name):
    wl = synth.BY_NAME[name]
    inp = synth.make_inputs(wl, 0)
    _, counts = region_counts(inp.ids, wl.epr, wl.ep)
    cap = wl.cap if wl.cap is not None else int(counts.max())
    say("powers of two", name, "T", wl.T, "k", wl.k)
    run = gpu_dispatch(inp.x, inp.ids, wl.E, wl.ep, cap, R=wl.R, fill=None)
    assert run.code == moe.MOE_OK and run.bits == 0
    slot = run.h.slot_index_view().reshape(-1).long()
    j = torch.arange(slot.numel(), device="cuda") % wl.k
    valid = slot >= 0
    flat = run.ws.view(-1, wl.H)
    flat[slot[valid]] = torch.pow(2.0, j[valid].float()).to(torch.bfloat16)[:, None].expand(-1, wl.H)
    out = moe.moe_combine(run.h, run.ws, None, False)
    want = synth.f32_to_bf16_bits(np.array([2.0 ** wl.k - 1], np.float32))[0]
    got = out.view(torch.int16)
    assert bool((got == int(want.astype(np.int16))).all()), "some token did not sum to 2^k - 1"


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("name", ["tiny", "decode", "fused"])
def test_seed_sweep_against_oracle(name, seed):
    wl = synth.BY_NAME[name]
    orc = oracle.load()
    inp = synth.make_inputs(wl, seed)
    _, counts = region_counts(inp.ids, wl.epr, wl.ep)
    cap = wl.cap if wl.cap is not None else int(counts.max())
    say("seed sweep", name, "seed", seed)
    ref = orc.dispatch(inp.x, inp.ids, wl.ep, wl.epr, cap)
    assert ref.status == 0
    run = gpu_dispatch(inp.x, inp.ids, wl.E, wl.ep, cap, R=wl.R)
    assert run.code == moe.MOE_OK and run.bits == 0
    check_dispatch(run, ref, inp.x, wl.k)
    y = synth.expert_outputs(wl, inp)
    expert_stage_oracle(ref, y)
    expert_stage_gpu(run, y)
    w = to_dev(inp.weights)
    if wl.combine == "fused":
        want_r, want_n = orc.combine_residual_rmsnorm(ref.ws, ref.slot_index, inp.weights, True,
                                                      inp.residual, inp.gamma, wl.eps)
        r_out, normed = moe.moe_combine_residual_rmsnorm(
            run.h, run.ws, w, True, to_dev_bf16(inp.residual), to_dev_bf16(inp.gamma), wl.eps)
        assert_bf16_close(to_u16(r_out), want_r, "residual_out")
        assert_bf16_close(to_u16(normed), want_n, "normed")
        assert compare.rel_err(to_u16(normed), want_n) <= 1e-2
        return
    weighted_modes = {"both": [True, False], "weighted": [True], "unweighted": [False]}[wl.combine]
    for i, weighted in enumerate(weighted_modes):
        if i:                                   # a second combine needs a second dispatch
            run = gpu_dispatch(inp.x, inp.ids, wl.E, wl.ep, cap, R=wl.R)
            expert_stage_gpu(run, y)
        got = to_u16(moe.moe_combine(run.h, run.ws, w if weighted else None, weighted))
        want = orc.combine(ref.ws, ref.slot_index, inp.weights, weighted, wl.H)
        assert_bf16_close(got, want, f"{name} seed {seed} combine")


@pytest.mark.parametrize("name", ["decode", "fused"])
def test_combine_reads_a_separate_expert_output_buffer(name):
    # expert_out need not be the dispatch workspace: the experts may write
    # their outputs into a buffer of their own with the same [ep, cap, H]
    # layout.  Its padding holds NaN, so a read outside the valid rows would
    # poison the output; the dispatch workspace must be left as dispatched.
    wl = synth.BY_NAME[name]
    orc = oracle.load()
    inp = synth.make_inputs(wl, 0)
    cap = wl.cap
    say("separate expert-output buffer", name)
    ref = orc.dispatch(inp.x, inp.ids, wl.ep, wl.epr, cap)
    y = synth.expert_outputs(wl, inp)
    expert_stage_oracle(ref, y)
    run = gpu_dispatch(inp.x, inp.ids, wl.E, wl.ep, cap, R=wl.R)
    dispatched = run.ws.clone()
    ybuf = run.h.new_workspace(CANARY)
    slot = run.h.slot_index_view().reshape(-1).long()
    valid = slot >= 0
    ybuf.view(-1, wl.H)[slot[valid]] = to_dev_bf16(y)[valid]
    w = to_dev(inp.weights)
    if wl.combine == "fused":
        want_r, want_n = orc.combine_residual_rmsnorm(ref.ws, ref.slot_index, inp.weights, True,
                                                      inp.residual, inp.gamma, wl.eps)
        r_out, normed = moe.moe_combine_residual_rmsnorm(
            run.h, ybuf, w, True, to_dev_bf16(inp.residual), to_dev_bf16(inp.gamma), wl.eps)
        assert_bf16_close(to_u16(r_out), want_r, "residual_out")
        assert_bf16_close(to_u16(normed), want_n, "normed")
    else:
        got = to_u16(moe.moe_combine(run.h, ybuf, w, True))
        assert_bf16_close(got, orc.combine(ref.ws, ref.slot_index, inp.weights, True, wl.H),
                          f"{name} combine")
    assert torch.equal(run.ws.view(torch.int16), dispatched.view(torch.int16))


def test_two_handles_on_two_streams():
    # the library keeps no state outside a handle and its buffers: two
    # handles driven on two streams at once give the same bytes as each
    # driven alone
    wl = synth.BY_NAME["fused"]
    inp = synth.make_inputs(wl, 5)
    say("two handles on two streams")
    x, ids, w = to_dev_bf16(inp.x), to_dev(inp.ids), to_dev(inp.weights)
    ids2 = torch.flip(ids, dims=[0]).contiguous()

    def make():
        h = moe.MoeA2A(wl.T, wl.H, wl.k, wl.E, wl.ep, wl.cap)
        return h, h.new_workspace(0), torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")

    def run(h, ws, out, ids_, stream):
        moe.moe_dispatch(h, x, ids_, wl.R, ws, stream=stream)
        moe.moe_combine(h, ws, w, True, out=out, stream=stream)

    (h1, ws1, o1), (h2, ws2, o2) = make(), make()
    cur = torch.cuda.current_stream()
    run(h1, ws1, o1, ids, cur)
    run(h2, ws2, o2, ids2, cur)
    torch.cuda.synchronize()
    want1, want2 = o1.clone(), o2.clone()
    o1.zero_(); o2.zero_()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(cur); s2.wait_stream(cur)
    for _ in range(3):
        run(h1, ws1, o1, ids, s1)
        run(h2, ws2, o2, ids2, s2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), want1.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), want2.view(torch.int16))
    assert moe.moe_sync_status(h1)[0] == moe.MOE_OK and moe.moe_sync_status(h2)[0] == moe.MOE_OK
