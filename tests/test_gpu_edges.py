"""Edge cases of the HIP path against the oracle: empty and ragged inputs,
degenerate layouts, the limits, error reporting, phase misuse, bf16 rounding
corners, and the pages' worked probes run through the GPU path."""
import zlib

import numpy as np
import pytest
import torch

import combine_moe_dispatch_03_amd as moe
import oracle
import pins
from gpu_harness import (CANARY, assert_bf16_close, check_dispatch, expert_stage_gpu,
                         expert_stage_oracle, gpu_dispatch, say, to_dev, to_dev_bf16, to_u16)

pytestmark = pytest.mark.gpu


def random_case(seed, T, H, k, E, ep, p_missing=0.0, duplicates=False):
    rng = np.random.default_rng(seed)
    x = pins.random_bf16(rng, (T, H))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32).reshape(T, k)
    if duplicates and k > 1:
        ids[::3, 1] = ids[::3, 0]
    if p_missing:
        ids[rng.random(ids.shape) < p_missing] = -1
    w = rng.random((T, k)).astype(np.float32)
    y = pins.random_bf16(rng, (T * k, H))
    return x, ids, w, y


def roundtrip(x, ids, w, y, E, ep, cap, R=None, fused=False, eps=1e-6, seed=0):
    """Dispatch, expert stage and combine on both sides; everything compared."""
    orc = oracle.load()
    T, H = x.shape
    k = ids.shape[1]
    ref = orc.dispatch(x, ids, ep, E // ep, cap)
    run = gpu_dispatch(x, ids, E, ep, cap, R=R)
    assert run.bits == ref.status, (run.bits, ref.status)
    check_dispatch(run, ref, x, k)
    expert_stage_oracle(ref, y)
    expert_stage_gpu(run, y)
    h = run.h
    for weighted in (False, True):
        if weighted:   # combine consumed the dispatch; dispatch again for the second mode
            run = gpu_dispatch(x, ids, E, ep, cap, R=R)
            expert_stage_gpu(run, y)
            h = run.h
        if not fused:
            out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
            moe.moe_combine(h, run.ws, to_dev(w) if weighted else None, weighted, out=out)
            want = orc.combine(ref.ws, ref.slot_index, w, weighted, H)
            assert_bf16_close(to_u16(out), want, f"combine weighted={weighted}")
        else:
            rng = np.random.default_rng(seed + 1)
            res = pins.random_bf16(rng, (T, H))
            gamma = pins.torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
            r_out, normed = moe.moe_combine_residual_rmsnorm(
                h, run.ws, to_dev(w) if weighted else None, weighted, to_dev_bf16(res),
                to_dev_bf16(gamma), eps)
            want_r, want_n = orc.combine_residual_rmsnorm(ref.ws, ref.slot_index, w, weighted,
                                                          res, gamma, eps)
            assert_bf16_close(to_u16(r_out), want_r, "residual_out")
            assert_bf16_close(to_u16(normed), want_n, "normed")
        assert h.handle.phase == 0
    return run


ROUNDTRIP_CASES = [
    # (name, T, H, k, E, ep)
    ("ragged_rows_and_vectors", 37, 136, 3, 12, 4),
    ("one_vector_rows", 5, 8, 2, 4, 2),
    ("one_region", 19, 64, 4, 8, 1),
    ("top1", 33, 256, 1, 16, 8),
    ("single_token_decode_row", 1, 7168, 8, 256, 8),
    ("few_tokens_wide_rows", 3, 16384, 8, 64, 8),
    ("max_hidden", 3, 1 << 20, 2, 4, 2),               # MOE_MAX_HIDDEN: 2 MiB rows, 512 column blocks
    ("odd_hidden", 7, 9000, 5, 40, 5),
    ("max_regions_max_topk", 24, 64, 64, 512, 256),
    ("many_chunks_ragged", 4099, 24, 6, 36, 6),
    ("single_launch_short_ids", 256, 128, 8, 64, 8), # 2048 copies: one launch, 8 ids per lane
    ("single_launch_long_ids", 257, 128, 8, 64, 8),  # 2056 copies: one launch, 16 ids per lane
    ("single_launch_limit", 512, 128, 8, 64, 8),     # 4096 copies: the last one-launch size
    ("first_multi_block_size", 513, 128, 8, 64, 8),  # 4104 copies: the single pass
    ("single_launch_long_wide_rows", 300, 7168, 8, 256, 8),  # 2400 copies, whole-token blocks
    ("single_launch_short_wide_rows", 256, 7168, 8, 256, 8), # 2048 copies, blocks of 2 copies
    # the routing kernel loads its chunk's ids 4 tiles of 256 at a time:
    ("full_and_partial_tile_group", 9000, 16, 8, 64, 8),   # 1128 copies per chunk: 4 + 1 tiles
    ("five_tile_groups", 40000, 8, 8, 64, 8),              # 5000 copies per chunk: 20 tiles
    ("copy_sums_small_rows", 3000, 64, 3, 48, 16),         # more regions than copies
]


@pytest.mark.parametrize("case", ROUNDTRIP_CASES, ids=[c[0] for c in ROUNDTRIP_CASES])
def test_roundtrip_shapes(case):
    name, T, H, k, E, ep = case
    say("roundtrip", name, T, H, k, E, ep)
    x, ids, w, y = random_case(zlib.crc32(name.encode()), T, H, k, E, ep, p_missing=0.1,
                              duplicates=True)
    roundtrip(x, ids, w, y, E, ep, cap=T * k)


# Rows of at least 8 KB go to the copy kernel two copies per block (a token's
# blocks share an XCD): ragged top-k (a last block with one copy), ragged
# rows, more regions than copies (per-copy prefix sums) and fewer (per-region
# sums), and rows over two column blocks.  cap is sized from the routing.
SPLIT_CASES = [
    # (name, T, H, k, E, ep)
    ("pairs_region_sums_ragged", 389, 4104, 7, 40, 4),
    ("pairs_copy_sums", 301, 4096, 7, 64, 16),
    ("pairs_top64_many_regions", 40, 4096, 64, 512, 256),
    ("pairs_two_column_blocks", 300, 32768, 7, 56, 8),
    ("pairs_top1", 2100, 4096, 1, 8, 4),                   # one copy: a single half-full block
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_copy_pairs_shapes(case):
    name, T, H, k, E, ep = case
    say("copy pairs", name, T, H, k, E, ep)
    x, ids, w, y = random_case(zlib.crc32(name.encode()), T, H, k, E, ep, p_missing=0.1,
                              duplicates=True)
    dest = np.where(ids >= 0, ids // (E // ep), -1).reshape(-1)
    cap = int(np.bincount(dest[dest >= 0], minlength=ep).max()) + 3
    roundtrip(x, ids, w, y, E, ep, cap=cap)


def test_copy_split_over_two_launches():
    # The copy kernel's launches hold at most 2^22 blocks along x; small rows
    # run one block per token, so 2^22 + 13 tokens at top-1 take two launches
    # (the second starts at token 2^22, mid-chunk, with a padded tail).
    T, H, k, E, ep = (1 << 22) + 13, 8, 1, 4, 2
    say("two copy launches", T, H, k, E, ep)
    rng = np.random.default_rng(22)
    x = pins.random_bf16(rng, (T, H))
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[rng.random(ids.shape) < 0.05] = -1
    w = rng.random((T, k)).astype(np.float32)
    y = pins.random_bf16(rng, (T * k, H))
    roundtrip(x, ids, w, y, E, ep, cap=T // 2 + 32768)


@pytest.mark.parametrize("H", [136, 7168, 9000, 16384])
def test_fused_shapes(H):
    say("fused roundtrip H", H)
    x, ids, w, y = random_case(H, 9, H, 4, 16, 4, p_missing=0.1)
    roundtrip(x, ids, w, y, 16, 4, cap=36, fused=True)


def test_empty_batch():
    say("empty batch")
    x = np.zeros((0, 64), np.uint16)
    ids = np.zeros((0, 4), np.int32)
    run = gpu_dispatch(x, ids, 8, 2, 16, R=8, max_tokens=8)
    assert run.code == moe.MOE_OK
    assert (run.h.counts.cpu().numpy() == 0).all()
    assert bool((run.ws.view(torch.int16) == CANARY).all())
    out = moe.moe_combine(run.h, run.ws, None, False)
    assert out.shape == (0, 64) and run.h.handle.phase == 0


def test_all_copies_unrouted_give_positive_zero():
    say("all ids -1")
    T, H, k = 6, 64, 3
    x = pins.random_bf16(np.random.default_rng(1), (T, H))
    ids = np.full((T, k), -1, np.int32)
    run = gpu_dispatch(x, ids, 6, 3, 4)
    assert run.code == moe.MOE_OK and (run.h.counts.cpu().numpy() == 0).all()
    out = moe.moe_combine(run.h, run.ws, to_dev(np.ones((T, k), np.float32)), True)
    assert (to_u16(out) == 0).all()
    assert bool((run.ws.view(torch.int16) == CANARY).all())


def test_runtime_rung_above_token_count_and_handle_reuse():
    say("rung > T, reused handle")
    orc = oracle.load()
    E, ep, H, k = 16, 4, 128, 4
    h = moe.MoeA2A(64, H, k, E, ep, 256)
    ws = h.new_workspace(CANARY)
    for T, R in [(50, 64), (20, 32), (64, 64), (1, 1)]:
        x, ids, w, y = random_case(T, T, H, k, E, ep)
        ws.view(torch.int16).fill_(CANARY)
        moe.moe_dispatch(h, to_dev_bf16(x), to_dev(ids), R, ws)
        assert moe.moe_sync_status(h) == (moe.MOE_OK, 0)
        ref = orc.dispatch(x, ids, ep, E // ep, 256)
        assert np.array_equal(h.counts.cpu().numpy(), ref.counts)
        assert np.array_equal(h.slot_index_view().cpu().numpy(), ref.slot_index)
        out = to_u16(moe.moe_combine(h, ws, to_dev(w), True))
        assert_bf16_close(out, orc.combine(ref.ws, ref.slot_index, w, True, H), f"T={T}")


def test_bad_expert_ids_are_reported_and_skipped():
    say("bad ids")
    orc = oracle.load()
    T, H, k, E, ep = 16, 64, 4, 8, 4
    x, ids, w, y = random_case(3, T, H, k, E, ep)
    ids[2, 1], ids[5, 3], ids[9, 0] = E, -7, 1 << 30
    ref = orc.dispatch(x, ids, ep, E // ep, T * k)
    assert ref.status == oracle.STATUS_BAD_ID
    run = gpu_dispatch(x, ids, E, ep, T * k)
    assert run.code == moe.MOE_ERR_EXPERT_ID and run.bits == moe.MOE_STATUS_EXPERT_ID
    check_dispatch(run, ref, x, k)
    assert moe.moe_sync_status(run.h) == (moe.MOE_OK, 0)     # cleared after reading
    out = to_u16(moe.moe_combine(run.h, run.ws, to_dev(w), True))
    assert_bf16_close(out, orc.combine(ref.ws, ref.slot_index, w, True, H), "combine")


def test_overflow_is_reported_and_never_written_past_cap():
    say("overflow")
    orc = oracle.load()
    T, H, k, E, ep = 64, 64, 4, 8, 2
    x, ids, w, y = random_case(4, T, H, k, E, ep)
    cap = 100                                   # each region is sent about 128 copies
    ref = orc.dispatch(x, ids, ep, E // ep, cap)
    assert ref.status == oracle.STATUS_OVERFLOW
    run = gpu_dispatch(x, ids, E, ep, cap)
    assert run.code == moe.MOE_ERR_OVERFLOW and run.bits & moe.MOE_STATUS_OVERFLOW
    check_dispatch(run, ref, x, k)
    out = to_u16(moe.moe_combine(run.h, run.ws, to_dev(w), True))
    assert_bf16_close(out, orc.combine(ref.ws, ref.slot_index, w, True, H), "combine")


def test_phase_errors_on_device_handles():
    say("phase errors")
    x, ids, w, y = random_case(5, 8, 64, 2, 4, 2)
    run = gpu_dispatch(x, ids, 4, 2, 16)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_dispatch(run.h, run.x, run.ids, 8, run.ws)
    assert e.value.code == moe.MOE_ERR_PHASE
    moe.moe_combine(run.h, run.ws, None, False)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_combine(run.h, run.ws, None, False)
    assert e.value.code == moe.MOE_ERR_PHASE
    moe.moe_dispatch(run.h, run.x, run.ids, 8, run.ws)
    moe.moe_reset(run.h)
    with pytest.raises(moe.MoeError):
        moe.moe_combine(run.h, run.ws, None, False)


def test_combine_overwrites_and_repeats_bit_identically():
    say("combine overwrite")
    x, ids, w, y = random_case(6, 40, 256, 4, 16, 4)
    outs = []
    for fill in (float("nan"), 3.0):
        run = gpu_dispatch(x, ids, 16, 4, 160)
        expert_stage_gpu(run, y)
        out = torch.full((40, 256), fill, dtype=torch.bfloat16, device="cuda")
        moe.moe_combine(run.h, run.ws, to_dev(w), True, out=out)
        outs.append(to_u16(out))
    assert np.array_equal(outs[0], outs[1])


def test_rounding_corners_through_the_combine():
    # one token per case, every column the same; sums chosen to land on
    # nearest-even ties, subnormals and the overflow threshold
    say("rounding corners")
    orc = oracle.load()
    cases = [  # (copy values, gates or None)
        ([1.0, 2.0 ** -8], None),                  # tie -> 1.0
        ([1.0, 3 * 2.0 ** -8], None),              # tie -> 1 + 2^-6
        ([-1.0, -(2.0 ** -8)], None),
        ([2.0 ** -133], [0.75]),                   # fp32 subnormal product -> smallest bf16
        ([2.0 ** -133], [0.5]),                    # tie with zero -> +0
        ([2.0 ** -126, -(2.0 ** -127)], None),     # subnormal result, exact
        ([(2 - 2 ** -7) * 2.0 ** 127], [1.00390625]),   # rounds past the largest bf16 -> inf
        ([(2 - 2 ** -7) * 2.0 ** 127] * 2, None),  # fp32 overflow -> inf
        ([-0.0], None),                            # +0 accumulator start
        ([1.0] + [2.0 ** -9] * 7, None),           # the pages' discriminating probe
    ]
    for vals, gates in cases:
        k = len(vals)
        ws, slot = pins.one_token_case(vals, H=64)
        w = np.array([gates if gates else [1.0] * k], np.float32)
        want = orc.combine(ws, slot, w, gates is not None, 64)
        x = np.zeros((1, 64), np.uint16)
        ids = np.arange(k, dtype=np.int32).reshape(1, k)
        run = gpu_dispatch(x, ids, k, k, 1)        # copy j -> region j, row 0
        run.ws.copy_(to_dev_bf16(ws).view(run.ws.shape))
        out = to_u16(moe.moe_combine(run.h, run.ws, to_dev(w), gates is not None))
        assert np.array_equal(out, want), (vals, gates, hex(out[0, 0]), hex(want[0, 0]))


@pytest.mark.parametrize("golden,key", [("reduction_probe.txt", "fp32_then_narrow"),
                                        ("power_of_two_probe.txt", "expected")])
def test_page_probes_on_gpu(golden, key):
    say("page probe", golden)
    g = pins.read_golden(golden)
    vals = [float(v) for v in g["contributions"][0]]
    ws, slot = pins.one_token_case(vals, H=64)
    k = len(vals)
    run = gpu_dispatch(np.zeros((1, 64), np.uint16), np.arange(k, dtype=np.int32).reshape(1, k),
                       k, k, 1)
    run.ws.copy_(to_dev_bf16(ws).view(run.ws.shape))
    out = to_u16(moe.moe_combine(run.h, run.ws, None, False))
    assert (out == pins.exact_bits(float(g[key][0][0]))).all()


def test_page_staged_sum_on_gpu():
    say("staged sum probe")
    g = pins.read_golden("staged_sum.txt")
    vals = [0.0] * 8
    present = [int(r) for r, _ in g["contribution"]]
    for r, v in g["contribution"]:
        vals[int(r)] = float(v)
    ids = np.array([[r if r in present else -1 for r in range(8)]], np.int32)
    ws, _ = pins.one_token_case(vals, H=64, missing=[r for r in range(8) if r not in present])
    run = gpu_dispatch(np.zeros((1, 64), np.uint16), ids, 8, 8, 1)
    run.ws.copy_(to_dev_bf16(ws).view(run.ws.shape))
    out = to_u16(moe.moe_combine(run.h, run.ws, None, False))
    assert (out == pins.exact_bits(float(g["expected"][0][0]))).all()
    # the missing region's row was never written and never read
    assert bool((run.ws[3].view(torch.int16) == CANARY).all())


@pytest.mark.parametrize("fused", [False, True], ids=["combine", "fused"])
def test_outputs_past_the_cached_store_limit(fused):
    # launches writing more than 120 MiB of output use non-temporal stores
    # instead of cache-resident ones: T * H * 2 bytes (twice that when fused)
    T = 4608 if fused else 9216
    H, k, E, ep = 7168, 2, 16, 4
    assert T * H * 2 * (2 if fused else 1) > 120 << 20
    say("outputs past the cached-store limit", "fused" if fused else "combine", T)
    rng = np.random.default_rng(77)
    x = pins.random_bf16(rng, (T, H))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    y = pins.random_bf16(rng, (T * k, H))
    roundtrip(x, ids, w, y, E, ep, cap=T * k, fused=fused)


@pytest.mark.parametrize("eps", [1e-6, 0.0], ids=["eps_1e-6", "eps_0"])
def test_fused_epilogue_over_the_whole_bf16_range(eps):
    # The epilogue takes the sum of squares, its root and the normalising
    # product in fp64, so rows far from fp32's comfortable range still match
    # the oracle (fp64): elements near 2^100 and 2^120 (their squares
    # overflow fp32), near 2^-100 and 2^-120 (their squares underflow fp32;
    # with eps = 0 nothing else keeps the root off zero), a token with no
    # copy and a zero residual (eps > 0: +0; eps = 0: 0/0, NaN on both sides)
    # and ordinary rows.
    from oracle import compare
    T, H, k, E, ep = 8, 256, 2, 4, 2
    rng = np.random.default_rng(123)
    x = pins.random_bf16(rng, (T, H))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[2] = -1
    w = rng.random((T, k)).astype(np.float32)
    scale = np.ones(T, np.float32)
    scale[[0, 1, 5, 6]] = np.float32(2.0 ** 100), np.float32(2.0 ** -100), np.float32(2.0 ** 120), \
        np.float32(2.0 ** -120)
    yf = rng.standard_normal((T * k, H)).astype(np.float32) * np.repeat(scale, k)[:, None]
    rf = rng.standard_normal((T, H)).astype(np.float32) * scale[:, None]
    rf[2] = 0.0
    y, res = pins.torch_bf16_bits(yf), pins.torch_bf16_bits(rf)
    gamma = pins.torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    say("fused epilogue over the bf16 range", "eps", eps)
    orc = oracle.load()
    ref = orc.dispatch(x, ids, ep, E // ep, T * k)
    expert_stage_oracle(ref, y)
    run = gpu_dispatch(x, ids, E, ep, T * k)
    expert_stage_gpu(run, y)
    r_out, normed = moe.moe_combine_residual_rmsnorm(run.h, run.ws, to_dev(w), True,
                                                     to_dev_bf16(res), to_dev_bf16(gamma), eps)
    want_r, want_n = orc.combine_residual_rmsnorm(ref.ws, ref.slot_index, w, True, res, gamma, eps)
    assert_bf16_close(to_u16(r_out), want_r, "residual_out")
    got = to_u16(normed)
    gn, wn = compare.is_nan_bits(got), compare.is_nan_bits(want_n)
    assert np.array_equal(gn, wn), "NaN positions differ"
    assert bool(gn[2].all()) == (eps == 0.0) and not gn[[0, 1, 3, 4, 5, 6, 7]].any()
    assert_bf16_close(np.where(gn, 0, got).astype(np.uint16),
                      np.where(wn, 0, want_n).astype(np.uint16), "normed")
    # the huge rows (and, without eps, the tiny ones) normalise to unit scale
    vals = (got.astype(np.uint32) << 16).view(np.float32)
    rows = [0, 5] + ([1, 6] if eps == 0.0 else [])
    rms = np.sqrt(np.mean(vals[rows].astype(np.float64) ** 2, axis=1))
    assert ((rms > 0.5) & (rms < 2.0)).all(), rms


@pytest.mark.parametrize("fused", [False, True], ids=["combine", "fused"])
def test_nonfinite_expert_outputs_propagate(fused):
    # NaN and +-Inf entries in the expert outputs propagate as IEEE arithmetic
    # says on both sides (Inf - Inf and 0 * Inf give NaN; an Inf in a row
    # makes the RMSNorm of that row 0 or NaN).  Where either output is NaN
    # both must be (NaN bits may differ: the sign of a NaN produced by
    # arithmetic is unspecified); everything else bit for bit.
    from oracle import compare
    T, H, k, E, ep = 64, 256, 4, 16, 4
    rng = np.random.default_rng(91)
    x = pins.random_bf16(rng, (T, H))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    w[::7, 0] = 0.0                                  # 0 * Inf where an Inf lands there
    y = pins.random_bf16(rng, (T * k, H))
    for bits, share in ((0x7FC0, 0.002), (0x7F80, 0.003), (0xFF80, 0.003)):
        y[rng.random(y.shape) < share] = bits
    say("non-finite expert outputs", "fused" if fused else "combine")
    orc = oracle.load()
    ref = orc.dispatch(x, ids, ep, E // ep, T * k)
    expert_stage_oracle(ref, y)

    def close(got, want, what):
        gn, wn = compare.is_nan_bits(got), compare.is_nan_bits(want)
        assert np.array_equal(gn, wn), f"{what}: NaN positions differ ({int(gn.sum())} vs {int(wn.sum())})"
        d = compare.ulp_distance(np.where(gn, 0, got).astype(np.uint16), np.where(wn, 0, want).astype(np.uint16))
        assert int(d.max()) == 0, f"{what}: {int(d.max())} ulp"
        return int(gn.sum())

    for weighted in (False, True):
        run = gpu_dispatch(x, ids, E, ep, T * k)
        expert_stage_gpu(run, y)
        if fused:
            res = pins.random_bf16(rng, (T, H))
            gamma = pins.torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
            r_out, normed = moe.moe_combine_residual_rmsnorm(
                run.h, run.ws, to_dev(w) if weighted else None, weighted, to_dev_bf16(res),
                to_dev_bf16(gamma), 1e-6)
            want_r, want_n = orc.combine_residual_rmsnorm(ref.ws, ref.slot_index, w, weighted, res,
                                                          gamma, 1e-6)
            close(to_u16(r_out), want_r, "residual_out")
            n = close(to_u16(normed), want_n, "normed")
        else:
            got = to_u16(moe.moe_combine(run.h, run.ws, to_dev(w) if weighted else None, weighted))
            n = close(got, orc.combine(ref.ws, ref.slot_index, w, weighted, H), "combine")
        assert n > 0                                  # the case does produce NaNs
