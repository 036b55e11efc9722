"""Parity of the partials reduction (the local half of a tensor-parallel
all-reduce) and its fused residual + RMSNorm form with the CPU oracle.

magik.net "Fusing the Allreduce: A Precision Investigation into FlashInfer's
Verify-Path Optimization", section "The Message Itself: Explanation and
Probe": the all-reduce of the hidden states and the residual add + RMSNorm
become one kernel.  On one GPU the P partials [P, T, H] are local; the sum
must equal the oracle bit for bit (fp32 in rank order, one narrowing), the
fused outputs too, and the normalised output is also checked against 1e-2
relative error (0.02 magnitude floor).  The full-size case is the shape the
benchmark times: 8 ranks, 2048 tokens, hidden 7168.
"""
import numpy as np
import pytest
import torch

import combine_moe_dispatch_03_amd as moe
import oracle
import synth
from gpu_harness import assert_bf16_close, say, to_dev_bf16, to_u16
from oracle import compare

pytestmark = pytest.mark.gpu

CASES = [
    # (P, T, H): the benchmark's shape, ragged rows, one rank, the most ranks,
    # one token, several column blocks (plain reduce) and the widest fused row
    (8, 2048, 7168),
    (3, 5, 136),
    (1, 17, 7168),
    (64, 7, 1024),
    (8, 1, 7168),
    (5, 1000, 1024),
    (2, 300, 16384),
    (4, 33, 8),
    (64, 64, 16384),          # the most ranks at the widest fused row
]


def _inputs(P, T, H, seed):
    return synth.make_partials(synth.PartialsWorkload("case", P, T, H), seed)


@pytest.mark.parametrize("P,T,H", CASES, ids=[f"P{p}_T{t}_H{h}" for p, t, h in CASES])
def test_partials_reduce_and_fused(P, T, H):
    say("partials", "P", P, "T", T, "H", H)
    orc = oracle.load()
    partials, residual, gamma = _inputs(P, T, H, seed=P + T + H)
    want = orc.partials_reduce(partials)
    pd = to_dev_bf16(partials)
    out = moe.moe_partials_reduce(pd)
    torch.cuda.synchronize()
    assert_bf16_close(to_u16(out), want, "partials reduce")
    eps = 1e-6
    want_r, want_n = orc.partials_reduce_residual_rmsnorm(partials, residual, gamma, eps)
    rd, gd = to_dev_bf16(residual), to_dev_bf16(gamma)
    r_out, normed = moe.moe_partials_reduce_residual_rmsnorm(pd, rd, gd, eps)
    torch.cuda.synchronize()
    got_r, got_n = to_u16(r_out), to_u16(normed)
    assert_bf16_close(got_r, want_r, "residual_out")
    assert_bf16_close(got_n, want_n, "normed")
    assert compare.rel_err(got_n, want_n) <= 1e-2
    # the residual is untouched when residual_out is another buffer
    assert np.array_equal(to_u16(rd), residual)


def test_partials_reduce_largest_hidden():
    # the plain reduction at MOE_MAX_HIDDEN: rows of 2 MiB over many column blocks
    P, T, H = 3, 2, moe.MOE_MAX_HIDDEN
    say("partials max hidden", P, T, H)
    partials, _, _ = _inputs(P, T, H, seed=9)
    out = moe.moe_partials_reduce(to_dev_bf16(partials))
    torch.cuda.synchronize()
    assert_bf16_close(to_u16(out), oracle.load().partials_reduce(partials), "partials reduce")


@pytest.mark.parametrize("seed", range(20))
def test_partials_random_shapes(seed):
    rng = np.random.default_rng(1000 + seed)
    P = int(rng.integers(1, 17))
    T = int(rng.integers(0, 400))
    H = int(rng.choice([8, 64, 136, 1024, 4104, 7168]))
    eps = float(rng.choice([0.0, 1e-6, 0.5]))
    say("partials random", seed, "P", P, "T", T, "H", H, "eps", eps)
    orc = oracle.load()
    partials, residual, gamma = _inputs(P, T, H, seed=seed)
    pd = to_dev_bf16(partials)
    out = moe.moe_partials_reduce(pd)
    r_out, normed = moe.moe_partials_reduce_residual_rmsnorm(pd, to_dev_bf16(residual),
                                                             to_dev_bf16(gamma), eps)
    torch.cuda.synchronize()
    assert_bf16_close(to_u16(out), orc.partials_reduce(partials), "partials reduce")
    want_r, want_n = orc.partials_reduce_residual_rmsnorm(partials, residual, gamma, eps)
    assert_bf16_close(to_u16(r_out), want_r, "residual_out")
    assert_bf16_close(to_u16(normed), want_n, "normed")


def test_partials_empty_batch():
    pd = torch.empty((8, 0, 7168), dtype=torch.bfloat16, device="cuda")
    out = moe.moe_partials_reduce(pd)
    rd = torch.empty((0, 7168), dtype=torch.bfloat16, device="cuda")
    gd = torch.ones(7168, dtype=torch.bfloat16, device="cuda")
    r_out, normed = moe.moe_partials_reduce_residual_rmsnorm(pd, rd, gd, 1e-6)
    torch.cuda.synchronize()
    assert out.shape == (0, 7168) and r_out.shape == (0, 7168) and normed.shape == (0, 7168)


def test_partials_power_of_two_probe():
    # rank p contributes 2^p to every element: a single reduction gives 255
    # exactly; a rank counted twice or missed changes the sum
    P, T, H = 8, 64, 7168
    partials = np.stack([np.full((T, H), synth.f32_to_bf16_bits(np.float32(2.0 ** p)), np.uint16)
                         for p in range(P)])
    out = to_u16(moe.moe_partials_reduce(to_dev_bf16(partials)))
    assert (out == synth.f32_to_bf16_bits(np.float32(255.0))).all()


def test_partials_fused_in_place_and_repeatable():
    P, T, H = 8, 256, 7168
    orc = oracle.load()
    partials, residual, gamma = _inputs(P, T, H, seed=5)
    want_r, want_n = orc.partials_reduce_residual_rmsnorm(partials, residual, gamma, 1e-6)
    pd, gd = to_dev_bf16(partials), to_dev_bf16(gamma)
    outs = []
    for _ in range(2):
        rd = to_dev_bf16(residual)
        normed = torch.empty_like(rd)
        r_out, normed = moe.moe_partials_reduce_residual_rmsnorm(pd, rd, gd, 1e-6,
                                                                 residual_out=rd, normed=normed)
        torch.cuda.synchronize()
        assert r_out.data_ptr() == rd.data_ptr()
        outs.append((to_u16(rd), to_u16(normed)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert_bf16_close(outs[0][0], want_r, "residual_out in place")
    assert_bf16_close(outs[0][1], want_n, "normed")


def test_partials_binding_rejects_bad_tensors():
    pd = torch.zeros((2, 4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        moe.moe_partials_reduce(pd[0])                               # not [P, T, H]
    with pytest.raises(TypeError):
        moe.moe_partials_reduce(pd.float())
    with pytest.raises(moe.MoeError):
        moe.moe_partials_reduce(torch.zeros((65, 1, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        moe.moe_partials_reduce_residual_rmsnorm(
            pd, torch.zeros((4, 32), dtype=torch.bfloat16, device="cuda"),
            torch.ones(64, dtype=torch.bfloat16, device="cuda"), 1e-6)
