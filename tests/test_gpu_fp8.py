"""Parity of the FP8 (OCP E4M3) dispatch payload with the oracle on the GPU.

Codes, per-row scales, counts, slot_index and src_index must match the
oracle bit for bit (the quantisation is fp32 arithmetic plus a
nearest-even conversion on both sides); padding bytes and scales keep their
NaN fill.  Full prefill / decode / skewed shapes, both layouts and every
dispatch path (single launch, single pass, routing then copy), plus rows
that exercise zero, subnormal and saturating codes.
"""
import numpy as np
import pytest

import oracle
import pins
import synth
from gpu_harness import fp8_check, say

pytestmark = pytest.mark.gpu

@pytest.mark.parametrize("name,layout", [("prefill", "copy"), ("decode", "copy"),
                                         ("skewed", "copy"), ("prefill", "region"),
                                         ("decode", "region")])
def test_fp8_dispatch_full_size(name, layout):
    wl = synth.BY_NAME[name]
    say("fp8 dispatch", name, layout)
    inp = synth.make_inputs(wl, 0)
    cap = wl.T if layout == "region" else wl.cap
    if cap is None:
        cap = int(oracle.load().dispatch(np.zeros((wl.T, 1), np.uint16), inp.ids, wl.ep, wl.epr,
                                         wl.T * wl.k).counts.max())
    fp8_check(inp.x, inp.ids, wl.E, wl.ep, cap, R=wl.R, layout=layout)


def test_fp8_rows_with_zero_subnormal_and_extreme_values():
    say("fp8 special rows")
    rng = np.random.default_rng(3)
    T, H, k, E, ep = 12, 256, 2, 8, 4
    xf = rng.standard_normal((T, H)).astype(np.float32)
    xf[0] = 0.0                                        # all zero: scale 0, codes 0
    xf[1] = 0.0
    xf[1, 7] = -5.0                                    # one element: -448, rest zero
    xf[2] *= np.float32(2.0 ** -100)                   # tiny magnitudes
    xf[3] *= np.float32(2.0 ** 100)                    # huge magnitudes
    xf[4, :] = rng.standard_normal(H).astype(np.float32) * 1e-4
    xf[4, 0] = 300.0                                   # most codes subnormal or zero
    xf[5, :] = 1.0                                     # constant row
    x = pins.torch_bf16_bits(xf)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    fp8_check(x, ids, E, ep, T * k)


@pytest.mark.parametrize("T,H", [(37, 136), (5, 16384), (2500, 64)])
def test_fp8_ragged_and_larger_shapes(T, H):
    # 7500 copies at T = 2500: the single pass (per copy) and the two kernels
    # (per region); the others one launch
    say("fp8 shapes", T, H)
    rng = np.random.default_rng(T + H)
    x = pins.random_bf16(rng, (T, H))
    ids = rng.integers(-1, 24, size=(T, 3)).astype(np.int32)
    fp8_check(x, ids, 24, 4, T * 3)
    fp8_check(x, ids, 24, 4, T, layout="region")


@pytest.mark.parametrize("k", [8, 6, 3])
@pytest.mark.parametrize("many", [False, True], ids=["single_launch", "routed"])
def test_fp8_split_blocks(k, many):
    # rows of 8 KB and more: the fp8 copy runs four copies per block (two
    # blocks a token at top-8 and top-6, the second partial for top-6; one
    # partial block at top-3); 2100 to 2400 copies take the single launch,
    # 9000 and more the single pass (per copy; four copies a block above
    # 8192 copies) or the two kernels (per region)
    H, E, ep = 4096, 64, 8
    T = 9000 // k + 1 if many else max(300, 2100 // k)
    say("fp8 split blocks", T, H, k)
    rng = np.random.default_rng(100 + k)
    x = pins.random_bf16(rng, (T, H))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[rng.random(ids.shape) < 0.05] = -1
    fp8_check(x, ids, E, ep, T * k)
    fp8_check(x, ids, E, ep, T, layout="region")


@pytest.mark.parametrize("T", [1024, 1025, 3072, 3073])
def test_fp8_block_sizes_at_the_whole_token_limits(T):
    # a whole token per block up to 8192 copies in the single pass (per
    # copy) and up to 24576 in the routed copy (per region), four copies
    # per block above
    H, k, E, ep = 4096, 8, 64, 8
    say("fp8 block sizes", T)
    rng = np.random.default_rng(300 + T)
    x = pins.random_bf16(rng, (T, H))
    ids = rng.integers(-1, E, size=(T, k)).astype(np.int32)
    fp8_check(x, ids, E, ep, T * k, epoch=1)
    fp8_check(x, ids, E, ep, T, layout="region", epoch=0)


def test_fp8_bad_ids_and_overflow():
    say("fp8 bad ids / overflow")
    rng = np.random.default_rng(9)
    T, H, k, E, ep = 50, 64, 4, 8, 2
    x = pins.random_bf16(rng, (T, H))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[4, 1] = 99
    ref = fp8_check(x, ids, E, ep, 60)
    assert ref.status == oracle.STATUS_BAD_ID | oracle.STATUS_OVERFLOW
