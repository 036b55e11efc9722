"""moe_dispatch_noalloc: the dispatch whose routing scratch is a static array
in the library's device code, checked against moe_dispatch.

Two calls in a row on one handle that binds no scratch of its own, the
second with a smaller batch, both above the single-launch limit (so the
routing kernel and the copy kernel use the static array).  Each is called
through the C ABI and compared with moe_dispatch on a separate handle and
the same inputs: counts, slot_index, src_index and every workspace byte
(padding included) must be equal, and so must the combines that follow.
"""
import ctypes

import numpy as np
import pytest
import torch

import combine_moe_dispatch_03_amd as moe
import pins
from gpu_harness import CANARY, say, to_dev, to_dev_bf16, to_u16

pytestmark = pytest.mark.gpu


def test_noalloc_dispatch_matches_dispatch_on_two_calls():
    T_max, H, k, E, ep = 4096, 256, 8, 64, 8
    cap = T_max * k
    rng = np.random.default_rng(77)
    h_ref = moe.MoeA2A(T_max, H, k, E, ep, cap)
    h_na = moe.MoeA2A(T_max, H, k, E, ep, cap, scratch=False)
    assert h_na.handle.scratch is None and h_na.handle.scratch_bytes == 0
    lib = moe.library()
    for T in (4096, 3000):                      # the second call is smaller
        say("noalloc dispatch", T, H, k, E, ep)
        x = to_dev_bf16(pins.random_bf16(rng, (T, H)))
        ids_np = rng.integers(0, E, size=(T, k)).astype(np.int32)
        ids_np[rng.random((T, k)) < 0.05] = -1
        ids = to_dev(ids_np)
        ws_ref, ws_na = h_ref.new_workspace(CANARY), h_na.new_workspace(CANARY)
        moe.moe_dispatch(h_ref, x, ids, T_max, ws_ref)
        stream = torch.cuda.current_stream().cuda_stream
        rc = lib.moe_dispatch_noalloc(ctypes.byref(h_na.handle), x.data_ptr(), ids.data_ptr(), T,
                                      T_max, ws_na.data_ptr(), stream)
        assert rc == moe.MOE_OK, moe.moe_strerror(rc)
        assert moe.moe_sync_status(h_ref) == (moe.MOE_OK, 0)
        assert moe.moe_sync_status(h_na) == (moe.MOE_OK, 0)
        assert h_na.handle.phase == 1 and h_na.handle.num_tokens == T
        assert torch.equal(h_na.counts, h_ref.counts)
        assert torch.equal(h_na.slot_index_view(), h_ref.slot_index_view())
        assert torch.equal(h_na.src_index, h_ref.src_index)
        assert torch.equal(ws_na.view(torch.int16), ws_ref.view(torch.int16))
        out_ref = moe.moe_combine(h_ref, ws_ref)
        out_na = moe.moe_combine(h_na, ws_na)
        assert np.array_equal(to_u16(out_na), to_u16(out_ref))
        assert h_na.handle.phase == 0


def test_noalloc_handle_rejects_the_scratch_calls():
    h = moe.MoeA2A(64, 128, 2, 8, 4, 128, scratch=False)
    x = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((8, 2), dtype=torch.int32, device="cuda")
    ws = h.new_workspace(0)
    with pytest.raises(moe.MoeError) as err:
        moe.moe_dispatch(h, x, ids, 8, ws)
    assert err.value.code == moe.MOE_ERR_ARG
    with pytest.raises(moe.MoeError) as err:
        moe.moe_route_counts(h, ids)
    assert err.value.code == moe.MOE_ERR_ARG
    moe.moe_dispatch_noalloc(h, x, ids, 8, ws)    # the small path: no scratch at all
    assert moe.moe_sync_status(h) == (moe.MOE_OK, 0)
    moe.moe_reset(h)
