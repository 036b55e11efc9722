"""The Python binding's own logic: argument checks and the stream it launches
on.  The checks run on every call, so they are one combined test on the
common path with the messages built only on failure; these tests pin the
messages and that nothing malformed slips through."""
import pytest
import torch

import combine_moe_dispatch_03_amd as moe


@pytest.mark.parametrize("case, exc, text", [
    ("not_a_tensor", TypeError, "must be a tensor"),
    ("wrong_dtype", TypeError, "must be torch.bfloat16"),
    ("on_cpu", ValueError, "must be on the GPU"),
])
def test_need_rejects(case, exc, text):
    t = {"not_a_tensor": [1, 2], "wrong_dtype": torch.zeros(4, 8, dtype=torch.float32),
         "on_cpu": torch.zeros(4, 8, dtype=torch.bfloat16)}[case]
    with pytest.raises(exc, match=text):
        moe._need(t, "x", torch.bfloat16, shape=(4, 8))


def test_explicit_stream_handles_pass_through():
    class FakeStream:
        cuda_stream = 0x1234
    assert moe._stream(FakeStream(), 0) == 0x1234
    assert moe._stream(0x5678, 0) == 0x5678


@pytest.mark.gpu
def test_need_rejects_shape_layout_and_size_on_gpu():
    t = torch.zeros(4, 8, dtype=torch.bfloat16, device="cuda")
    moe._need(t, "x", torch.bfloat16, shape=(4, 8), numel=32)
    with pytest.raises(ValueError, match=r"must have shape \(4, 9\)"):
        moe._need(t, "x", torch.bfloat16, shape=(4, 9))
    with pytest.raises(ValueError, match="must be contiguous"):
        moe._need(t.t(), "x", torch.bfloat16, shape=(8, 4))
    with pytest.raises(ValueError, match="must have 33 elements"):
        moe._need(t, "x", torch.bfloat16, numel=33)


@pytest.mark.gpu
def test_default_stream_is_torchs_current_stream():
    h = moe.MoeA2A(8, 64, 2, 8, 4, 16)
    assert moe._stream(None, h.device_index) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert moe._stream(None, h.device_index) == side.cuda_stream
        x = torch.randn(8, 64, device="cuda").to(torch.bfloat16)
        ids = torch.randint(0, 8, (8, 2), dtype=torch.int32, device="cuda")
        ws = h.new_workspace(0)
        moe.moe_dispatch(h, x, ids, 8, ws)               # launched on `side`
        out = moe.moe_combine(h, ws)
    side.synchronize()
    want = (x.float() * 2).to(torch.bfloat16)             # both copies of a row, summed once
    assert torch.equal(out, want)
