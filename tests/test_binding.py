"""The Python binding's own logic: argument checks and the stream it launches
on.  The checks run on every call, so they are one combined test on the
common path with the messages built only on failure; these tests pin the
messages and that nothing malformed slips through."""
import ctypes
import os

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
        moe._need(t, "x", torch.bfloat16, 0, shape=(4, 8))


def test_partials_on_the_host_are_rejected_before_the_library():
    # the partials tensor names the device; a host tensor must not reach a launch
    cpu = torch.zeros(2, 4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="must be on the GPU"):
        moe.moe_partials_reduce(cpu)
    with pytest.raises(ValueError, match="must be on the GPU"):
        moe.moe_partials_reduce_residual_rmsnorm(cpu, torch.zeros(4, 8, dtype=torch.bfloat16),
                                                 torch.ones(8, dtype=torch.bfloat16), 1e-6)


def test_handle_on_the_host_is_rejected():
    # its index buffers are written by the kernels, so they must be device memory
    with pytest.raises(ValueError, match="needs a GPU device"):
        moe.MoeA2A(64, 128, 2, 8, 4, 128, device="cpu")


def test_explicit_stream_handles_pass_through():
    class FakeStream:
        cuda_stream = 0x1234
    assert moe._stream(FakeStream(), 0) == 0x1234
    assert moe._stream(0x5678, 0) == 0x5678


@pytest.mark.gpu
def test_partials_outputs_on_another_device_kind_are_rejected():
    pd = torch.zeros(2, 4, 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="must be on the GPU"):
        moe.moe_partials_reduce(pd, out=torch.zeros(4, 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must be on the GPU"):
        moe.moe_partials_reduce_residual_rmsnorm(pd, torch.zeros(4, 8, dtype=torch.bfloat16),
                                                 torch.ones(8, dtype=torch.bfloat16, device="cuda"),
                                                 1e-6)


@pytest.mark.gpu
def test_need_rejects_shape_layout_and_size_on_gpu():
    t = torch.zeros(4, 8, dtype=torch.bfloat16, device="cuda")
    moe._need(t, "x", torch.bfloat16, 0, shape=(4, 8), numel=32)
    with pytest.raises(ValueError, match=r"must have shape \(4, 9\)"):
        moe._need(t, "x", torch.bfloat16, 0, shape=(4, 9))
    with pytest.raises(ValueError, match="must be contiguous"):
        moe._need(t.t(), "x", torch.bfloat16, 0, shape=(8, 4))
    with pytest.raises(ValueError, match="must have 33 elements"):
        moe._need(t, "x", torch.bfloat16, 0, numel=33)
    # a handle bound to another device index rejects this device's tensors
    with pytest.raises(ValueError, match="must be on the handle's device cuda:1"):
        moe._need(t, "x", torch.bfloat16, 1, shape=(4, 8))


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


FAKE = 0x100000   # aligned, never dereferenced by the host-side checks


def fake_handle(k=2):
    lib = moe.library()
    h = moe.MoeHandle()
    rc = lib.moe_init(ctypes.byref(h), 64, 128, k, 8, 4, 128, 0, FAKE, FAKE, FAKE, FAKE, FAKE,
                      lib.moe_scratch_bytes(64, k, 4))
    assert rc == moe.MOE_OK
    return h


def test_fast_module_is_the_in_tree_build():
    fast = moe._fast()
    assert os.path.samefile(fast.__file__, moe.FAST_MODULE)


def test_fast_calls_reject_malformed_arguments():
    fast = moe._fast()
    with pytest.raises(TypeError, match="takes 7 arguments"):
        fast.dispatch(0, 0, 0)
    with pytest.raises(OverflowError):
        fast.dispatch(ctypes.addressof(fake_handle()), FAKE, FAKE, 1 << 40, 1, FAKE, None)
    with pytest.raises(TypeError):
        fast.combine(ctypes.addressof(fake_handle()), "not a pointer", None, 0, FAKE, None)


def test_fast_calls_return_the_library_codes():
    # host-side rejections (no HIP call): the extension and ctypes give the same code
    lib, fast = moe.library(), moe._fast()
    cases = [
        ("combine before dispatch", lambda h, a: fast.combine(a, FAKE, None, 0, FAKE, None),
         lambda h: lib.moe_combine(ctypes.byref(h), FAKE, None, 0, FAKE, None)),
        ("null workspace", lambda h, a: fast.dispatch(a, FAKE, FAKE, 8, 8, None, None),
         lambda h: lib.moe_dispatch(ctypes.byref(h), FAKE, FAKE, 8, 8, None, None)),
        ("rung above max_tokens", lambda h, a: fast.dispatch(a, FAKE, FAKE, 8, 65, FAKE, None),
         lambda h: lib.moe_dispatch(ctypes.byref(h), FAKE, FAKE, 8, 65, FAKE, None)),
        ("misaligned rows", lambda h, a: fast.dispatch(a, FAKE + 2, FAKE, 8, 8, FAKE, None),
         lambda h: lib.moe_dispatch(ctypes.byref(h), FAKE + 2, FAKE, 8, 8, FAKE, None)),
        ("fp8 null scales", lambda h, a: fast.dispatch_fp8(a, FAKE, FAKE, 8, 8, FAKE, None, None),
         lambda h: lib.moe_dispatch_fp8(ctypes.byref(h), FAKE, FAKE, 8, 8, FAKE, None, None)),
        ("fused before dispatch",
         lambda h, a: fast.combine_residual_rmsnorm(a, FAKE, None, 0, FAKE, FAKE, FAKE, 1e-6, FAKE, None),
         lambda h: lib.moe_combine_residual_rmsnorm(ctypes.byref(h), FAKE, None, 0, FAKE, FAKE, FAKE,
                                                    1e-6, FAKE, None)),
        ("route counts above max_tokens", lambda h, a: fast.route_counts(a, FAKE, 65, None),
         lambda h: lib.moe_route_counts(ctypes.byref(h), FAKE, 65, None)),
    ]
    for name, via_fast, via_ctypes in cases:
        h1, h2 = fake_handle(), fake_handle()
        got = via_fast(h1, ctypes.addressof(h1))
        want = via_ctypes(h2)
        assert got == want != moe.MOE_OK, name
