"""dispatch + combine captured in a HIP graph (torch.cuda.CUDAGraph).

The hot-path calls only enqueue kernels (no host synchronisation, no memset),
so a caller can capture them.  Each graph is replayed several times with the
program's own eager work and synchronisations in between, and every replay is
checked bit for bit against the eager result.  (moe_sync_status synchronises
and is not captured.)
"""
import numpy as np
import pytest
import torch

import combine_moe_dispatch_03_amd as moe
import synth
from gpu_harness import FP8_FILL, say, to_dev, to_dev_bf16, to_u16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,layout,fused", [("decode", "copy", False),
                                               ("decode", "region", False),
                                               ("fused", "copy", True)])
def test_graph_replays_match_eager(name, layout, fused):
    wl = synth.BY_NAME[name]
    say("graph", name, layout, "fused" if fused else "")
    inp = synth.make_inputs(wl, 0)
    x, ids = to_dev_bf16(inp.x), to_dev(inp.ids)
    weighted = layout == "copy"
    w = to_dev(inp.weights) if weighted else None
    cap = wl.cap if layout == "copy" else wl.T
    h = moe.MoeA2A(wl.R, wl.H, wl.k, wl.E, wl.ep, cap, layout=layout)
    ws = h.new_workspace(0)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    if fused:
        res, gamma = to_dev_bf16(inp.residual), to_dev_bf16(inp.gamma)
        res_out = torch.empty_like(res)

    def step():
        moe.moe_dispatch(h, x, ids, wl.R, ws)
        if fused:
            moe.moe_combine_residual_rmsnorm(h, ws, w, weighted, res, gamma, wl.eps,
                                             residual_out=res_out, normed=out)
        else:
            moe.moe_combine(h, ws, w, weighted, out=out)

    step()                                            # eager reference
    torch.cuda.synchronize()
    assert moe.moe_sync_status(h) == (moe.MOE_OK, 0)
    want = [to_u16(out), h.slot_index_view().cpu().numpy().copy()]
    if fused:
        want.append(to_u16(res_out))

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                        # warm the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    assert h.handle.phase == 0

    for rep in range(4):
        out.zero_()                                   # eager work between replays
        h.slot_index.fill_(-7)
        if fused:
            res_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [to_u16(out), h.slot_index_view().cpu().numpy()]
        if fused:
            got.append(to_u16(res_out))
        for a, b in zip(got, want):
            assert np.array_equal(a, b), f"replay {rep} differs"
    assert moe.moe_sync_status(h) == (moe.MOE_OK, 0)


def test_fp8_graph_replays_match_eager():
    """The fp8 dispatch at 16,384 copies: eagerly the single pass, captured
    the routing kernel + copy kernel (a captured epoch would be stale on
    replay).  Every replay's codes, scales (padding fill included) and index
    maps equal the eager call's bit for bit."""
    wl = synth.BY_NAME["fused"]
    say("graph", "fp8", wl.T * wl.k, "copies")
    inp = synth.make_inputs(wl, 1)
    x, ids = to_dev_bf16(inp.x), to_dev(inp.ids)
    h = moe.MoeA2A(wl.R, wl.H, wl.k, wl.E, wl.ep, wl.cap)
    ws = h.new_workspace_fp8(FP8_FILL)
    scales = h.new_scales()

    def step():
        moe.moe_dispatch_fp8(h, x, ids, wl.R, ws, scales)
        moe.moe_reset(h)

    def snapshot():                                   # on the GPU: the workspace is 940 MB
        return [ws.clone(), scales.view(torch.int32).clone(), h.counts.clone(),
                h.slot_index_view().clone(), h.src_index.clone()]

    step()                                            # eager: the single pass
    torch.cuda.synchronize()
    assert moe.moe_sync_status(h) == (moe.MOE_OK, 0)
    assert h.handle.onepass_epoch == 1
    want = snapshot()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                        # warm the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    assert h.handle.onepass_epoch == 2                # the capture took no epoch

    for rep in range(4):
        ws.fill_(FP8_FILL)                            # eager work between replays
        scales.fill_(float("nan"))
        h.slot_index.fill_(-7)
        h.src_index.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(snapshot(), want)):
            assert torch.equal(a, b), f"replay {rep} differs in output {i}"
    assert moe.moe_sync_status(h) == (moe.MOE_OK, 0)


def test_partials_graph_replays_match_eager():
    # the partials reduction fused with residual + RMSNorm, then the plain
    # reduction, captured together
    P, T, H = 8, 512, 7168
    say("graph", "partials", P, T, H)
    partials, residual, gamma = synth.make_partials(synth.PartialsWorkload("graph", P, T, H), 3)
    pd, rd, gd = to_dev_bf16(partials), to_dev_bf16(residual), to_dev_bf16(gamma)
    ro, nd, od = torch.empty_like(rd), torch.empty_like(rd), torch.empty_like(rd)

    def step():
        moe.moe_partials_reduce_residual_rmsnorm(pd, rd, gd, 1e-6, residual_out=ro, normed=nd)
        moe.moe_partials_reduce(pd, out=od)

    step()
    torch.cuda.synchronize()
    want = [to_u16(ro), to_u16(nd), to_u16(od)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (ro, nd, od):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip([to_u16(ro), to_u16(nd), to_u16(od)], want):
            assert np.array_equal(a, b), f"replay {rep} differs"
