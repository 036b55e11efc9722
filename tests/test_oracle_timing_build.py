"""The CPU baseline's build of the oracle (-O3 -march=native, the same
source and arithmetic flags) computes the same bytes as the parity build, on
the small workloads and a cut of the fused one."""
import numpy as np

import oracle
import synth


def test_timing_build_matches_parity_build():
    fast = oracle.load_timing(rebuild=True)
    ref = oracle.load()
    for name in ("tiny", "decode"):
        wl = synth.BY_NAME[name]
        inp = synth.make_inputs(wl, 0)
        a = ref.dispatch(inp.x, inp.ids, wl.ep, wl.epr, wl.cap)
        b = fast.dispatch(inp.x, inp.ids, wl.ep, wl.epr, wl.cap)
        assert np.array_equal(a.counts, b.counts) and np.array_equal(a.slot_index, b.slot_index)
        assert np.array_equal(a.src_index, b.src_index)
        for r in range(wl.ep):
            n = int(a.counts[r])
            assert np.array_equal(a.ws[r, :n], b.ws[r, :n])
        for weighted in (False, True):
            assert np.array_equal(ref.combine(a.ws, a.slot_index, inp.weights, weighted, wl.H),
                                  fast.combine(b.ws, b.slot_index, inp.weights, weighted, wl.H))
    wl = synth.BY_NAME["fused"]
    inp = synth.make_inputs(wl, 0)
    T = 64
    x, ids, w = inp.x[:T], inp.ids[:T], inp.weights[:T]
    a = ref.dispatch(x, ids, wl.ep, wl.epr, T * wl.k)
    b = fast.dispatch(x, ids, wl.ep, wl.epr, T * wl.k)
    ra, na = ref.combine_residual_rmsnorm(a.ws, a.slot_index, w, True, inp.residual[:T],
                                          inp.gamma, wl.eps)
    rb, nb = fast.combine_residual_rmsnorm(b.ws, b.slot_index, w, True, inp.residual[:T],
                                           inp.gamma, wl.eps)
    assert np.array_equal(ra, rb) and np.array_equal(na, nb)
