"""The oracle against the exact-rational brute force on random shapes.

The pins check the oracle on exhaustive tiny routings and on hand-built
cases; here hypothesis draws the shape (tokens, hidden size, top-k, regions,
experts per region, capacity), the share of unrouted copies and of ids
outside [-1, E), and a seed for the values, and every drawn case must agree
bit for bit with oracle/brute.py: dispatch (counts, status, slot_index,
src_index, rows) in both layouts, the weighted and unweighted combine, the
per-region combine and the fused residual + RMSNorm epilogue; and for the
reduction of P tensor-parallel partials (plain and fused), random P, T, H,
eps and value scale.  Runs are derandomized, so the suite is reproducible.
"""
import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from oracle import brute
from pins import random_bf16, torch_bf16_bits

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True)


@st.composite
def routings(draw, max_tokens=12, hidden=(1, 2, 3, 8)):
    ep = draw(st.integers(1, 6))
    epr = draw(st.integers(1, 4))
    k = draw(st.integers(1, 5))
    T = draw(st.integers(0, max_tokens))
    H = draw(st.sampled_from(hidden))
    cap = draw(st.integers(1, max(1, T * k)))
    p_missing = draw(st.sampled_from([0.0, 0.2, 0.5]))
    p_bad = draw(st.sampled_from([0.0, 0.0, 0.1]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    E = ep * epr
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)      # repeats allowed
    ids[rng.random((T, k)) < p_missing] = -1
    bad = rng.random((T, k)) < p_bad
    ids[bad] = rng.choice(np.array([-3, -2, E, E + 1], np.int32), size=int(bad.sum()))
    x = random_bf16(rng, (T, H))
    return dict(T=T, H=H, k=k, ep=ep, epr=epr, cap=cap, ids=ids, x=x, rng=rng)


def check_dispatch(d, brute_result):
    rows, counts, slot, src, status = brute_result
    assert d.status == status
    assert list(d.counts) == counts
    assert d.slot_index.tolist() == slot
    for (r, s), f in src.items():
        assert d.src_index[r, s] == f
        assert d.ws[r, s].tolist() == rows[(r, s)]


def staged_workspace(d, rng, H):
    """Fill every workspace row with fresh expert outputs; the dict form the
    brute force reads."""
    d.ws[...] = random_bf16(rng, d.ws.shape)
    ep, cap = d.ws.shape[:2]
    return {(r, s): list(d.ws[r, s]) for r in range(ep) for s in range(cap)}


@SETTINGS
@given(routings())
def test_per_copy_dispatch_and_combine_match_brute_force(c):
    orc = oracle.load()
    T, H, k, ep, epr, cap = c["T"], c["H"], c["k"], c["ep"], c["epr"], c["cap"]
    d = orc.dispatch(c["x"], c["ids"], ep, epr, cap)
    check_dispatch(d, brute.dispatch(c["x"], c["ids"], ep, epr, cap))
    rows = staged_workspace(d, c["rng"], H)
    w = c["rng"].standard_normal((T, k)).astype(np.float32)
    for weighted in (False, True):
        got = orc.combine(d.ws, d.slot_index, w, weighted, H)
        assert got.tolist() == brute.combine(rows, d.slot_index.tolist(), w.tolist(), weighted,
                                             T, H, cap)


@SETTINGS
@given(routings())
def test_per_region_dispatch_and_combine_match_brute_force(c):
    orc = oracle.load()
    T, H, ep, epr, cap = c["T"], c["H"], c["ep"], c["epr"], c["cap"]
    d = orc.dispatch(c["x"], c["ids"], ep, epr, cap, layout="region")
    check_dispatch(d, brute.dispatch_region(c["x"], c["ids"], ep, epr, cap))
    rows = staged_workspace(d, c["rng"], H)
    got = orc.combine(d.ws, d.slot_index, None, False, H, layout="region")
    assert got.tolist() == brute.combine_region(rows, d.slot_index.tolist(), T, H, cap)


@settings(max_examples=25, deadline=None, derandomize=True)
@given(routings(max_tokens=3, hidden=(1, 4, 8)), st.sampled_from([0.0, 1e-6, 0.25]))
def test_fused_epilogue_matches_brute_force(c, eps):
    orc = oracle.load()
    T, H, k, ep, epr, cap = c["T"], c["H"], c["k"], c["ep"], c["epr"], c["cap"]
    rng = c["rng"]
    d = orc.dispatch(c["x"], c["ids"], ep, epr, cap)
    rows = staged_workspace(d, rng, H)
    w = rng.random((T, k)).astype(np.float32)
    res = random_bf16(rng, (T, H))
    gamma = torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    for weighted in (False, True):
        r_out, normed = orc.combine_residual_rmsnorm(d.ws, d.slot_index, w, weighted, res, gamma, eps)
        want_r, want_n = brute.combine_residual_rmsnorm(rows, d.slot_index.tolist(), w.tolist(),
                                                        weighted, res.tolist(), gamma.tolist(), eps,
                                                        T, H, cap)
        assert r_out.tolist() == want_r
        assert normed.tolist() == want_n


@settings(max_examples=30, deadline=None, derandomize=True)
@given(st.integers(1, 9), st.integers(0, 4), st.sampled_from([1, 2, 8]),
       st.sampled_from([0.0, 1e-6, 0.25]), st.integers(0, 2 ** 31 - 1))
def test_partials_reduction_matches_brute_force(P, T, H, eps, seed):
    # partial p of token t is row (p, t) of a workspace with cap = T
    orc = oracle.load()
    rng = np.random.default_rng(seed)
    partials = random_bf16(rng, (P, T, H), scale=float(rng.choice([1.0, 1e-3, 1e3])))
    rows = {(p, t): list(partials[p, t]) for p in range(P) for t in range(T)}
    slot = [[p * T + t for p in range(P)] for t in range(T)]
    cap = max(T, 1)
    assert orc.partials_reduce(partials).tolist() == brute.combine(rows, slot, None, False, T, H, cap)
    res = random_bf16(rng, (T, H))
    gamma = torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    r_out, normed = orc.partials_reduce_residual_rmsnorm(partials, res, gamma, eps)
    want_r, want_n = brute.combine_residual_rmsnorm(rows, slot, None, False, res.tolist(),
                                                    gamma.tolist(), eps, T, H, cap)
    assert r_out.tolist() == want_r
    assert normed.tolist() == want_n
