"""Pins that hold the CPU oracle to something other than itself.

Each ``pin_*`` function takes a compiled oracle and raises AssertionError if
the oracle disagrees with what the pages, the mathematics or an independent
library fix.  The test modules call them one by one; ``test_oracle_mutations``
runs all of them against deliberately broken copies of the oracle to show that
each plausible mistake is caught by at least one pin.

Kinds of pin used here:
  * values the pages print for a worked example (``tests/golden/*.txt``);
  * closed forms (histograms, k*x for identity experts, x for gates summing
    to one, constant-row RMSNorm);
  * independent library routines (torch's bf16 conversions, numpy bincount,
    numpy fp64 textbook RMSNorm);
  * an exact-rational brute force on tiny inputs (``oracle.brute``).
"""
from __future__ import annotations

import itertools
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import brute, compare

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CANARY = 0x7FC0          # bf16 quiet NaN used to mark padding rows


def read_golden(name: str) -> dict:
    """key -> list of whitespace-separated fields (repeated keys accumulate)."""
    out: dict = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            out.setdefault(key, []).append(rest)
    return out


def torch_bf16_bits(a) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def torch_bf16_value(bits) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).float().numpy()


def exact_bits(v: float) -> int:
    return brute.bf16_bits(Fraction(v))


def printed_bits(v: float, decimals: int = 10) -> int:
    """The bf16 pattern a page prints to ``decimals`` places (nearest bf16,
    checked to be within the printed precision)."""
    bits = brute.round_to_bf16_bits(Fraction(v))
    assert abs(float(brute.bf16_value(bits)) - v) <= 0.5 * 10.0 ** -decimals + 1e-15
    return bits


def one_token_case(values, H: int = 8, missing=()):
    """One token with k = len(values) copies, copy j in region j (epr = 1).

    Returns (ws [k, 1, H], slot_index [1, k]); every column of a row holds the
    copy's value (a bf16 value, or a bf16 value printed to 10 decimals);
    regions listed in ``missing`` hold no row (slot -1)."""
    k = len(values)
    ws = np.full((k, 1, H), CANARY, dtype=np.uint16)
    slot = np.full((1, k), -1, dtype=np.int32)
    for j, v in enumerate(values):
        if j in missing:
            continue
        ws[j, 0, :] = printed_bits(v)
        slot[0, j] = j          # row j*cap + 0 with cap = 1
    return ws, slot


def random_bf16(rng, shape, scale=1.0) -> np.ndarray:
    return torch_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


# ---------------------------------------------------------------- codec pins

def pin_codec_page_staged_sum(o):
    g = read_golden("staged_sum.txt")
    s = float(g["sum"][0][0])
    want = exact_bits(float(g["expected"][0][0]))
    got = int(o.f64_to_bf16(np.array([s]))[0])
    assert got == want, (hex(got), hex(want))
    assert got != exact_bits(float(g["wrong"][0][0]))


def pin_codec_ties(o):
    cases = {
        1 + 2 ** -8: 1.0,                    # tie, even neighbour below
        1 + 3 * 2 ** -8: 1 + 2 ** -6,        # tie, even neighbour above
        -(1 + 2 ** -8): -1.0,
        1 + 2 ** -8 + 2 ** -30: 1 + 2 ** -7,  # just above the tie
        1 + 2 ** -8 - 2 ** -30: 1.0,          # just below the tie
        3.0 + 2 ** -7: 3.0,                  # tie at [2,4): spacing 2^-6
    }
    for v, want in cases.items():
        got = int(o.f64_to_bf16(np.array([v]))[0])
        assert got == exact_bits(want), (v, hex(got))
        if float(np.float32(v)) == v:
            got32 = int(o.f32_to_bf16(np.array([v], dtype=np.float32))[0])
            assert got32 == exact_bits(want), (v, hex(got32))


def pin_codec_special(o):
    cases = [
        (0.0, 0x0000), (-0.0, 0x8000),
        (2.0 ** -133, 0x0001),               # smallest subnormal
        (2.0 ** -134, 0x0000),               # tie with zero -> even (zero)
        (3 * 2.0 ** -134, 0x0002),           # tie between 1 and 2 quanta -> 2
        (2.0 ** -126, 0x0080),               # smallest normal
        ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F),  # largest finite
        ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80),  # tie with 2^128 -> even -> inf
        ((2 - 2 ** -8 - 2 ** -20) * 2.0 ** 127, 0x7F7F),
        (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
        (-2.0 ** -133, 0x8001),
    ]
    for v, want in cases:
        got = int(o.f64_to_bf16(np.array([v]))[0])
        assert got == want, (v, hex(got), hex(want))
    nan = int(o.f64_to_bf16(np.array([float("nan")]))[0])
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def pin_codec_vs_torch(o):
    rng = np.random.default_rng(1234)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    f = np.concatenate([f, rng.standard_normal(1 << 18).astype(np.float32)])
    got = o.f32_to_bf16(f)
    want = torch_bf16_bits(f)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(f[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def pin_decode_vs_torch(o):
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.bf16_to_f32(allbits)
    want = torch_bf16_value(allbits)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    assert (np.signbit(got) == np.signbit(want)).all()


# ------------------------------------------------------------- dispatch pins

def _random_routing(rng, T, k, E, p_missing=0.0):
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if p_missing:
        ids[rng.random(ids.shape) < p_missing] = -1
    return ids


def pin_counts_histogram(o):
    rng = np.random.default_rng(7)
    for (T, k, E, ep) in [(100, 4, 12, 3), (257, 8, 64, 8), (33, 2, 8, 4), (50, 3, 5, 5)]:
        epr = E // ep
        ids = _random_routing(rng, T, k, E, p_missing=0.1)
        x = random_bf16(rng, (T, 8))
        d = o.dispatch(x, ids, ep, epr, T * k)
        v = ids.reshape(-1)
        want = np.bincount(v[v >= 0] // epr, minlength=ep)
        assert (d.counts == want).all(), (d.counts, want)
        assert d.counts.sum() == (v >= 0).sum()
        assert d.status == 0


def pin_dispatch_layout(o):
    rng = np.random.default_rng(11)
    T, H, k, E, ep = 300, 24, 4, 12, 3
    epr = E // ep
    cap = 500
    ids = _random_routing(rng, T, k, E, p_missing=0.05)
    x = random_bf16(rng, (T, H))
    ws = np.full((ep, cap, H), CANARY, dtype=np.uint16)
    d = o.dispatch(x, ids, ep, epr, cap, ws=ws)
    flat_ids = ids.reshape(-1)
    for r in range(ep):
        n = int(d.counts[r])
        src = d.src_index[r, :n]
        # stable: increasing flat index; exactly the copies routed to r
        assert (np.diff(src) > 0).all()
        want = np.nonzero((flat_ids >= 0) & (flat_ids // epr == r))[0]
        assert np.array_equal(src, want)
        # inverse maps
        assert (d.slot_index.reshape(-1)[src] == r * cap + np.arange(n)).all()
        # payload rows are the source tokens
        assert np.array_equal(ws[r, :n], x[src // k])
        # padding untouched
        assert (ws[r, n:] == CANARY).all()
        assert (d.src_index[r, n:] == -1).all()
    s = d.slot_index.reshape(-1)
    assert ((s == -1) == (flat_ids == -1)).all()


def pin_full_routing_token_order(o):
    # Every token reaches every region (k = ep, one expert per region): row s
    # of each region must hold token s, the order the pages found the FlashInfer
    # kernel does NOT keep ("Verified: per-rank permutation") but which a
    # stable layout does.
    rng = np.random.default_rng(3)
    T, k, H = 4, 8, 8
    ids = np.stack([rng.permutation(8) for _ in range(T)]).astype(np.int32)
    x = np.stack([np.full(H, exact_bits(float(t)), dtype=np.uint16) for t in range(T)])
    d = o.dispatch(x, ids, 8, 1, T)
    assert (d.counts == T).all()
    for r in range(8):
        assert np.array_equal(d.src_index[r] // k, np.arange(T))
        assert np.array_equal(d.ws[r, :, 0], x[:, 0])


def pin_overflow(o):
    rng = np.random.default_rng(5)
    T, H, k, E, ep = 40, 8, 4, 8, 2
    epr = E // ep
    cap = 30                                    # each region gets ~80 copies
    ids = _random_routing(rng, T, k, E)
    x = random_bf16(rng, (T, H))
    ws = np.full((ep, cap, H), CANARY, dtype=np.uint16)
    d = o.dispatch(x, ids, ep, epr, cap, ws=ws)
    assert d.status & 1
    v = ids.reshape(-1)
    assert (d.counts == np.bincount(v // epr, minlength=ep)).all()    # not clamped
    s = d.slot_index.reshape(-1)
    for r in range(ep):
        mine = np.nonzero(v // epr == r)[0]
        assert (s[mine[:cap]] == r * cap + np.arange(cap)).all()
        assert (s[mine[cap:]] == -1).all()
        assert np.array_equal(ws[r], x[mine[:cap] // k])


def pin_bad_ids(o):
    T, H, k, E, ep = 3, 8, 2, 4, 2
    ids = np.array([[0, 3], [-1, 4], [-2, 1]], dtype=np.int32)
    x = np.arange(T * H, dtype=np.uint16).reshape(T, H) + 0x3F80
    d = o.dispatch(x, ids, ep, E // ep, 8)
    assert d.status == 2
    assert list(d.slot_index.reshape(-1)) == [0, 8, -1, -1, -1, 1]
    assert list(d.counts) == [2, 1]
    ok = o.dispatch(x, np.array([[0, 3], [-1, 2], [-1, -1]], dtype=np.int32), ep, E // ep, 8)
    assert ok.status == 0
    for bad in (-2, -1000, E, 1 << 30):          # each bad id alone is flagged
        d = o.dispatch(x, np.array([[0, 3], [bad, 2], [-1, -1]], dtype=np.int32), ep, E // ep, 8)
        assert d.status == 2, bad
        assert d.slot_index[1, 0] == -1


def pin_dispatch_brute(o):
    # exhaustive over every routing of 2 tokens x 2 copies with ids in -1..4
    # (4 is out of range for E = 4), for 1 and 2 regions and a tight capacity
    T, k, E, H = 2, 2, 4, 4
    rng = np.random.default_rng(0)
    x = random_bf16(rng, (T, H))
    for ep, cap in [(1, 4), (2, 2), (2, 1), (4, 1)]:
        epr = E // ep
        for combo in itertools.product(range(-1, 5), repeat=T * k):
            ids = np.array(combo, dtype=np.int32).reshape(T, k)
            d = o.dispatch(x, ids, ep, epr, cap)
            rows, counts, slot, src, status = brute.dispatch(x, ids, ep, epr, cap)
            assert d.status == status, combo
            assert list(d.counts) == counts, combo
            assert d.slot_index.tolist() == slot, combo
            for (r, s), f in src.items():
                assert d.src_index[r, s] == f, combo
                assert d.ws[r, s].tolist() == rows[(r, s)], combo


# -------------------------------------------------------------- combine pins

def pin_reduction_probe(o):
    g = read_golden("reduction_probe.txt")
    vals = [float(v) for v in g["contributions"][0]]
    ws, slot = one_token_case(vals)
    out = o.combine(ws, slot, None, False, ws.shape[-1])
    assert (out == exact_bits(float(g["fp32_then_narrow"][0][0]))).all(), hex(out[0, 0])
    assert (out != exact_bits(float(g["bf16_pairwise_tree"][0][0]))).all()
    assert (out != exact_bits(float(g["bf16_sequential"][0][0]))).all()


def pin_power_of_two(o):
    g = read_golden("power_of_two_probe.txt")
    vals = [float(v) for v in g["contributions"][0]]
    ws, slot = one_token_case(vals)
    out = o.combine(ws, slot, None, False, ws.shape[-1])
    assert (out == exact_bits(float(g["expected"][0][0]))).all(), hex(out[0, 0])
    # the same probe, weighted with unit gates, is the same reduction
    w = np.ones((1, len(vals)), dtype=np.float32)
    assert (o.combine(ws, slot, w, True, ws.shape[-1]) == out).all()


def pin_staged_sum_combine(o):
    g = read_golden("staged_sum.txt")
    vals = [0.0] * 8
    present = []
    for region, v in g["contribution"]:
        vals[int(region)] = float(v)
        present.append(int(region))
    missing = [r for r in range(8) if r not in present]
    ws, slot = one_token_case(vals, missing=missing)
    out = o.combine(ws, slot, None, False, ws.shape[-1])
    assert (out == exact_bits(float(g["expected"][0][0]))).all(), hex(out[0, 0])


def pin_identity_unweighted(o):
    rng = np.random.default_rng(2)
    for (T, H, k, E, ep) in [(64, 128, 2, 8, 4), (16, 64, 8, 64, 8), (10, 32, 3, 9, 3)]:
        epr = E // ep
        ids = _random_routing(rng, T, k, E)
        x = random_bf16(rng, (T, H))
        d = o.dispatch(x, ids, ep, epr, T * k)
        out = o.combine(d.ws, d.slot_index, None, False, H)
        want = torch_bf16_bits(torch_bf16_value(x) * np.float32(k))
        assert np.array_equal(out, want), (T, H, k)


def pin_identity_weighted(o):
    rng = np.random.default_rng(4)
    for (T, H, k, E, ep) in [(64, 128, 2, 8, 4), (16, 64, 8, 64, 8)]:
        epr = E // ep
        ids = _random_routing(rng, T, k, E)
        x = random_bf16(rng, (T, H))
        logits = rng.standard_normal((T, k))
        w = (np.exp(logits) / np.exp(logits).sum(1, keepdims=True)).astype(np.float32)
        d = o.dispatch(x, ids, ep, epr, T * k)
        out = o.combine(d.ws, d.slot_index, w, True, H)
        assert compare.ulp_distance(out, x).max() <= 1


def pin_weighted_closed_form(o):
    # decode-shaped expert stage: y = bf16(x * (1 + e/256)), gates from a
    # softmax; all terms share the sign of x, so the fp32 sum is within a few
    # fp32 ulps of the exact one and the narrowed result within 1 bf16 ulp.
    rng = np.random.default_rng(9)
    T, H, k, E, ep = 24, 256, 8, 256, 8
    epr = E // ep
    ids = _random_routing(rng, T, k, E)
    x = random_bf16(rng, (T, H))
    logits = rng.standard_normal((T, k))
    w = (np.exp(logits) / np.exp(logits).sum(1, keepdims=True)).astype(np.float32)
    d = o.dispatch(x, ids, ep, epr, T * k)
    scale = (1 + ids.astype(np.float32) / 256).astype(np.float32)       # [T, k]
    y_copy = torch_bf16_bits(torch_bf16_value(np.repeat(x, k, 0)) * scale.reshape(-1, 1))
    flat = d.ws.reshape(-1, H)
    s = d.slot_index.reshape(-1)
    flat[s] = y_copy
    out = o.combine(d.ws, d.slot_index, w, True, H)
    exact = (torch_bf16_value(y_copy).astype(np.float64).reshape(T, k, H)
             * w.astype(np.float64)[:, :, None]).sum(1)
    got = torch_bf16_value(out).astype(np.float64)
    spacing = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 2.0 ** -126))) - 7)
    assert (np.abs(got - exact) <= spacing).all()


def pin_combine_brute(o):
    rng = np.random.default_rng(21)
    for trial in range(6):
        T, H, k, E, ep = 3, 4, 3, 6, 3
        epr = E // ep
        ids = _random_routing(rng, T, k, E, p_missing=0.2)
        ids[0, 1] = ids[0, 0] if ids[0, 0] >= 0 else 2  # a duplicate id: two rows
        x = random_bf16(rng, (T, H))
        cap = T * k
        d = o.dispatch(x, ids, ep, epr, cap)
        # expert outputs with spread exponents, so rounding order matters
        y = random_bf16(rng, (T * k, H), scale=1.0)
        y = (y.astype(np.int32) + rng.integers(-6, 6, size=y.shape) * 128).astype(np.uint16)
        flat = d.ws.reshape(-1, H)
        s = d.slot_index.reshape(-1)
        flat[s[s >= 0]] = y[s >= 0]
        w = rng.random((T, k)).astype(np.float32)
        rows = {(r, q): list(d.ws[r, q]) for r in range(ep) for q in range(cap)}
        for weighted in (False, True):
            got = o.combine(d.ws, d.slot_index, w, weighted, H)
            want = brute.combine(rows, d.slot_index.tolist(), w.tolist(), weighted, T, H, cap)
            assert got.tolist() == want, (trial, weighted)


def pin_combine_cancellation(o):
    # gates near 1/8 over terms of both signs: fp32 fused multiply-adds in
    # j order, checked value by value against exact rationals
    rng = np.random.default_rng(33)
    T, H, k = 2, 64, 8
    ws = random_bf16(rng, (k, T, H), scale=0.25)
    slot = np.array([[j * T + t for j in range(k)] for t in range(T)], dtype=np.int32)
    w = (np.full((T, k), 0.125) + rng.standard_normal((T, k)) * 1e-3).astype(np.float32)
    got = o.combine(ws, slot, w, True, H)
    rows = {(j, t): list(ws[j, t]) for j in range(k) for t in range(T)}
    want = brute.combine(rows, slot.tolist(), w.tolist(), True, T, H, T)
    assert got.tolist() == want


def pin_detector(o):
    rng = np.random.default_rng(8)
    T, H, k, E, ep = 32, 64, 8, 64, 8
    ids = _random_routing(rng, T, k, E)
    x = random_bf16(rng, (T, H))
    d = o.dispatch(x, ids, ep, E // ep, T * k)
    once = o.combine(d.ws, d.slot_index, None, False, H)
    twice = torch_bf16_bits(torch_bf16_value(once) * 2)
    assert not compare.reduced_more_than_once(once, once)
    assert compare.reduced_more_than_once(twice, once)
    assert abs(np.median(compare.reduce_multiplicity(once, x)) - k) < 1e-6


# -------------------------------------------------------------- RMSNorm pins

def _fused_case(rng, T, H, k, weighted, res_scale=1.0):
    E, ep = 4 * k, k
    ids = _random_routing(rng, T, k, E)
    x = random_bf16(rng, (T, H))
    return ids, x, E, ep


def pin_rmsnorm_constant_row(o):
    H = 64
    for c, eps in [(1.0, 1e-6), (2.0 ** -10, 1e-6), (3.0, 0.5), (-0.75, 1e-6)]:
        ws, slot = one_token_case([c], H=H)
        res = np.zeros((1, H), dtype=np.uint16)
        gamma = torch_bf16_bits(np.linspace(0.5, 1.5, H).astype(np.float32))
        r_out, normed = o.combine_residual_rmsnorm(ws, slot, None, False, res, gamma, eps)
        assert (r_out == exact_bits(c)).all()
        e32 = float(np.float32(eps))
        g = torch_bf16_value(gamma).astype(np.float64)
        want = [brute.round_to_bf16_bits(Fraction(c / np.sqrt(c * c + e32) * gi)) for gi in g]
        assert normed[0].tolist() == want, (c, eps)


def pin_rmsnorm_textbook(o):
    rng = np.random.default_rng(12)
    T, H, k = 4, 256, 4
    ws = random_bf16(rng, (k, T, H))
    slot = np.array([[j * T + t for j in range(k)] for t in range(T)], dtype=np.int32)
    res = random_bf16(rng, (T, H))
    gamma = torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    eps = 1e-6
    r_out, normed, n64 = o.combine_residual_rmsnorm(ws, slot, None, False, res, gamma, eps,
                                                    want_f64=True)
    # the unweighted fp32 accumulator, j in order, then + residual, in numpy fp32
    acc = np.zeros((T, H), dtype=np.float32)
    for j in range(k):
        acc = (acc + torch_bf16_value(ws[j])).astype(np.float32)
    s = (acc + torch_bf16_value(res)).astype(np.float32)
    assert np.array_equal(r_out, torch_bf16_bits(s))
    s64 = s.astype(np.float64)
    ref = s64 / np.sqrt((s64 ** 2).mean(axis=1, keepdims=True) + np.float32(eps)) \
        * torch_bf16_value(gamma).astype(np.float64)
    assert np.allclose(n64, ref, rtol=1e-12, atol=0)
    assert compare.ulp_distance(normed, torch_bf16_bits(ref.astype(np.float32))).max() <= 1


def pin_rmsnorm_brute(o):
    rng = np.random.default_rng(14)
    T, H, k, cap = 2, 8, 3, 2
    ws = random_bf16(rng, (k, cap, H))
    slot = np.array([[0 * cap + 0, 1 * cap + 0, -1], [2 * cap + 1, 0 * cap + 1, 1 * cap + 1]],
                    dtype=np.int32)
    w = rng.random((T, k)).astype(np.float32)
    res = random_bf16(rng, (T, H))
    gamma = torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    rows = {(r, q): list(ws[r, q]) for r in range(k) for q in range(cap)}
    for weighted in (False, True):
        r_out, normed = o.combine_residual_rmsnorm(ws, slot, w, weighted, res, gamma, 1e-6)
        want_r, want_n = brute.combine_residual_rmsnorm(rows, slot.tolist(), w.tolist(), weighted,
                                                        res.tolist(), gamma.tolist(), 1e-6,
                                                        T, H, cap)
        assert r_out.tolist() == want_r
        assert normed.tolist() == want_n


def pin_rmsnorm_scale_invariance(o):
    # with eps = 0, doubling every input doubles s exactly and leaves the
    # normalised row bit-identical
    rng = np.random.default_rng(15)
    T, H, k = 3, 128, 2
    ws = random_bf16(rng, (k, T, H))
    slot = np.array([[j * T + t for j in range(k)] for t in range(T)], dtype=np.int32)
    res = random_bf16(rng, (T, H))
    gamma = torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    r1, n1 = o.combine_residual_rmsnorm(ws, slot, None, False, res, gamma, 0.0)
    ws2 = torch_bf16_bits(torch_bf16_value(ws) * 2)
    res2 = torch_bf16_bits(torch_bf16_value(res) * 2)
    r2, n2 = o.combine_residual_rmsnorm(ws2, slot, None, False, res2, gamma, 0.0)
    assert np.array_equal(n1, n2)
    assert np.array_equal(torch_bf16_bits(torch_bf16_value(r1) * 2), r2)


# ------------------------------------- reduction of tensor-parallel partials
# magik.net "Fusing the Allreduce: A Precision Investigation into FlashInfer's
# Verify-Path Optimization", section "The Message Itself: Explanation and
# Probe": the all-reduce of the hidden states and the residual add + RMSNorm
# that follows become one kernel.  On one GPU the P partials [P, T, H] are
# local and their sum is one reduction, the same "fp32, one narrowing" sum as
# the combine; the pages' reduction probes apply to it unchanged (each
# partial standing for one contribution).

def _partials_rows(partials):
    """The partials as the brute force's rows: partial p of token t is row
    (p, t) of a workspace with cap = T."""
    P, T, _ = partials.shape
    rows = {(p, t): list(partials[p, t]) for p in range(P) for t in range(T)}
    slot = [[p * T + t for p in range(P)] for t in range(T)]
    return rows, slot


def pin_partials_power_of_two(o):
    g = read_golden("power_of_two_probe.txt")
    vals = [float(v) for v in g["contributions"][0]]
    T, H = 3, 16
    partials = np.stack([np.full((T, H), exact_bits(v), np.uint16) for v in vals])
    want = exact_bits(float(g["expected"][0][0]))
    assert (o.partials_reduce(partials) == want).all()
    res = np.zeros((T, H), np.uint16)
    gamma = np.full(H, exact_bits(1.0), np.uint16)
    r_out, _ = o.partials_reduce_residual_rmsnorm(partials, res, gamma, 1e-6)
    assert (r_out == want).all()


def pin_partials_reduction_probe(o):
    g = read_golden("reduction_probe.txt")
    vals = [float(v) for v in g["contributions"][0]]
    partials = np.stack([np.full((1, 8), exact_bits(v), np.uint16) for v in vals])
    out = o.partials_reduce(partials)
    assert (out == exact_bits(float(g["fp32_then_narrow"][0][0]))).all(), hex(out[0, 0])
    assert (out != exact_bits(float(g["bf16_pairwise_tree"][0][0]))).all()
    assert (out != exact_bits(float(g["bf16_sequential"][0][0]))).all()


def pin_partials_closed_forms(o):
    rng = np.random.default_rng(21)
    T, H = 5, 64
    x = random_bf16(rng, (T, H))
    # one partial: the all-reduce of one rank is its own value
    assert np.array_equal(o.partials_reduce(x[None]), x)
    # P identical partials, P a power of two: exactly P * x
    for P in (2, 4, 8):
        want = torch_bf16_bits(torch_bf16_value(x) * np.float32(P))
        assert np.array_equal(o.partials_reduce(np.stack([x] * P)), want), P
    # a partial and its negation cancel exactly; the others survive
    y = random_bf16(rng, (T, H))
    neg = x ^ np.uint16(0x8000)
    assert np.array_equal(o.partials_reduce(np.stack([x, y, neg])), y)


def pin_partials_textbook(o):
    # numpy fp32, partials added in rank order, torch's nearest-even narrowing;
    # then the textbook fp64 RMSNorm of (sum + residual)
    rng = np.random.default_rng(22)
    P, T, H = 6, 4, 256
    partials = random_bf16(rng, (P, T, H))
    acc = np.zeros((T, H), dtype=np.float32)
    for p in range(P):
        acc = (acc + torch_bf16_value(partials[p])).astype(np.float32)
    assert np.array_equal(o.partials_reduce(partials), torch_bf16_bits(acc))
    res = random_bf16(rng, (T, H))
    gamma = torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    eps = 1e-6
    r_out, normed, n64 = o.partials_reduce_residual_rmsnorm(partials, res, gamma, eps,
                                                            want_f64=True)
    s = (acc + torch_bf16_value(res)).astype(np.float32)
    assert np.array_equal(r_out, torch_bf16_bits(s))
    s64 = s.astype(np.float64)
    ref = s64 / np.sqrt((s64 ** 2).mean(axis=1, keepdims=True) + np.float32(eps)) \
        * torch_bf16_value(gamma).astype(np.float64)
    assert np.allclose(n64, ref, rtol=1e-12, atol=0)
    assert compare.ulp_distance(normed, torch_bf16_bits(ref.astype(np.float32))).max() <= 1


def pin_partials_brute(o):
    rng = np.random.default_rng(23)
    P, T, H = 3, 2, 8
    partials = random_bf16(rng, (P, T, H))
    rows, slot = _partials_rows(partials)
    assert o.partials_reduce(partials).tolist() == brute.combine(rows, slot, None, False, T, H, T)
    res = random_bf16(rng, (T, H))
    gamma = torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    r_out, normed = o.partials_reduce_residual_rmsnorm(partials, res, gamma, 1e-6)
    want_r, want_n = brute.combine_residual_rmsnorm(rows, slot, None, False, res.tolist(),
                                                    gamma.tolist(), 1e-6, T, H, T)
    assert r_out.tolist() == want_r
    assert normed.tolist() == want_n


# --------------------------------------------------- per-region layout pins
# The FlashInfer form the pages measure: one row per (token, region), the
# region's experts return one message per token, the combine adds each
# region's message once.  InferenceX PR #2450 prints the probes used here:
# "Synthesis" (duplicate experts on one rank read once -> 1.0; partial routing
# to two destinations -> 2.0; 2^rank over 8 ranks -> 255), "The oracle was
# never wrong" (seven staged per-rank messages -> 0.255859375) and "Bring-up
# progress" (about 5.3 distinct ranks per token for top-8 over 8 ranks).

def _region_combine_of(o, ids, ep, messages, H=8):
    """Per-region dispatch of ids (expert = region, epr = 1) with region r's
    rows holding messages[r], then the per-region combine."""
    x = np.zeros((ids.shape[0], H), np.uint16)
    d = o.dispatch(x, ids, ep, 1, ids.shape[0], layout="region")
    flat = d.ws.reshape(-1, H)
    for r in range(ep):
        for s in range(int(d.counts[r])):
            flat[r * ids.shape[0] + s] = printed_bits(messages[r])
    return d, o.combine(d.ws, d.slot_index, None, False, H, layout="region")


def pin_region_duplicates_read_once(o):
    ids = np.array([[0, 0]], np.int32)               # both experts on region 0
    d, out = _region_combine_of(o, ids, 1, [1.0])
    assert list(d.counts) == [1]
    assert d.slot_index[0, 0] == d.slot_index[0, 1] == 0
    assert (out == exact_bits(1.0)).all()            # read once, not 2.0


def pin_region_partial_routing(o):
    ids = np.array([[0, 1, 0, 1], [1, 1, 0, 0], [0, 0, 0, 1], [1, 0, 1, 1]], np.int32)
    d, out = _region_combine_of(o, ids, 2, [1.0, 1.0])
    assert list(d.counts) == [4, 4]
    assert (out == exact_bits(2.0)).all()


def pin_region_power_of_two(o):
    g = read_golden("power_of_two_probe.txt")
    msgs = [float(v) for v in g["contributions"][0]]
    ids = np.array([[3, 0, 1, 2, 4, 5, 7, 6, 0, 3]], np.int32)   # 8 regions, 2 duplicates
    d, out = _region_combine_of(o, ids, 8, msgs)
    assert (out == exact_bits(float(g["expected"][0][0]))).all(), hex(out[0, 0])


def pin_region_staged_sum(o):
    g = read_golden("staged_sum.txt")
    msgs = [0.0] * 8
    for r, v in g["contribution"]:
        msgs[int(r)] = float(v)
    ids = np.array([[0, 1, 2, 4, 5, 6, 7, 0]], np.int32)   # region 3 hosts none; 0 hosts two
    d, out = _region_combine_of(o, ids, 8, msgs)
    assert d.counts[3] == 0 and d.counts.sum() == 7
    assert (out == exact_bits(float(g["expected"][0][0]))).all(), hex(out[0, 0])


def pin_region_counts_distinct(o):
    rng = np.random.default_rng(17)
    for (T, k, E, ep) in [(200, 8, 64, 8), (97, 4, 12, 3), (50, 6, 6, 6), (33, 3, 20, 1)]:
        epr = E // ep
        ids = _random_routing(rng, T, k, E, p_missing=0.1)
        d = o.dispatch(random_bf16(rng, (T, 8)), ids, ep, epr, T, layout="region")
        reg = np.where(ids >= 0, ids // epr, -1)
        want = [int((reg == r).any(axis=1).sum()) for r in range(ep)]
        assert list(d.counts) == want, (d.counts, want)
        assert d.status == 0


def pin_region_layout(o):
    rng = np.random.default_rng(19)
    T, H, k, E, ep = 150, 16, 6, 24, 4
    epr = E // ep
    ids = _random_routing(rng, T, k, E, p_missing=0.05)
    x = random_bf16(rng, (T, H))
    ws = np.full((ep, T, H), CANARY, dtype=np.uint16)
    d = o.dispatch(x, ids, ep, epr, T, ws=ws, layout="region")
    reg = np.where(ids >= 0, ids // epr, -1)
    for r in range(ep):
        n = int(d.counts[r])
        src = d.src_index[r, :n]
        assert (np.diff(src) > 0).all()
        toks = src // k
        assert np.array_equal(toks, np.nonzero((reg == r).any(axis=1))[0])
        # the row's copy is the token's first copy to r
        assert all(reg[t, :f % k].tolist().count(r) == 0 and reg[t, f % k] == r
                   for t, f in zip(toks, src))
        assert np.array_equal(ws[r, :n], x[toks])
        assert (ws[r, n:] == CANARY).all()
    for t in range(T):                         # copies to one region share its row
        for j in range(k):
            if reg[t, j] < 0:
                assert d.slot_index[t, j] == -1
            else:
                row = d.slot_index[t, j]
                assert row // T == reg[t, j] and d.src_index.reshape(-1)[row] // k == t


def pin_region_full_routing_token_order(o):
    rng = np.random.default_rng(23)
    T, k = 5, 8
    ids = np.stack([rng.permutation(8) for _ in range(T)]).astype(np.int32)
    x = np.stack([np.full(8, exact_bits(float(t)), np.uint16) for t in range(T)])
    d = o.dispatch(x, ids, 8, 1, T, layout="region")
    assert (d.counts == T).all()
    for r in range(8):
        assert np.array_equal(d.src_index[r] // k, np.arange(T))


def pin_region_matches_copy_combine_without_duplicates(o):
    # skipping a duplicate row is the same as that copy being unrouted: the
    # per-region combine equals the (pinned) per-copy combine and fused
    # epilogue on a slot map whose duplicates are set to -1
    rng = np.random.default_rng(29)
    T, H, k, E, ep = 40, 64, 6, 12, 4
    ids = _random_routing(rng, T, k, E, p_missing=0.1)
    d = o.dispatch(random_bf16(rng, (T, H)), ids, ep, E // ep, T, layout="region")
    d.ws[...] = random_bf16(rng, d.ws.shape)
    masked = d.slot_index.copy()
    for t in range(T):
        for j in range(k):
            if masked[t, j] >= 0 and masked[t, j] in d.slot_index[t, :j]:
                masked[t, j] = -1
    assert (masked != d.slot_index).any()
    got = o.combine(d.ws, d.slot_index, None, False, H, layout="region")
    assert np.array_equal(got, o.combine(d.ws, masked, None, False, H))
    res = random_bf16(rng, (T, H))
    gamma = torch_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    a = o.combine_residual_rmsnorm(d.ws, d.slot_index, None, False, res, gamma, 1e-6,
                                   layout="region")
    b = o.combine_residual_rmsnorm(d.ws, masked, None, False, res, gamma, 1e-6)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def pin_region_brute(o):
    # every routing of one token x 3 copies with ids in -1..4 (4 out of range),
    # and a seeded sample of two-token routings, over four layouts
    k, E, H = 3, 4, 3
    rng = np.random.default_rng(31)
    y = random_bf16(rng, (8 * 4, H))
    combos = [c for c in itertools.product(range(-1, 5), repeat=k)]
    combos += [tuple(rng.integers(-1, 5, size=2 * k)) for _ in range(150)]
    for ep, cap in [(2, 2), (2, 1), (4, 1), (1, 2)]:
        epr = E // ep
        for combo in combos:
            T = len(combo) // k
            x = random_bf16(np.random.default_rng(T), (T, H))
            ids = np.array(combo, dtype=np.int32).reshape(T, k)
            d = o.dispatch(x, ids, ep, epr, cap, layout="region")
            rows, counts, slot, src, status = brute.dispatch_region(x, ids, ep, epr, cap)
            assert (d.status, list(d.counts), d.slot_index.tolist()) == (status, counts, slot), combo
            for (r, s_), f in src.items():
                assert d.src_index[r, s_] == f and d.ws[r, s_].tolist() == rows[(r, s_)], combo
            d.ws[...] = y[: ep * cap].reshape(d.ws.shape)
            yr = {(r, s_): list(d.ws[r, s_]) for r in range(ep) for s_ in range(cap)}
            got = o.combine(d.ws, d.slot_index, None, False, H, layout="region")
            assert got.tolist() == brute.combine_region(yr, d.slot_index.tolist(), T, H, cap), combo


def pin_region_distinct_closed_form(o):
    g = read_golden("routing_statistics.txt")
    E, k, ep = int(g["E"][0][0]), int(g["k"][0][0]), int(g["ep"][0][0])
    rng = np.random.default_rng(0)
    T = 4096
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    d = o.dispatch(np.zeros((T, 1), np.uint16), ids, ep, E // ep, T, layout="region")
    per_token = d.counts.sum() / T
    assert abs(per_token - float(g["distinct_regions_closed_form"][0][0])) < 0.03, per_token


# ---------------------------------------------------------------- FP8 pins
# The FP8 payload: OCP E4M3 codes (torch.float8_e4m3fn is an independent
# implementation of the same format) and one fp32 scale per row.

def torch_e4m3_bits(a) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_decode_vs_torch(o):
    codes = np.arange(256, dtype=np.uint8)
    got = o.e4m3_to_f32(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert ((got == want) | (np.isnan(got) & np.isnan(want))).all()
    assert (np.signbit(got) == np.signbit(want)).all()


def pin_e4m3_encode_vs_torch(o):
    rng = np.random.default_rng(41)
    v = np.concatenate([rng.standard_normal(1 << 16) * 100, rng.standard_normal(1 << 16) * 0.02,
                        rng.uniform(-463.9, 463.9, 1 << 14)]).astype(np.float32)
    assert np.array_equal(o.f32_to_e4m3(v), torch_e4m3_bits(v))


def pin_e4m3_special(o):
    cases = [(448.0, 0x7E), (464.0, 0x7E), (465.0, 0x7F), (1e6, 0x7F), (-448.0, 0xFE),
             (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (2.0 ** -6, 0x08),
             (7 * 2.0 ** -9, 0x07), (15 * 2.0 ** -10, 0x08), (1.0, 0x38), (1.0625, 0x38),
             (1.1875, 0x3A), (-0.0, 0x80), (0.0, 0x00), (2.0 ** -11, 0x00)]
    for v, want in cases:
        got = int(o.f32_to_e4m3(np.array([v], np.float32))[0])
        assert got == want, (v, hex(got), hex(want))
    assert int(o.f32_to_e4m3(np.array([np.nan], np.float32))[0]) & 0x7F == 0x7F


def pin_fp8_row_quantisation(o):
    rng = np.random.default_rng(43)
    T, H = 24, 200
    xf = (rng.standard_normal((T, H)) * np.exp(rng.uniform(-8, 8, (T, 1)))).astype(np.float32)
    xf[5] = 0.0                                           # an all-zero row
    xf[6, :] = 0.0
    xf[6, 17] = -3.0                                      # one non-zero element
    x = torch_bf16_bits(xf)
    q, scale = o.quantize_e4m3_rows(x)
    xv = torch_bf16_value(x)
    amax = np.abs(xv).max(axis=1)
    assert np.array_equal(scale, (amax / np.float32(448)).astype(np.float32))
    inv = np.where(amax > 0, np.float32(448) / np.where(amax > 0, amax, 1), 0).astype(np.float32)
    assert np.array_equal(q, torch_e4m3_bits((xv * inv[:, None]).astype(np.float32)))
    assert (q[5] == 0).all() and scale[5] == 0
    assert q[6, 17] == 0xFE and (np.delete(q[6], 17) == 0).all()
    for t in range(T):                                    # the row maximum maps to +-448
        if amax[t] > 0:
            assert (np.abs(o.e4m3_to_f32(q[t])) == 448).any()
    # round trip: within half a step of the 3-bit significand, or half the
    # subnormal step (2^-10 in scaled units) near zero
    back = o.e4m3_to_f32(q).astype(np.float64) * scale[:, None]
    bound = np.maximum(np.abs(xv) * 2.0 ** -4, scale[:, None] * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(back - xv) <= bound).all()


def pin_fp8_dispatch_places_rows_and_scales(o):
    rng = np.random.default_rng(47)
    T, H, k, E, ep = 60, 32, 4, 16, 4
    ids = _random_routing(rng, T, k, E, p_missing=0.1)
    x = random_bf16(rng, (T, H))
    q, scale = o.quantize_e4m3_rows(x)
    for layout in ("copy", "region"):
        d, scales = o.dispatch_fp8(x, ids, ep, E // ep, T * k, layout=layout)
        for r in range(ep):
            n = int(d.counts[r])
            toks = d.src_index[r, :n] // k
            assert np.array_equal(d.ws[r, :n], q[toks])
            assert np.array_equal(scales[r, :n], scale[toks])


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
