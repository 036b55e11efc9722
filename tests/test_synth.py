"""The seeded workload generators: shapes, determinism and routing statistics."""
import dataclasses
from math import comb

import numpy as np
import pytest

import pins
import synth


@pytest.mark.parametrize("wl", [synth.TINY, synth.DECODE,
                                dataclasses.replace(synth.FUSED, T=32, H=512)],
                         ids=lambda w: w.name)
def test_inputs_shape_and_determinism(wl):
    a = synth.make_inputs(wl, 0)
    b = synth.make_inputs(wl, 0)
    c = synth.make_inputs(wl, 1)
    assert a.x.shape == (wl.T, wl.H) and a.x.dtype == np.uint16
    assert a.ids.shape == (wl.T, wl.k) and a.ids.dtype == np.int32
    assert a.weights.shape == (wl.T, wl.k) and a.weights.dtype == np.float32
    assert np.array_equal(a.x, b.x) and np.array_equal(a.ids, b.ids)
    assert np.array_equal(a.weights, b.weights)
    assert not np.array_equal(a.ids, c.ids)
    # k distinct experts per token, all in range
    assert ((a.ids >= 0) & (a.ids < wl.E)).all()
    assert all(len(set(row)) == wl.k for row in a.ids.tolist())
    assert np.allclose(a.weights.sum(1), 1.0, atol=1e-6) and (a.weights > 0).all()
    if wl.combine == "fused":
        assert a.residual.shape == (wl.T, wl.H) and a.gamma.shape == (wl.H,)
        g = pins.torch_bf16_value(a.gamma)
        assert (g >= 0.5).all() and (g <= 1.5).all()


def test_uniform_routing_reaches_the_pages_distinct_region_count():
    # mean number of distinct regions a token reaches under uniform top-8 of
    # 256 experts over 8 regions: the closed form, the value the page derives
    # from its receive counts, and the generator all agree
    g = pins.read_golden("routing_statistics.txt")
    E, k, ep = int(g["E"][0][0]), int(g["k"][0][0]), int(g["ep"][0][0])
    epr = E // ep
    closed = ep * (1 - comb(E - epr, k) / comb(E, k))
    assert abs(closed - float(g["distinct_regions_closed_form"][0][0])) < 1e-4
    page = float(g["run5_recv"][0][0]) / (int(g["run5_T"][0][0]) * int(g["run5_source_ranks"][0][0]))
    assert abs(page - closed) < 0.01
    rng = np.random.default_rng(0)
    ids = synth.draw_routing(rng, 8192, E, k, "uniform")
    distinct = np.array([len(set(r)) for r in (ids // epr).tolist()])
    assert abs(distinct.mean() - closed) < 0.02


def test_zipf_routing_is_skewed_toward_low_expert_ids():
    rng = np.random.default_rng(0)
    ids = synth.draw_routing(rng, 8192, 256, 8, "zipf1.2")
    assert all(len(set(r)) == 8 for r in ids.tolist())
    freq = np.bincount(ids.reshape(-1), minlength=256)
    assert freq[0] > 0.8 * 8192                 # the hottest expert: most tokens
    assert freq[0] > freq[8] > freq[64] > freq[255]
    region0 = (ids // 16 == 0).mean()           # 16 regions of 16 experts
    assert 0.5 < region0 < 0.7


def test_expert_stage_rows_are_per_copy():
    wl = synth.DECODE
    inp = synth.make_inputs(wl, 0)
    y = synth.expert_outputs(wl, inp)
    assert y.shape == (wl.T * wl.k, wl.H)
    t, j = 5, 3
    e = int(inp.ids[t, j])
    want = pins.torch_bf16_bits(pins.torch_bf16_value(inp.x[t]) * np.float32(1 + e / 256))
    assert np.array_equal(y[t * wl.k + j], want)
    ident = synth.expert_outputs(synth.TINY, synth.make_inputs(synth.TINY, 0))
    assert np.array_equal(ident[::2], synth.make_inputs(synth.TINY, 0).x)
