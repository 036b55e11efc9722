"""Seeded synthetic inputs for the five workloads.

This module only draws random numbers and shapes them; it holds none of the
dispatch / combine / normalisation arithmetic.  The same bytes feed the CPU
oracle and the HIP library.

Recipe (numpy ``default_rng(seed)``, draws taken in this order):

1. ``x``        : fp32 N(0,1) of shape [T, H], rounded to bf16 (nearest-even).
2. routing keys : uniform  -> U(0,1) keys [T, E]; the k smallest keys give a
                  token's k distinct experts, in key order.
                  zipf1.2  -> popularity p_e proportional to (e+1)^-1.2, expert
                  0 the hottest; Gumbel(0,1) noise [T, E] is added to log p_e
                  and the k largest keys are taken (Gumbel-top-k, which draws k
                  experts without replacement in proportion to p).
3. ``weights``  : softmax (computed in fp64, stored fp32) over k i.i.d. N(0,1)
                  logits per token.
4. fused workload only: ``residual`` N(0,1) [T, H] bf16, ``gamma`` U(0.5,1.5)
   [H] bf16, then the Gaussian expert outputs N(0,1) [T*k, H] bf16.

Synthetic expert stages (per routed copy f = t*k + j, expert e = ids[t, j]):

  identity                      y_f = x_t
  scale_by_expert               y_f = bf16( fp32(x_t) * (1 + e/256) )
                                (the fp32 product is exact: 8 x 9 bits)
  scale_by_expert_times_weight  y_f = bf16( fp32( fp32(x_t)*(1 + e/256) ) * w_f )
                                (the gate applied by the expert side, so the
                                combine itself runs unweighted)
  gaussian                      y_f ~ N(0,1) i.i.d., bf16

Partials workload (``make_partials``, its own ``default_rng(seed)``):
``partials`` N(0,1) [P, T, H] bf16, ``residual`` N(0,1) [T, H] bf16,
``gamma`` U(0.5,1.5) [H] bf16, drawn in that order.

All bf16 values are carried as ``uint16`` bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import PartialsWorkload, Workload


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, nearest-even, using torch's conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values, using torch's conversion."""
    t = torch.from_numpy(np.ascontiguousarray(u, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float32).numpy()


@dataclass
class Inputs:
    x: np.ndarray                     # uint16 [T, H]
    ids: np.ndarray                   # int32  [T, k]
    weights: np.ndarray               # fp32   [T, k]
    residual: Optional[np.ndarray] = None   # uint16 [T, H]
    gamma: Optional[np.ndarray] = None      # uint16 [H]
    gaussian_y: Optional[np.ndarray] = None  # uint16 [T*k, H]


def draw_routing(rng: np.random.Generator, T: int, E: int, k: int, routing: str) -> np.ndarray:
    if routing == "uniform":
        keys = rng.random((T, E))
        ids = np.argsort(keys, axis=1, kind="stable")[:, :k]
    elif routing == "zipf1.2":
        logp = -1.2 * np.log(np.arange(1, E + 1, dtype=np.float64))
        keys = logp[None, :] + rng.gumbel(size=(T, E))
        ids = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    else:
        raise ValueError(f"unknown routing {routing!r}")
    return np.ascontiguousarray(ids, dtype=np.int32)


def draw_softmax_weights(rng: np.random.Generator, T: int, k: int) -> np.ndarray:
    logits = rng.standard_normal((T, k))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return np.ascontiguousarray(z / z.sum(axis=1, keepdims=True), dtype=np.float32)


def make_inputs(wl: Workload, seed: int = 0) -> Inputs:
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal((wl.T, wl.H), dtype=np.float32))
    ids = draw_routing(rng, wl.T, wl.E, wl.k, wl.routing)
    w = draw_softmax_weights(rng, wl.T, wl.k)
    inp = Inputs(x=x, ids=ids, weights=w)
    if wl.combine == "fused":
        inp.residual = f32_to_bf16_bits(rng.standard_normal((wl.T, wl.H), dtype=np.float32))
        inp.gamma = f32_to_bf16_bits(rng.uniform(0.5, 1.5, size=wl.H).astype(np.float32))
    if wl.expert == "gaussian":
        inp.gaussian_y = f32_to_bf16_bits(
            rng.standard_normal((wl.T * wl.k, wl.H), dtype=np.float32))
    return inp


def expert_outputs(wl: Workload, inp: Inputs) -> np.ndarray:
    """The synthetic expert output of every routed copy, uint16 [T*k, H].

    Row f = t*k + j belongs to token t's j-th expert.  The rows are defined per
    copy, not per slot, so any dispatch layout can place them.
    """
    T, k = inp.ids.shape
    if wl.expert == "gaussian":
        return inp.gaussian_y
    xr = np.repeat(inp.x, k, axis=0)                       # [T*k, H]
    if wl.expert == "identity":
        return xr
    scale = (1.0 + inp.ids.reshape(-1).astype(np.float32) / np.float32(256.0)).astype(np.float32)
    y = bf16_bits_to_f32(xr) * scale[:, None]               # exact in fp32
    if wl.expert == "scale_by_expert":
        return f32_to_bf16_bits(y)
    if wl.expert == "scale_by_expert_times_weight":
        y = (y * inp.weights.reshape(-1)[:, None]).astype(np.float32)
        return f32_to_bf16_bits(y)
    raise ValueError(f"unknown expert stage {wl.expert!r}")


def region_messages(ids: np.ndarray, weights: np.ndarray, y_rows: np.ndarray, epr: int,
                    gated: bool = True) -> np.ndarray:
    """The expert side's message under the per-region layout, uint16 [T*k, H].

    Region r's experts return, for token t, one row: the sum of the token's
    copies local to r, each gated (w_j * y_j, fp32 product) when ``gated``,
    accumulated in fp32 in j order and rounded to bf16 once.  The message sits
    at the flat index of the token's first copy to r; other rows are zero.
    """
    T, k = ids.shape
    H = y_rows.shape[1]
    region = np.where(ids >= 0, ids // epr, -1)
    y = bf16_bits_to_f32(y_rows).reshape(T, k, H)
    w = weights.astype(np.float32) if gated else np.ones((T, k), np.float32)
    out = np.zeros((T, k, H), dtype=np.uint16)
    for j in range(k):
        first = region[:, j] >= 0
        for i in range(j):
            first &= region[:, i] != region[:, j]
        if not first.any():
            continue
        acc = np.zeros((int(first.sum()), H), dtype=np.float32)
        for i in range(j, k):
            same = (region[first, i] == region[first, j])[:, None]
            term = (y[first, i] * w[first, i][:, None]).astype(np.float32)
            acc = np.where(same, (acc + term).astype(np.float32), acc)
        out[first, j] = f32_to_bf16_bits(acc)
    return out.reshape(T * k, H)


def make_partials(pw: PartialsWorkload, seed: int = 0):
    """(partials [P, T, H], residual [T, H], gamma [H]) as bf16 patterns."""
    rng = np.random.default_rng(seed)
    partials = np.empty((pw.P, pw.T, pw.H), dtype=np.uint16)
    for p in range(pw.P):
        partials[p] = f32_to_bf16_bits(rng.standard_normal((pw.T, pw.H), dtype=np.float32))
    residual = f32_to_bf16_bits(rng.standard_normal((pw.T, pw.H), dtype=np.float32))
    gamma = f32_to_bf16_bits(rng.uniform(0.5, 1.5, size=pw.H).astype(np.float32))
    return partials, residual, gamma
