"""Pure-Python brute force of dispatch, combine and the fused epilogue.

TEST INFRASTRUCTURE ONLY, for tiny inputs.  Every number is an exact
rational (``fractions.Fraction``); each rounding the method performs is done
by one generic round-to-nearest-even routine written from the definition of a
binary floating-point format.  It shares no code with ``moe_oracle.c`` and
exists to catch coding mistakes there: a dropped term, a wrong index, a
mis-rounded tie.  The square root of the RMSNorm is taken with 60 decimal
digits, well beyond what any bf16 rounding can see.
"""
from __future__ import annotations

import decimal
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

import numpy as np

# (significand bits incl. the leading one, minimum normal exponent, maximum exponent)
FP32 = (24, -126, 127)
BF16 = (8, -126, 127)

INF = float("inf")


def round_binary(q: Fraction, fmt=FP32):
    """Nearest value of a binary format to the rational q, ties to even.

    Returns a Fraction, or +-inf when the rounded magnitude reaches 2^(emax+1).
    """
    p, emin, emax = fmt
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)                         # below 2^emin: fixed (subnormal) spacing
    quantum = Fraction(2) ** (e - p + 1)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** (emax + 1):
        return sign * INF
    return sign * r


def bf16_value(bits: int) -> Fraction:
    """Exact value of a bf16 bit pattern (finite patterns only)."""
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    assert exp != 0xFF, "non-finite pattern"
    if exp == 0:
        return sign * Fraction(frac, 128) * Fraction(2) ** -126
    return sign * (1 + Fraction(frac, 128)) * Fraction(2) ** (exp - 127)


def bf16_bits(v) -> int:
    """Bit pattern of a value that is exactly a bf16 number (or +-inf)."""
    if v == INF:
        return 0x7F80
    if v == -INF:
        return 0xFF80
    v = Fraction(v)
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    for exp in range(1, 255):
        scale = Fraction(2) ** (exp - 127)
        m = a / scale                         # in [1, 2) for the right exponent
        if 1 <= m < 2:
            frac = (m - 1) * 128
            assert frac.denominator == 1, "not a bf16 value"
            return sign | (exp << 7) | int(frac)
    frac = a / Fraction(2) ** -126 * 128     # subnormal
    assert frac.denominator == 1 and frac < 128, "not a bf16 value"
    return sign | int(frac)


def round_to_bf16_bits(q: Fraction) -> int:
    return bf16_bits(round_binary(q, BF16))


def dispatch(x_bits: np.ndarray, ids: np.ndarray, ep: int, epr: int, cap: int):
    """Returns (rows, counts, slot_index, src_index, status).

    rows maps (r, s) -> list of H bf16 patterns; src_index maps (r, s) -> f.
    Copies go to region e // epr in increasing f; -1 means no expert; other
    out-of-range ids set bit 2 of status; a full region sets bit 1.
    """
    T, H = x_bits.shape
    k = ids.shape[1]
    E = ep * epr
    regions: List[List[int]] = [[] for _ in range(ep)]
    slot_index = [[-1] * k for _ in range(T)]
    status = 0
    for t in range(T):
        for j in range(k):
            e = int(ids[t][j])
            if e == -1:
                continue
            if not (0 <= e < E):
                status |= 2
                continue
            r = e // epr
            f = t * k + j
            s = len(regions[r])
            regions[r].append(f)
            if s >= cap:
                status |= 1
                continue
            slot_index[t][j] = r * cap + s
    counts = [len(g) for g in regions]
    src_index = {}
    rows = {}
    for r in range(ep):
        for s, f in enumerate(regions[r][:cap]):
            src_index[(r, s)] = f
            rows[(r, s)] = [int(v) for v in x_bits[f // k]]
    return rows, counts, slot_index, src_index, status


def _accumulate(y_rows, slot_index, weights, weighted, t, h, cap) -> Fraction:
    """fp32 accumulator over j = 0..k-1; each step rounds once (fma semantics)."""
    acc = Fraction(0)
    for j, row in enumerate(slot_index[t]):
        if row < 0:
            continue
        v = bf16_value(int(y_rows[(row // cap, row % cap)][h]))
        c = Fraction(float(np.float32(weights[t][j]))) if weighted else Fraction(1)
        acc = round_binary(acc + c * v, FP32)
    return acc


def combine(y_rows, slot_index, weights, weighted: bool, T: int, H: int, cap: int) -> List[List[int]]:
    """out[t][h] as bf16 patterns: the fp32 sum narrowed once, nearest-even."""
    return [[round_to_bf16_bits(_accumulate(y_rows, slot_index, weights, weighted, t, h, cap))
             for h in range(H)] for t in range(T)]


def combine_residual_rmsnorm(y_rows, slot_index, weights, weighted: bool, residual_bits,
                             gamma_bits, eps: float, T: int, H: int, cap: int
                             ) -> Tuple[List[List[int]], List[List[int]]]:
    """(residual_out, normed) as bf16 patterns."""
    ctx = decimal.Context(prec=60)
    res_out, normed = [], []
    for t in range(T):
        s = [round_binary(_accumulate(y_rows, slot_index, weights, weighted, t, h, cap)
                          + bf16_value(int(residual_bits[t][h])), FP32) for h in range(H)]
        ms = sum(v * v for v in s) / H + Fraction(float(np.float32(eps)))
        root = ctx.sqrt(ctx.divide(decimal.Decimal(ms.numerator), decimal.Decimal(ms.denominator)))
        inv = Fraction(ctx.divide(decimal.Decimal(1), root))
        res_out.append([round_to_bf16_bits(v) for v in s])
        normed.append([round_to_bf16_bits(v * inv * bf16_value(int(gamma_bits[h])))
                       for h, v in enumerate(s)])
    return res_out, normed


def dispatch_region(x_bits: np.ndarray, ids: np.ndarray, ep: int, epr: int, cap: int):
    """Per-region layout: one row per (token, region) for the token's first
    copy to that region; later copies to the same region share its row.
    Returns (rows, counts, slot_index, src_index, status) like ``dispatch``."""
    T, H = x_bits.shape
    k = ids.shape[1]
    E = ep * epr
    regions: List[List[int]] = [[] for _ in range(ep)]
    slot_index = [[-1] * k for _ in range(T)]
    status = 0
    for t in range(T):
        seen = {}                                  # region -> slot of the token's first copy
        for j in range(k):
            e = int(ids[t][j])
            if e == -1:
                continue
            if not (0 <= e < E):
                status |= 2
                continue
            r = e // epr
            if r in seen:
                slot_index[t][j] = seen[r]
                continue
            s = len(regions[r])
            regions[r].append(t * k + j)
            slot = r * cap + s if s < cap else -1
            if s >= cap:
                status |= 1
            seen[r] = slot
            slot_index[t][j] = slot
    counts = [len(g) for g in regions]
    src_index, rows = {}, {}
    for r in range(ep):
        for s, f in enumerate(regions[r][:cap]):
            src_index[(r, s)] = f
            rows[(r, s)] = [int(v) for v in x_bits[f // k]]
    return rows, counts, slot_index, src_index, status


def combine_region(y_rows, slot_index, T: int, H: int, cap: int) -> List[List[int]]:
    """Each distinct row of a token added once (order of first copies), fp32,
    narrowed once."""
    out = []
    for t in range(T):
        distinct = []
        for row in slot_index[t]:
            if row >= 0 and row not in distinct:
                distinct.append(row)
        line = []
        for h in range(H):
            acc = Fraction(0)
            for row in distinct:
                acc = round_binary(acc + bf16_value(int(y_rows[(row // cap, row % cap)][h])), FP32)
            line.append(round_to_bf16_bits(acc))
        out.append(line)
    return out
