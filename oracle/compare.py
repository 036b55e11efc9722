"""Comparators and the double-reduce detector.

TEST INFRASTRUCTURE ONLY.

* ``ulp_distance``: distance between two bf16 bit patterns counted in
  representable steps.  Patterns are mapped to ordered integers (negative
  numbers below positive ones, +0 and -0 both to 0), so one step across zero
  counts as one.
* ``rel_err``: max |a - b| / max(|b|, floor).  The 0.02 floor is the magnitude
  floor of the CollectiveX combine gate (InferenceX PR #2450, "Anatomy of the
  failing element": cancelling contributions near zero turn one ulp into a
  large relative error, which the floor keeps from dominating).
* ``reduce_multiplicity``: how many times a combine output counts the
  once-reduced result.  vLLM PR #41382 ("Fix double reduce ...") describes a
  framework summing again over the experts dimension after the all-to-all had
  already done it; the least-squares factor alpha_t = <out_t, once_t> /
  <once_t, once_t> per token is 1 for a correct combine and 2 for a result
  reduced twice.
"""
from __future__ import annotations

import numpy as np


def _ordered(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def is_nan_bits(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Elementwise bf16 step distance; NaN on either side counts as 1 << 20."""
    d = np.abs(_ordered(a_bits) - _ordered(b_bits))
    return np.where(is_nan_bits(a_bits) | is_nan_bits(b_bits), 1 << 20, d)


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def rel_err(a_bits: np.ndarray, b_bits: np.ndarray, floor: float = 0.02) -> float:
    a = bf16_to_float(a_bits).astype(np.float64)
    b = bf16_to_float(b_bits).astype(np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), floor)))


def reduce_multiplicity(out_bits: np.ndarray, once_bits: np.ndarray) -> np.ndarray:
    """Per-token factor alpha_t with out_t ~ alpha_t * once_t."""
    o = bf16_to_float(out_bits).astype(np.float64).reshape(out_bits.shape[0], -1)
    r = bf16_to_float(once_bits).astype(np.float64).reshape(once_bits.shape[0], -1)
    den = np.einsum("th,th->t", r, r)
    num = np.einsum("th,th->t", o, r)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), 1.0)


def reduced_more_than_once(out_bits: np.ndarray, once_bits: np.ndarray) -> bool:
    """True if the median token counts its reduction about twice or more."""
    alpha = reduce_multiplicity(out_bits, once_bits)
    return bool(np.median(alpha) > 1.5)
