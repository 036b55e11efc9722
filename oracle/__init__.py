"""CPU oracle for MoE dispatch, reduce-once combine and the fused epilogue.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
benchmark's CPU-baseline leg are its only users; the product path never
imports it.  The arithmetic lives in ``moe_oracle.c`` (plain scalar C); this
module builds it with gcc and wraps it over numpy arrays.  ``brute`` holds a
second, pure-Python rendering for tiny inputs; ``compare`` holds the
comparators and the double-reduce detector.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "moe_oracle.c")
LIBRARY = os.path.join(HERE, "libmoe_oracle.so")
# -ffp-contract=off: every fused multiply-add in the oracle is an explicit fmaf.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]
# The same source built for timing only (the CPU baseline): -O3 for the host
# it runs on.  The arithmetic flags are the same, so the results are too.
TIMING_LIBRARY = os.path.join(HERE, "libmoe_oracle_timing.so")
TIMING_CFLAGS = ["-O3", "-march=native", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                 "-fno-fast-math"]

STATUS_OVERFLOW = 1
STATUS_BAD_ID = 2


def build(source: str = SOURCE, output: str = LIBRARY, flags=CFLAGS) -> str:
    """Compile the oracle with gcc; returns the path of the shared library."""
    tmp = output + ".tmp"
    subprocess.run(["gcc", *flags, "-o", tmp, source, "-lm"], check=True)
    os.replace(tmp, output)
    return output


def build_timing(output: str = TIMING_LIBRARY) -> str:
    """The timing build (-O3 -march=native).  Build it on the host that times
    it: -march=native targets the CPU doing the compiling."""
    return build(SOURCE, output, TIMING_CFLAGS)


def load_timing(rebuild: bool = True) -> "Oracle":
    """The timing build of the oracle, compiled here first unless told not to."""
    if rebuild or not os.path.exists(TIMING_LIBRARY):
        build_timing()
    return Oracle(TIMING_LIBRARY)


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    lib.oracle_dispatch.argtypes = [_P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P]
    lib.oracle_dispatch.restype = ctypes.c_int
    lib.oracle_combine.argtypes = [_P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P]
    lib.oracle_combine.restype = ctypes.c_int
    lib.oracle_combine_residual_rmsnorm.argtypes = [
        _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P, _P, ctypes.c_float, _P, _P, _P, _P]
    lib.oracle_combine_residual_rmsnorm.restype = ctypes.c_int
    lib.oracle_dispatch_region.argtypes = lib.oracle_dispatch.argtypes
    lib.oracle_dispatch_region.restype = ctypes.c_int
    lib.oracle_combine_region.argtypes = [_P, _P, _I64, _I64, _I64, _P]
    lib.oracle_combine_region.restype = ctypes.c_int
    lib.oracle_combine_residual_rmsnorm_region.argtypes = [
        _P, _P, _I64, _I64, _I64, _P, _P, ctypes.c_float, _P, _P, _P, _P]
    lib.oracle_combine_residual_rmsnorm_region.restype = ctypes.c_int
    lib.oracle_partials_reduce.argtypes = [_P, _I64, _I64, _I64, _P]
    lib.oracle_partials_reduce.restype = ctypes.c_int
    lib.oracle_partials_reduce_residual_rmsnorm.argtypes = [
        _P, _I64, _I64, _I64, _P, _P, ctypes.c_float, _P, _P, _P, _P]
    lib.oracle_partials_reduce_residual_rmsnorm.restype = ctypes.c_int
    lib.oracle_quantize_e4m3_rows.argtypes = [_P, _I64, _I64, _P, _P]
    lib.oracle_quantize_e4m3_rows.restype = None
    for name in ("oracle_bf16_to_f32_array", "oracle_f32_to_bf16_array",
                 "oracle_f64_to_bf16_array", "oracle_e4m3_to_f32_array",
                 "oracle_f32_to_e4m3_array"):
        getattr(lib, name).argtypes = [_P, _P, _I64]
        getattr(lib, name).restype = None
    return lib


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        self.path = path
        self.lib = _declare(ctypes.CDLL(path))

    # -- codec -----------------------------------------------------------
    def bf16_to_f32(self, u: np.ndarray) -> np.ndarray:
        u = np.ascontiguousarray(u, dtype=np.uint16)
        out = np.empty(u.shape, dtype=np.float32)
        self.lib.oracle_bf16_to_f32_array(u.ctypes.data, out.ctypes.data, u.size)
        return out

    def f32_to_bf16(self, a: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float32)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.oracle_f32_to_bf16_array(a.ctypes.data, out.ctypes.data, a.size)
        return out

    def f64_to_bf16(self, a: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.oracle_f64_to_bf16_array(a.ctypes.data, out.ctypes.data, a.size)
        return out

    def e4m3_to_f32(self, c: np.ndarray) -> np.ndarray:
        c = np.ascontiguousarray(c, dtype=np.uint8)
        out = np.empty(c.shape, dtype=np.float32)
        self.lib.oracle_e4m3_to_f32_array(c.ctypes.data, out.ctypes.data, c.size)
        return out

    def f32_to_e4m3(self, a: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float32)
        out = np.empty(a.shape, dtype=np.uint8)
        self.lib.oracle_f32_to_e4m3_array(a.ctypes.data, out.ctypes.data, a.size)
        return out

    def quantize_e4m3_rows(self, x: np.ndarray):
        """(q uint8 [T, H], scale fp32 [T]) of the FP8 payload."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        T, H = x.shape
        q = np.empty((T, H), dtype=np.uint8)
        scale = np.empty(T, dtype=np.float32)
        self.lib.oracle_quantize_e4m3_rows(x.ctypes.data, T, H, q.ctypes.data, scale.ctypes.data)
        return q, scale

    def dispatch_fp8(self, x: np.ndarray, ids: np.ndarray, ep: int, epr: int, cap: int,
                     layout: str = "copy"):
        """FP8 dispatch: quantised rows placed exactly as the bf16 rows are
        (a byte copy of each quantised row), plus each row's scale.
        Returns (DispatchResult with ws uint8 [ep, cap, H], scales fp32 [ep, cap])."""
        q, scale = self.quantize_e4m3_rows(x)
        T, H = q.shape
        k = ids.shape[1]
        d = self.dispatch(q.view(np.uint16), ids, ep, epr, cap, layout=layout)
        d.ws = d.ws.view(np.uint8).reshape(ep, cap, H)
        scales = np.full((ep, cap), np.nan, dtype=np.float32)
        for r in range(ep):
            n = min(int(d.counts[r]), cap)
            scales[r, :n] = scale[d.src_index[r, :n] // k]
        return d, scales

    # -- the method --------------------------------------------------------
    def dispatch(self, x: np.ndarray, ids: np.ndarray, ep: int, epr: int, cap: int,
                 ws: Optional[np.ndarray] = None, src_fill: int = -1,
                 layout: str = "copy") -> "DispatchResult":
        """Route every copy into the padded workspace.

        ``layout`` is "copy" (one row per routed copy) or "region" (one row
        per token and destination region).  ``ws`` may be passed in (e.g.
        pre-filled with canaries); otherwise an uninitialised [ep, cap, H]
        array is allocated, whose padding rows stay untouched (so never
        committed to memory by the OS).
        """
        x = np.ascontiguousarray(x, dtype=np.uint16)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        T, H = x.shape
        k = ids.shape[1] if ids.ndim == 2 else (ids.size // T if T else 0)
        if ws is None:
            ws = np.empty((ep, cap, H), dtype=np.uint16)
        assert ws.dtype == np.uint16 and ws.flags.c_contiguous and ws.size == ep * cap * H
        counts = np.zeros(ep, dtype=np.int32)
        slot_index = np.empty(T * k, dtype=np.int32)
        src_index = np.full(ep * cap, src_fill, dtype=np.int32)
        fn = {"copy": self.lib.oracle_dispatch, "region": self.lib.oracle_dispatch_region}[layout]
        status = fn(
            x.ctypes.data, ids.ctypes.data, T, H, k, ep, epr, cap, ws.ctypes.data,
            counts.ctypes.data, slot_index.ctypes.data, src_index.ctypes.data)
        return DispatchResult(ws=ws, counts=counts, slot_index=slot_index.reshape(T, k),
                              src_index=src_index.reshape(ep, cap), status=status)

    def combine(self, y: np.ndarray, slot_index: np.ndarray, weights: Optional[np.ndarray],
                weighted: bool, H: int, layout: str = "copy") -> np.ndarray:
        y = np.ascontiguousarray(y, dtype=np.uint16)
        slot_index = np.ascontiguousarray(slot_index, dtype=np.int32)
        T, k = slot_index.shape
        if layout == "region":
            assert not weighted, "the per-region combine is unweighted"
            out = np.empty((T, H), dtype=np.uint16)
            self.lib.oracle_combine_region(y.ctypes.data, slot_index.ctypes.data, T, H, k,
                                           out.ctypes.data)
            return out
        w = np.ascontiguousarray(weights if weights is not None else np.zeros((T, k)),
                                 dtype=np.float32)
        out = np.empty((T, H), dtype=np.uint16)
        self.lib.oracle_combine(y.ctypes.data, slot_index.ctypes.data, w.ctypes.data,
                                int(bool(weighted)), T, H, k, out.ctypes.data)
        return out

    def combine_residual_rmsnorm(self, y, slot_index, weights, weighted: bool,
                                 residual: np.ndarray, gamma: np.ndarray, eps: float,
                                 want_f64: bool = False, layout: str = "copy"):
        """Returns (residual_out, normed[, normed_f64])."""
        y = np.ascontiguousarray(y, dtype=np.uint16)
        slot_index = np.ascontiguousarray(slot_index, dtype=np.int32)
        residual = np.ascontiguousarray(residual, dtype=np.uint16)
        gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
        T, k = slot_index.shape
        H = residual.shape[1]
        w = np.ascontiguousarray(weights if weights is not None else np.zeros((T, k)),
                                 dtype=np.float32)
        res_out = np.empty((T, H), dtype=np.uint16)
        normed = np.empty((T, H), dtype=np.uint16)
        nf64 = np.empty((T, H), dtype=np.float64) if want_f64 else None
        scratch = np.empty(H, dtype=np.float32)
        if layout == "region":
            assert not weighted, "the per-region combine is unweighted"
            self.lib.oracle_combine_residual_rmsnorm_region(
                y.ctypes.data, slot_index.ctypes.data, T, H, k, residual.ctypes.data,
                gamma.ctypes.data, float(eps), res_out.ctypes.data, normed.ctypes.data,
                nf64.ctypes.data if want_f64 else None, scratch.ctypes.data)
        else:
            self.lib.oracle_combine_residual_rmsnorm(
                y.ctypes.data, slot_index.ctypes.data, w.ctypes.data, int(bool(weighted)),
                T, H, k, residual.ctypes.data, gamma.ctypes.data, float(eps),
                res_out.ctypes.data, normed.ctypes.data,
                nf64.ctypes.data if want_f64 else None, scratch.ctypes.data)
        return (res_out, normed, nf64) if want_f64 else (res_out, normed)

    def partials_reduce(self, partials: np.ndarray) -> np.ndarray:
        """Sum of P partial hidden states [P, T, H] (bf16 patterns) -> [T, H]:
        fp32 in rank order, one narrowing."""
        partials = np.ascontiguousarray(partials, dtype=np.uint16)
        P, T, H = partials.shape
        out = np.empty((T, H), dtype=np.uint16)
        self.lib.oracle_partials_reduce(partials.ctypes.data, P, T, H, out.ctypes.data)
        return out

    def partials_reduce_residual_rmsnorm(self, partials: np.ndarray, residual: np.ndarray,
                                         gamma: np.ndarray, eps: float, want_f64: bool = False):
        """The sum of the partials, + residual, RMSNorm; returns
        (residual_out, normed[, normed_f64])."""
        partials = np.ascontiguousarray(partials, dtype=np.uint16)
        residual = np.ascontiguousarray(residual, dtype=np.uint16)
        gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
        P, T, H = partials.shape
        res_out = np.empty((T, H), dtype=np.uint16)
        normed = np.empty((T, H), dtype=np.uint16)
        nf64 = np.empty((T, H), dtype=np.float64) if want_f64 else None
        scratch = np.empty(H, dtype=np.float32)
        self.lib.oracle_partials_reduce_residual_rmsnorm(
            partials.ctypes.data, P, T, H, residual.ctypes.data, gamma.ctypes.data, float(eps),
            res_out.ctypes.data, normed.ctypes.data, nf64.ctypes.data if want_f64 else None,
            scratch.ctypes.data)
        return (res_out, normed, nf64) if want_f64 else (res_out, normed)


@dataclass
class DispatchResult:
    ws: np.ndarray           # uint16 [ep, cap, H]
    counts: np.ndarray       # int32 [ep]
    slot_index: np.ndarray   # int32 [T, k]
    src_index: np.ndarray    # int32 [ep, cap]
    status: int


_DEFAULT: Optional[Oracle] = None


def load(rebuild: bool = False) -> Oracle:
    """The oracle built from ``moe_oracle.c`` (compiled on first use)."""
    global _DEFAULT
    if _DEFAULT is None or rebuild:
        stale = (not os.path.exists(LIBRARY)
                 or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE))
        if rebuild or stale:
            build()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT


def place_expert_outputs(ws: np.ndarray, slot_index: np.ndarray, y_rows: np.ndarray) -> None:
    """Expert stage: write each copy's output row into the row it was routed to.

    Under the per-region layout pass one message per first copy (rows of the
    other copies are ignored: they share the first copy's row)."""
    flat = ws.reshape(-1, ws.shape[-1])
    s = slot_index.reshape(-1)
    valid = s >= 0
    _, first = np.unique(s, return_index=True)     # first copy naming each row
    first = first[s[first] >= 0]
    flat[s[first]] = y_rows[first]
    assert valid.sum() >= first.size
