"""The C ABI on the host, no GPU needed.

* the shared library loads and exports every function include/moe_a2a.h
  declares;
* the ctypes mirror of ``moe_handle`` and the constants match the header
  (checked by compiling the header with gcc);
* every argument and phase check returns its documented code before any HIP
  call is made (fake, aligned device addresses are never dereferenced on
  these paths).
"""
import ctypes
import os
import re
import subprocess

import pytest

import combine_moe_dispatch_03_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_a2a.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIBRARY):
        from combine_moe_dispatch_03_amd import build
        build.build()
    return moe.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(moe.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (moe_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_handle_layout_and_constants_match_header(tmp_path):
    fields = [f for f, _ in moe.MoeHandle._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "moe_a2a.h"',
            "int main(void){", 'printf("%zu\\n", sizeof(moe_handle));']
    prog += [f'printf("%zu\\n", offsetof(moe_handle, {f}));' for f in fields]
    consts = ["MOE_OK", "MOE_ERR_ARG", "MOE_ERR_PHASE", "MOE_ERR_OVERFLOW", "MOE_ERR_EXPERT_ID",
              "MOE_ERR_HIP", "MOE_ERR_NOALLOC_SIZE", "MOE_ERR_GAVE_UP", "MOE_NOALLOC_MAX_ITEMS", "MOE_STATUS_OVERFLOW", "MOE_STATUS_EXPERT_ID", "MOE_STATUS_GAVE_UP", "MOE_MAX_EP",
              "MOE_MAX_TOP_K", "MOE_MAX_FUSED_HIDDEN", "MOE_MAX_HIDDEN", "MOE_MAX_TOKENS", "MOE_MAX_PARTIALS", "MOE_LAYOUT_PER_COPY",
              "MOE_LAYOUT_PER_REGION"]
    prog += [f'printf("%d\\n", (int){c});' for c in consts]
    prog += ["return 0;}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), "-o", str(exe), str(src)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(moe.MoeHandle)
    for f, off in zip(fields, vals[1:1 + len(fields)]):
        assert getattr(moe.MoeHandle, f).offset == off, f
    for c, v in zip(consts, vals[1 + len(fields):]):
        assert getattr(moe, c) == v, c


FAKE = 0x100000   # aligned, never dereferenced by the validation paths


def make_handle(lib, max_tokens=64, H=128, k=2, E=8, ep=4, cap=128, layout=0):
    h = moe.MoeHandle()
    rc = lib.moe_init(ctypes.byref(h), max_tokens, H, k, E, ep, cap, layout, FAKE, FAKE, FAKE,
                      FAKE, FAKE, lib.moe_scratch_bytes(max_tokens, k, ep))
    assert rc == moe.MOE_OK
    return h


def test_sizes(lib):
    assert lib.moe_workspace_bytes(8, 32768, 7168) == 8 * 32768 * 7168 * 2
    assert lib.moe_workspace_bytes(0, 1, 8) == 0
    assert lib.moe_scratch_bytes(4096, 8, 8) >= (4096 * 8 + 64 * 8) * 4
    assert lib.moe_scratch_bytes(4096, 8, 8) % 256 == 0
    assert lib.moe_scratch_bytes(0, 8, 8) == 0
    assert lib.moe_scratch_bytes(16, 65, 8) == 0
    assert lib.moe_scratch_bytes(16, 8, 257) == 0
    assert lib.moe_scratch_bytes(1 << 30, 8, 8) == 0      # T*k beyond int32
    assert lib.moe_scratch_bytes((1 << 23) + 1, 1, 1) == 0  # past MOE_MAX_TOKENS
    assert lib.moe_scratch_bytes(1 << 23, 1, 1) > 0


@pytest.mark.parametrize("args", [
    dict(max_tokens=0), dict(max_tokens=(1 << 23) + 1), dict(H=0), dict(H=12), dict(H=4),
    dict(H=(1 << 20) + 8), dict(k=0), dict(k=65),
    dict(ep=0), dict(ep=257), dict(E=7), dict(E=2), dict(cap=0),
    dict(ep=8, E=8, cap=1 << 29), dict(layout=2), dict(layout=-1),
])
def test_init_rejects(lib, args):
    p = dict(max_tokens=64, H=128, k=2, E=8, ep=4, cap=128, layout=0)
    p.update(args)
    h = moe.MoeHandle()
    sb = lib.moe_scratch_bytes(max(p["max_tokens"], 1), max(min(p["k"], 64), 1),
                               max(min(p["ep"], 256), 1))
    rc = lib.moe_init(ctypes.byref(h), p["max_tokens"], p["H"], p["k"], p["E"], p["ep"],
                      p["cap"], p["layout"], FAKE, FAKE, FAKE, FAKE, FAKE, sb)
    assert rc == moe.MOE_ERR_ARG


def test_init_rejects_pointers_and_scratch(lib):
    h = moe.MoeHandle()
    sb = lib.moe_scratch_bytes(64, 2, 4)
    args = [64, 128, 2, 8, 4, 128, 0]
    assert lib.moe_init(ctypes.byref(h), *args, None, FAKE, FAKE, FAKE, FAKE, sb) == moe.MOE_ERR_ARG
    assert lib.moe_init(ctypes.byref(h), *args, FAKE, FAKE, FAKE, FAKE + 2, FAKE, sb) == moe.MOE_ERR_ARG
    assert lib.moe_init(ctypes.byref(h), *args, FAKE, FAKE, FAKE, FAKE, FAKE, sb - 4) == moe.MOE_ERR_ARG
    assert lib.moe_init(None, *args, FAKE, FAKE, FAKE, FAKE, FAKE, sb) == moe.MOE_ERR_ARG
    assert lib.moe_init(ctypes.byref(h), *args, FAKE, FAKE, FAKE, FAKE, FAKE, sb) == moe.MOE_OK
    assert h.experts_per_rank == 2 and h.phase == 0


def test_scratch_free_handle_and_noalloc_size_limit(lib):
    h = moe.MoeHandle()
    args = [1 << 20, 128, 2, 8, 4, 128, 0]
    # no scratch (NULL, 0): a handle for moe_dispatch_noalloc only
    assert lib.moe_init(ctypes.byref(h), *args, FAKE, FAKE, FAKE, FAKE, None, 0) == moe.MOE_OK
    assert lib.moe_init(ctypes.byref(h), *args, FAKE, FAKE, FAKE, FAKE, None, 64) == moe.MOE_ERR_ARG
    assert lib.moe_init(ctypes.byref(h), *args, FAKE, FAKE, FAKE, FAKE, None, 0) == moe.MOE_OK
    assert lib.moe_dispatch(ctypes.byref(h), FAKE, FAKE, 8, 8, FAKE, None) == moe.MOE_ERR_ARG
    assert lib.moe_dispatch_fp8(ctypes.byref(h), FAKE, FAKE, 8, 8, FAKE, FAKE, None) == moe.MOE_ERR_ARG
    assert lib.moe_route_counts(ctypes.byref(h), FAKE, 8, None) == moe.MOE_ERR_ARG
    # the static scratch holds MOE_NOALLOC_MAX_ITEMS routed copies (top-2 here)
    T = moe.MOE_NOALLOC_MAX_ITEMS // 2 + 1
    rc = lib.moe_dispatch_noalloc(ctypes.byref(h), FAKE, FAKE, T, T, FAKE, None)
    assert rc == moe.MOE_ERR_NOALLOC_SIZE and h.phase == 0
    assert "static routing scratch" in moe.moe_strerror(rc)
    assert lib.moe_dispatch_noalloc(ctypes.byref(h), FAKE + 8, FAKE, 8, 8, FAKE, None) == moe.MOE_ERR_ARG
    assert isinstance(lib.moe_last_hip_error(), int)


def test_dispatch_argument_checks(lib):
    h = make_handle(lib)
    d = lambda x, ids, T, R, ws: lib.moe_dispatch(ctypes.byref(h), x, ids, T, R, ws, None)
    assert d(FAKE, FAKE, 65, 65, FAKE) == moe.MOE_ERR_ARG          # R > max_tokens
    assert d(FAKE, FAKE, 33, 32, FAKE) == moe.MOE_ERR_ARG          # T > R
    assert d(FAKE, FAKE, 8, 0, FAKE) == moe.MOE_ERR_ARG            # R < 1
    assert d(FAKE, FAKE, -1, 8, FAKE) == moe.MOE_ERR_ARG
    assert d(FAKE + 8, FAKE, 8, 8, FAKE) == moe.MOE_ERR_ARG        # x not 16-byte aligned
    assert d(FAKE, FAKE + 2, 8, 8, FAKE) == moe.MOE_ERR_ARG        # ids not 4-byte aligned
    assert d(FAKE, FAKE, 8, 8, FAKE + 4) == moe.MOE_ERR_ARG        # workspace misaligned
    assert d(None, FAKE, 8, 8, FAKE) == moe.MOE_ERR_ARG
    assert d(FAKE, None, 8, 8, FAKE) == moe.MOE_ERR_ARG
    assert d(FAKE, FAKE, 8, 8, None) == moe.MOE_ERR_ARG
    assert h.phase == 0
    h.phase = 1                                                    # already dispatched
    assert d(FAKE, FAKE, 8, 8, FAKE) == moe.MOE_ERR_PHASE
    assert lib.moe_route_counts(ctypes.byref(h), FAKE, 8, None) == moe.MOE_ERR_PHASE
    assert lib.moe_reset(ctypes.byref(h)) == moe.MOE_OK and h.phase == 0
    assert lib.moe_route_counts(ctypes.byref(h), FAKE, 65, None) == moe.MOE_ERR_ARG
    assert lib.moe_route_counts(ctypes.byref(h), FAKE + 1, 8, None) == moe.MOE_ERR_ARG


def test_fp8_dispatch_argument_checks(lib):
    h = make_handle(lib)
    d = lambda x, ids, T, R, ws, sc: lib.moe_dispatch_fp8(ctypes.byref(h), x, ids, T, R, ws, sc, None)
    assert d(FAKE, FAKE, 8, 8, FAKE, None) == moe.MOE_ERR_ARG      # no scales
    assert d(FAKE, FAKE, 8, 8, FAKE, FAKE + 2) == moe.MOE_ERR_ARG  # scales misaligned
    assert d(FAKE, FAKE, 8, 8, FAKE + 8, FAKE) == moe.MOE_ERR_ARG  # workspace misaligned
    assert d(FAKE, FAKE, 65, 65, FAKE, FAKE) == moe.MOE_ERR_ARG
    wide = make_handle(lib, H=16392)
    assert lib.moe_dispatch_fp8(ctypes.byref(wide), FAKE, FAKE, 8, 8, FAKE, FAKE,
                                None) == moe.MOE_ERR_ARG         # row too wide for one block
    h.phase = 1
    assert d(FAKE, FAKE, 8, 8, FAKE, FAKE) == moe.MOE_ERR_PHASE
    assert h.phase == 1 and wide.phase == 0


def test_combine_argument_and_phase_checks(lib):
    h = make_handle(lib)
    c = lambda y, w, weighted, out: lib.moe_combine(ctypes.byref(h), y, w, weighted, out, None)
    assert c(FAKE, FAKE, 1, FAKE) == moe.MOE_ERR_PHASE              # no dispatch yet
    h.phase, h.num_tokens = 1, 8
    assert c(FAKE + 8, FAKE, 1, FAKE) == moe.MOE_ERR_ARG            # expert_out misaligned
    assert c(FAKE, None, 1, FAKE) == moe.MOE_ERR_ARG                # weighted without gates
    assert c(FAKE, FAKE + 2, 1, FAKE) == moe.MOE_ERR_ARG
    assert c(FAKE, FAKE, 1, FAKE + 8) == moe.MOE_ERR_ARG            # out misaligned
    assert c(FAKE, None, 0, None) == moe.MOE_ERR_ARG
    assert h.phase == 1                                             # failed checks change nothing
    f = lambda res, res_out, gamma, eps, normed: lib.moe_combine_residual_rmsnorm(
        ctypes.byref(h), FAKE, None, 0, res, res_out, gamma, eps, normed, None)
    assert f(FAKE, FAKE, FAKE, float("nan"), FAKE) == moe.MOE_ERR_ARG
    assert f(FAKE, FAKE, FAKE, -1e-6, FAKE) == moe.MOE_ERR_ARG
    assert f(FAKE, FAKE, FAKE, float("inf"), FAKE) == moe.MOE_ERR_ARG
    assert f(FAKE + 8, FAKE, FAKE, 1e-6, FAKE) == moe.MOE_ERR_ARG
    assert f(FAKE, None, FAKE, 1e-6, FAKE) == moe.MOE_ERR_ARG
    assert f(FAKE, FAKE, FAKE + 2, 1e-6, FAKE) == moe.MOE_ERR_ARG
    assert f(FAKE, FAKE, FAKE, 1e-6, None) == moe.MOE_ERR_ARG
    big = make_handle(lib, H=16392)
    big.phase, big.num_tokens = 1, 8
    assert lib.moe_combine_residual_rmsnorm(ctypes.byref(big), FAKE, None, 0, FAKE, FAKE, FAKE,
                                            1e-6, FAKE, None) == moe.MOE_ERR_ARG


def test_per_region_layout_rejects_a_weighted_combine(lib):
    h = make_handle(lib, layout=moe.MOE_LAYOUT_PER_REGION)
    assert h.layout == moe.MOE_LAYOUT_PER_REGION
    h.phase, h.num_tokens = 1, 8
    assert lib.moe_combine(ctypes.byref(h), FAKE, FAKE, 1, FAKE, None) == moe.MOE_ERR_ARG
    assert lib.moe_combine_residual_rmsnorm(ctypes.byref(h), FAKE, FAKE, 1, FAKE, FAKE, FAKE,
                                            1e-6, FAKE, None) == moe.MOE_ERR_ARG
    assert h.phase == 1


def test_strerror_and_reduced_flag(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert moe.moe_strerror(code) and moe.moe_strerror(code) != moe.moe_strerror(99)
    assert moe.moe_output_is_reduced() is True
    assert lib.moe_reset(None) == moe.MOE_ERR_ARG
    assert lib.moe_sync_status(None, None, None) == moe.MOE_ERR_ARG


def test_partials_argument_checks(lib):
    r = lambda src, P, T, H, out: lib.moe_partials_reduce(src, P, T, H, out, None)
    assert r(FAKE, 0, 8, 128, FAKE) == moe.MOE_ERR_ARG                 # no partials
    assert r(FAKE, 65, 8, 128, FAKE) == moe.MOE_ERR_ARG                # past MOE_MAX_PARTIALS
    assert r(FAKE, 8, -1, 128, FAKE) == moe.MOE_ERR_ARG
    assert r(FAKE, 1, (1 << 23) + 1, 128, FAKE) == moe.MOE_ERR_ARG     # past MOE_MAX_TOKENS
    assert r(FAKE, 8, 8, 12, FAKE) == moe.MOE_ERR_ARG                  # H % 8
    assert r(FAKE, 8, 8, 0, FAKE) == moe.MOE_ERR_ARG
    assert r(FAKE, 8, 8, (1 << 20) + 8, FAKE) == moe.MOE_ERR_ARG
    assert r(FAKE + 8, 8, 8, 128, FAKE) == moe.MOE_ERR_ARG             # partials misaligned
    assert r(None, 8, 8, 128, FAKE) == moe.MOE_ERR_ARG
    assert r(FAKE, 8, 8, 128, FAKE + 8) == moe.MOE_ERR_ARG             # out misaligned
    assert r(FAKE, 8, 8, 128, None) == moe.MOE_ERR_ARG
    f = lambda H, res, res_out, gamma, eps, normed: lib.moe_partials_reduce_residual_rmsnorm(
        FAKE, 8, 8, H, res, res_out, gamma, eps, normed, None)
    assert f(16392, FAKE, FAKE, FAKE, 1e-6, FAKE) == moe.MOE_ERR_ARG   # past MOE_MAX_FUSED_HIDDEN
    assert f(128, FAKE, FAKE, FAKE, float("nan"), FAKE) == moe.MOE_ERR_ARG
    assert f(128, FAKE, FAKE, FAKE, -1e-6, FAKE) == moe.MOE_ERR_ARG
    assert f(128, FAKE + 8, FAKE, FAKE, 1e-6, FAKE) == moe.MOE_ERR_ARG
    assert f(128, FAKE, None, FAKE, 1e-6, FAKE) == moe.MOE_ERR_ARG
    assert f(128, FAKE, FAKE, FAKE + 2, 1e-6, FAKE) == moe.MOE_ERR_ARG
    assert f(128, FAKE, FAKE, FAKE, 1e-6, None) == moe.MOE_ERR_ARG


def test_partials_reject_overlapping_outputs(lib):
    # only rejected calls: a call that passed its checks would launch on fake addresses
    P, T, H = 8, 4, 128
    rows = T * H * 2
    r = lambda out: lib.moe_partials_reduce(FAKE, P, T, H, out, None)
    assert r(FAKE) == moe.MOE_ERR_ARG                                  # out is the partials
    assert r(FAKE + P * rows - 16) == moe.MOE_ERR_ARG                  # last 16 bytes shared
    assert r(FAKE - rows + 16) == moe.MOE_ERR_ARG                      # first 16 bytes shared
    base = FAKE + 64 * rows            # outputs clear of the partials
    f = lambda res, res_out, gamma, normed: lib.moe_partials_reduce_residual_rmsnorm(
        FAKE, P, T, H, res, res_out, gamma, 1e-6, normed, None)
    assert f(base, FAKE + rows, base + 8 * rows, base + 4 * rows) == moe.MOE_ERR_ARG  # residual_out in partials
    assert f(base, base + 2 * rows, base + 8 * rows, FAKE) == moe.MOE_ERR_ARG         # normed in partials
    assert f(base, base, base + 8 * rows, base) == moe.MOE_ERR_ARG                    # normed = residual
    assert f(base, base + 2 * rows, base + 8 * rows, base + 2 * rows) == moe.MOE_ERR_ARG  # normed = residual_out
    assert f(base, base + 2 * rows, base + 2 * rows, base + 4 * rows) == moe.MOE_ERR_ARG  # residual_out over gamma
    assert f(base, base + 16, base + 8 * rows, base + 4 * rows) == moe.MOE_ERR_ARG    # residual_out partly over residual


def test_dispatch_and_combine_reject_overlapping_buffers(lib):
    # only rejected calls (fake addresses); workspace [4, 128, 128] bf16 = 128 KiB at FAKE
    h = make_handle(lib)
    far = FAKE + (1 << 24)
    assert lib.moe_dispatch(ctypes.byref(h), FAKE + 4096, far, 8, 8, FAKE, None) == moe.MOE_ERR_ARG
    assert lib.moe_dispatch_fp8(ctypes.byref(h), far, far + (1 << 20), 8, 8, FAKE, FAKE + 256,
                                None) == moe.MOE_ERR_ARG                      # scales inside ws8
    assert h.phase == 0
    h.phase, h.num_tokens = 1, 8
    assert lib.moe_combine(ctypes.byref(h), FAKE, None, 0, FAKE + 4096, None) == moe.MOE_ERR_ARG
    rows = 8 * 128 * 2
    f = lambda res, res_out, gamma, normed: lib.moe_combine_residual_rmsnorm(
        ctypes.byref(h), FAKE, None, 0, res, res_out, gamma, 1e-6, normed, None)
    assert f(far, far, far + 4 * rows, FAKE + 4096) == moe.MOE_ERR_ARG       # normed inside ws
    assert f(far, far, far + 4 * rows, far + 16) == moe.MOE_ERR_ARG          # normed over residual
    assert f(far, far + 16, far + 4 * rows, far + 2 * rows) == moe.MOE_ERR_ARG  # residual_out shifted
    assert h.phase == 1


def test_stream_probe_library_rejects_bad_arguments_before_any_launch():
    """The reference streaming kernels' library (the benchmark's ceilings
    mode) exports its one entry point, and every malformed call returns -1
    without a HIP call (the fake addresses are never used)."""
    from combine_moe_dispatch_03_amd import build
    if not os.path.exists(build.PROBE_LIBRARY):
        build.build()
    out = subprocess.run(["nm", "-D", "--defined-only", build.PROBE_LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    assert set(re.findall(r" T (moe_\w+)", out)) == {"moe_probe_stream"}
    probe = ctypes.CDLL(build.PROBE_LIBRARY).moe_probe_stream
    probe.restype = ctypes.c_int
    probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                      ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    dst, src = 0x7F0000000000, 0x7F1000000000
    bad = [
        (0, 0, dst, src, 0, 1024, 0, 0),            # no bytes
        (0, 0, dst, src, 1000, 1024, 0, 0),         # not a multiple of 16
        (0, 0, dst + 8, src, 1 << 20, 1024, 0, 0),  # misaligned dst
        (1, 0, dst, src + 4, 1 << 20, 1024, 0, 0),  # misaligned src
        (1, 0, dst, None, 1 << 20, 1024, 0, 0),     # copy without a source
        (2, 0, dst, None, 1 << 20, 0, 0, 0),        # grid 0
        (2, 0, dst, None, 1 << 20, (1 << 20) + 1, 0, 0),
        (0, 0, dst, src, 4096, 2048, 0, 0),         # read sink larger than dst
        (3, 0, dst, None, 1 << 20, 0, 100, 1),      # row not a multiple of 16
        (3, 0, dst, None, 1 << 20, 0, 16384, 0),    # no rows per workgroup
        (3, 0, dst, None, 1 << 13, 0, 16384, 1),    # not one whole row
        (6, 0, dst, None, 1024, 512, 0, 0),         # empty launch: sink larger than dst
        (6, 0, dst, None, 1 << 20, 0, 0, 0),        # empty launch: grid 0
        (7, 0, dst, src, 1 << 20, 1024, 0, 0),      # unknown kind
    ]
    for args in bad:
        assert probe(*args, None) == -1, args


def test_scratch_holds_the_single_pass_words(lib):
    """The scratch a handle needs: ranks (int32 per routed copy) and chunk
    histograms (int32 per chunk and region, 64 chunks), then, 8-byte aligned,
    the single-pass dispatch's 64-bit words: one per routed copy up to its
    largest batch of 65536 copies, and one per chunk and region; rounded up to
    256 bytes."""
    def expected(items, ep):
        offset = ((items + 64 * ep) * 4 + 7) // 8 * 8
        words = min(items, 65536) + 64 * ep
        return (offset + words * 8 + 255) // 256 * 256

    for T, k, ep in ((4096, 8, 8), (8192, 8, 16), (8193, 8, 8), (100000, 2, 4), (7, 3, 5), (1, 1, 1)):
        assert lib.moe_scratch_bytes(T, k, ep) == expected(T * k, ep), (T, k, ep)
