"""Build the gfx950 shared library ``libmoe_a2a.so`` in-tree with hipcc, and
the small CPython extension ``_moe_fast`` (per-call entry points with the
argument conversion in C) against it with the host C compiler.

Run ``python -m combine_moe_dispatch_03_amd.build`` (or call ``build()``).
Compiles for gfx950 only.  Flags:
  -ffp-contract=off     every fused multiply-add in a kernel is written out;
                        no other add/multiply pair is contracted, so the fp32
                        accumulation order is exactly the one in the source
  -packed-fp32-ops off  keep the compiler from emitting packed fp32 ops
"""
from __future__ import annotations

import os
import subprocess
import sys
import sysconfig
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libmoe_a2a.so")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "api.hip")]
ARCH = "gfx950"
# Reference streaming kernels (plain read / copy / write), loaded only by
# the benchmark's ceilings mode; no part of the dispatch/combine path.
PROBE_LIBRARY = os.path.join(PKG, "libmoe_stream_probe.so")
PROBE_SOURCE = os.path.join(CSRC, "stream_probe.hip")
FAST_SOURCE = os.path.join(CSRC, "pyfast.c")
FAST_MODULE = os.path.join(PKG, "_moe_fast" + sysconfig.get_config_var("EXT_SUFFIX"))

HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


# The host (x86) pass does not know gfx950's -packed-fp32-ops feature and
# warns that it ignores it; the device pass must accept it silently.
FEATURE_WARNING = "is not a recognized feature for this target"


def check_device_feature() -> None:
    """Compile a one-kernel probe for the device alone with the library's
    flags; fail if that pass does not accept -packed-fp32-ops (then the
    warning dropped from the full build below would hide that the feature no
    longer applies to the GPU code)."""
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "feature_probe.hip")
        with open(src, "w") as fh:
            fh.write("#include <hip/hip_runtime.h>\n"
                     "__global__ void probe(float *p) { p[threadIdx.x] += 1.0f; }\n")
        flags = [f for f in HIPCC_FLAGS if f not in ("-shared",)]
        cmd = [hipcc(), *flags, "--offload-device-only", "-c", "-o", os.path.join(d, "probe.o"), src]
        res = subprocess.run(cmd, capture_output=True, text=True)
        out = res.stdout + res.stderr
        if res.returncode != 0 or FEATURE_WARNING in out:
            raise RuntimeError("the gfx950 device pass does not accept -packed-fp32-ops:\n" + out)


def _hipcc_shared(output: str, sources: list, verbose: bool) -> None:
    tmp = output + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # only the host pass's warning remains possible here (check_device_feature)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if FEATURE_WARNING not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, output)


def build(output: str = LIBRARY, verbose: bool = False) -> str:
    check_device_feature()
    _hipcc_shared(output, SOURCES, verbose)
    if output == LIBRARY:
        build_fast(verbose)
        _hipcc_shared(PROBE_LIBRARY, [PROBE_SOURCE], verbose)
    return output


def build_fast(verbose: bool = False) -> str:
    """The CPython extension, linked to the in-tree library (found at run time
    next to the extension through its $ORIGIN run path)."""
    tmp = FAST_MODULE + ".tmp"
    cmd = [os.environ.get("CC", "gcc"), "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-Werror", "-I", sysconfig.get_paths()["include"], "-I", INCLUDE, "-o", tmp, FAST_SOURCE,
           "-L", PKG, "-lmoe_a2a", "-Wl,-rpath,$ORIGIN"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building _moe_fast failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, FAST_MODULE)
    return FAST_MODULE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
