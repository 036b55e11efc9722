"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* the CPU oracle, built with gcc -fsanitize=address,undefined, driven through
  ordinary inputs and every edge case it handles (empty batches, overflow,
  bad ids, the limits, both layouts, every e4m3 code, special values);
* the host side of the C ABI (api.hip) built with host-only sanitizers
  against stub kernel launchers, driven through its argument checks, phase
  machine, HIP-error path and the single-pass branch (epochs, the clearing
  of its words, the fallback under capture), with the capture query and the
  memset stood in for by the driver.
GPU code is never built with a sanitizer here.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def _run(exe):
    # a library preloaded into every process would come before the ASan
    # runtime in the link order; let ASan accept that rather than touch it
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "runtime error" not in res.stderr and "ERROR: AddressSanitizer" not in res.stderr
    return res.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", *SAN, "-o", exe,
                    os.path.join(HERE, "sanitize_oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"], check=True)
    assert "ok" in _run(exe)


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc for the HIP runtime headers")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    exe = str(tmp_path / "abi_san")
    host_san = []
    for flag in SAN:
        host_san += ["-Xarch_host", flag] if flag.startswith("-fsanitize") or flag.startswith("-fno-sanitize") else [flag]
    subprocess.run([hipcc, "-O1", "-std=c++17", "--offload-arch=gfx950", *host_san,
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "combine_moe_dispatch_03_amd", "csrc"), "-o", exe,
                    os.path.join(HERE, "sanitize_abi_driver.cpp"),
                    os.path.join(ROOT, "combine_moe_dispatch_03_amd", "csrc", "api.hip")],
                   check=True, capture_output=True)
    assert "ok" in _run(exe)
