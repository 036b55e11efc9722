"""The library used from plain C (tests/c_consumer.c): the header compiles as
C11 together with the HIP runtime API, the program links against the shared
library alone, and on a GPU it runs a dispatch / combine round trip whose
results it checks itself (no Python, no torch, no oracle)."""
import os
import subprocess

import pytest

import combine_moe_dispatch_03_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_consumer(tmp_path):
    if not os.path.exists(moe.LIBRARY):
        from combine_moe_dispatch_03_amd import build
        build.build()
    libdir = os.path.dirname(moe.LIBRARY)
    exe = str(tmp_path / "c_consumer")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    os.path.join(ROOT, "tests", "c_consumer.c"), "-o", exe,
                    "-L", libdir, "-lmoe_a2a", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"],
                   check=True, capture_output=True, text=True)
    return exe


def test_c_consumer_builds(tmp_path):
    assert os.path.exists(build_consumer(tmp_path))


@pytest.mark.gpu
def test_c_consumer_round_trip_on_gpu(tmp_path):
    exe = build_consumer(tmp_path)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c consumer: ok" in res.stdout
