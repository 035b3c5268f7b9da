"""The C ABI driven end to end from plain C on the GPU: tests/c/abi_gpu_roundtrip.c
allocates device memory with the HIP runtime, runs layout, dispatch and
combine (normal mode, bf16), the fused low-latency FP8 call and message
mode (sizing, packer, delivery, receiver) through include/ep.h, and compares
every output with the oracle's C functions.
Compiling it needs only the headers, so that part runs on the CPU too."""
import os
import shutil
import subprocess

import pytest

from combine_ep_get_layout_amd import ep
from oracle import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.dirname(ep.LIB_PATH)
ORC = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SRC = os.path.join(ROOT, "tests", "c", "abi_gpu_roundtrip.c")


def build(exe):
    ep.lib()  # raises if the library has not been built
    orc.build()
    cmd = ["gcc", "-std=gnu99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", ORC, "-I", os.path.join(ROCM, "include"),
           SRC, "-L", PKG, "-lep", "-L", ORC, "-lep_oracle", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", "-lm", f"-Wl,-rpath,{PKG}:{ORC}:{os.path.join(ROCM, 'lib')}",
           "-o", str(exe)]
    return subprocess.run(cmd, capture_output=True, text=True)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_gpu_caller_compiles(tmp_path):
    r = build(tmp_path / "abi_gpu_roundtrip")
    assert r.returncode == 0, r.stderr


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_gpu_caller_matches_the_oracle(tmp_path):
    exe = tmp_path / "abi_gpu_roundtrip"
    r = build(exe)
    assert r.returncode == 0, r.stderr
    print("running", exe, flush=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "gpu roundtrip ok" in r.stdout
