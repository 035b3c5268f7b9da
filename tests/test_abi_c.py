"""The C ABI from plain C: include/ep.h compiles as strict C99, and a C
program linked against libep.so gets the sizing, status strings and host
argument checks it expects (tests/c/abi_host_check.c; no device memory)."""
import os
import shutil
import subprocess

import pytest

from combine_ep_get_layout_amd import ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.dirname(ep.LIB_PATH)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_is_strict_c99():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-fsyntax-only", "-x", "c", os.path.join(ROOT, "include", "ep.h")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_links_and_checks_host_paths(tmp_path):
    ep.lib()  # raises if the library has not been built
    exe = tmp_path / "abi_host_check"
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c", "abi_host_check.c"),
                        "-L", PKG, "-lep", f"-Wl,-rpath,{PKG}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi check ok" in r.stdout
