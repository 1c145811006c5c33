"""The C ABI from a C program (no Python, no torch): compiled on any machine
against include/specverify.h and libspecverify.so; run on the GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "verify_main.c")
PKG = os.path.join(ROOT, "rejection_sampling_verify_17_amd")


ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp) -> str:
    cc = shutil.which("gcc")
    if cc is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("no gcc or no HIP headers")
    if not os.path.exists(os.path.join(PKG, "libspecverify.so")):
        pytest.skip("library not built")
    exe = os.path.join(tmp, "verify_main")
    # plain C11, linked against the library and the HIP runtime
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), SRC, "-L", PKG, "-lspecverify", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program_builds(tmp_path):
    assert os.path.exists(_build(str(tmp_path)))


@pytest.mark.gpu
def test_c_program_runs(tmp_path):
    exe = _build(str(tmp_path))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "c abi ok" in r.stdout
