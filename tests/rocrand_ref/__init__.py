"""Build and load the rocRAND Philox cross-check helper (CPU only)."""
import ctypes
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "philox_rocrand.cpp")
LIB = os.path.join(HERE, "libphilox_rocrand.so")


def build(force: bool = False) -> str | None:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        return None
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.run([hipcc, "-O2", "-fPIC", "-shared", "--offload-arch=gfx950",
                        "-o", tmp, SRC], check=True)
        os.replace(tmp, LIB)
    return LIB


def load():
    path = build()
    if path is None:
        return None
    L = ctypes.CDLL(path)
    L.rr_philox_many.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int]
    L.rr_philox_many.restype = None
    return L
