"""Build and load the test-support HIP library tests/libfp8check.so (a device
check of the FP8 conversion the pack relies on; not part of libmoedx.so), and
build tests/c_consumer, a plain C program that uses libmoedx.so through
include/moedx.h only."""

from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "fp8_device_check.hip")
LIB = os.path.join(HERE, "libfp8check.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
C_SRC = os.path.join(HERE, "c_consumer.c")
C_BIN = os.path.join(HERE, "c_consumer")


def build() -> str:
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off",
           "-I", os.path.join(ROOT, "combine_get_dispatch_layout_amd", "csrc"), SRC,
           "-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_c_consumer(out: str = C_BIN) -> str:
    """gcc, C11, warnings as errors: the header must be plain C."""
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), C_SRC, "-o", out + ".tmp",
           "-L", os.path.join(ROOT, "combine_get_dispatch_layout_amd"), "-l:libmoedx.so",
           "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../combine_get_dispatch_layout_amd", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(out + ".tmp", out)
    return out


def load() -> ctypes.CDLL:
    if not os.path.exists(LIB):
        raise ImportError(f"{LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.fp8_cvt_check.restype = ctypes.c_int
    lib.fp8_cvt_check.argtypes = [ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32),
                                  ctypes.POINTER(ctypes.c_uint32)]
    return lib
