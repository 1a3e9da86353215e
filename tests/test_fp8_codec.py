"""The FP8 pack's arithmetic (csrc/fp8_codec.h) compiled for the host with g++
and checked against IEEE fp32 division and the oracle's brute-force E4M3FN
encoder (no GPU needed): the corrected-reciprocal quotient for every divisor
significand and bf16 numerator significand, the block scales for every bf16
value, the per-tensor quotient over scales spanning [2^-126, 2^126) with
subnormal numerators, and the branch-free encoder on a dense sweep."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _has_fma() -> bool:
    try:
        return " fma " in open("/proc/cpuinfo").read().replace("\n", " ")
    except OSError:
        return False


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc and g++")
def test_fp8_codec_against_ieee_and_oracle(tmp_path):
    obj = tmp_path / "oracle.o"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-c",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(obj)], check=True)
    exe = tmp_path / "fp8_check"
    # fused multiply-adds as the hardware instruction where the CPU has one (the
    # library fmaf otherwise: the same correctly rounded result, only slower);
    # no contraction of the separate multiplies
    fma = ["-mfma"] if _has_fma() else []
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", *fma,
                    "-pthread", "-I",
                    os.path.join(ROOT, "combine_get_dispatch_layout_amd", "csrc"),
                    os.path.join(ROOT, "tests", "fp8_check.cpp"), str(obj), "-lm",
                    "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok ")
