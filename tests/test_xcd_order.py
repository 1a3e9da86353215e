"""The combine's workgroup order across XCDs (xcd.h) on the host, compiled with
g++ (no GPU needed): a bijection of the grid that gives each XCD runs of
consecutive blocks."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_xcd_run_block_is_a_bijection_with_runs_per_xcd(tmp_path):
    exe = tmp_path / "xcd_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-I",
                    os.path.join(ROOT, "combine_get_dispatch_layout_amd", "csrc"),
                    os.path.join(ROOT, "tests", "xcd_check.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok ")
