"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: oracle.c
is built with -fsanitize=address,undefined (every report fatal) and the
hand-worked, property and FP8-mode pins run against that build in a child
Python process with the sanitizer runtime preloaded (host code only; nothing
here touches a GPU)."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BATTERY = ["tests/test_oracle_handworked.py", "tests/test_oracle_properties.py",
           "tests/test_oracle_fp8_modes.py"]


def _asan_runtime():
    if shutil.which("gcc") is None:
        return None
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _preload_in_use() -> bool:
    """A preload set up by the environment (not ours to replace)."""
    if os.environ.get("LD_PRELOAD"):
        return True
    try:
        return bool(open("/etc/ld.so.preload").read().strip())
    except OSError:
        return False


@pytest.mark.skipif(_asan_runtime() is None, reason="needs gcc's AddressSanitizer runtime")
@pytest.mark.skipif(_preload_in_use(), reason="the environment already preloads a library")
def test_oracle_battery_under_address_and_ub_sanitizers(tmp_path):
    lib = tmp_path / "liboracle_sanitized.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.c"),
                    "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", MOEDX_ORACLE_LIB=str(lib))
    # -s: a sanitizer report goes straight to the child's stderr, which is kept
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        *BATTERY], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    report = (r.stdout + r.stderr)[-4000:]
    assert "Sanitizer" not in r.stderr, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
