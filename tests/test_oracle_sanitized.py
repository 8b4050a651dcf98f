"""The oracle's pins, run against a build of the oracle with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only: the oracle is plain C).

The sanitized library is compiled into a temporary directory and loaded in a
child Python process with the sanitizer runtimes preloaded; any report (an
out-of-bounds access, a use after free, signed overflow, a misaligned load)
aborts the child, since the build does not recover from errors.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_act.py", "tests/test_oracle_formats.py", "tests/test_oracle_q4_0.py",
        "tests/test_oracle_affine.py", "tests/test_oracle_affine_bits.py", "tests/test_oracle_q4k.py",
        "tests/test_oracle_backward.py", "tests/test_oracle_threads.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.slow
def test_oracle_pins_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("the gcc sanitizer runtimes are not installed")
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env.update({"ORACLE_LIB": lib, "LD_PRELOAD": f"{asan}:{ubsan}",
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
