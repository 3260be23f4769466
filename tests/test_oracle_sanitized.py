"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only): an instrumented build of oracle.c is loaded into a child
process, with the ASan runtime preloaded, and every entry point runs on small
seeded descriptors (tests/sanitized_oracle_calls.py). An out-of-bounds access,
use after free or undefined operation in the oracle aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    try:
        path = subprocess.run(["gcc", f"-print-file-name={name}"], check=True,
                              capture_output=True, text=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no AddressSanitizer runtime for gcc here")
    sys.path.insert(0, ROOT)
    from oracle import build
    lib = build.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ, HP_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitized_oracle_calls.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    report = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, report
    assert "every entry point called" in r.stdout, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
