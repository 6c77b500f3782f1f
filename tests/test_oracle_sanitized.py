"""The C oracle's CPU checks run again against an AddressSanitizer +
UndefinedBehaviorSanitizer build of the oracle (gcc, host code only), in a
subprocess that preloads the ASan runtime: every parity claim rests on the
oracle's heap, ranking and mask code being free of out-of-bounds accesses
and undefined behaviour."""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's ASan runtime is not installed")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = O.build_oracle(sanitize=True, out=str(tmp_path / "libddtree_oracle_san.so"))
    env = dict(os.environ)
    env.update(DDT_ORACLE_LIB=lib, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", t) for t in
             ("test_oracle_pins.py", "test_parity_rules.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-m", "not gpu",
                        "-p", "no:cacheprovider", "-W", "ignore::DeprecationWarning", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
