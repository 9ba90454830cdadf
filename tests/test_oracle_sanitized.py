"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

A build of the C oracle with -fsanitize=address,undefined runs every pin in a
child process (the sanitizer runtime preloaded, since the Python interpreter
itself is not instrumented).  Any out-of-bounds access, use after free,
signed overflow, misaligned access or other undefined behaviour in the oracle
aborts that process and fails the test."""
import os
import subprocess
import sys

import pytest

import oracle

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


SCRIPT = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
o = oracle.Oracle({lib!r})
for pin in oracle_pins.ALL_PINS:
    pin(o)
    print("pin ok", pin.__name__, flush=True)
print("ALL PINS OK", flush=True)
"""


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_sanitized.so")
    oracle.build_library(lib, extra_flags=("-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                           "-fno-sanitize-recover=undefined"))
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    # Python's own allocations are not instrumented and are never freed at exit: leak reports would be noise.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", SCRIPT.format(root=ROOT, tests=TESTS, lib=lib)], env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "ALL PINS OK" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
