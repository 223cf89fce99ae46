"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
its pins run again in a child process against the instrumented build, with the
sanitizer runtime preloaded; any out-of-bounds access, use of uninitialised pointers'
memory, overflow or other undefined behaviour ends that run with an error."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_pins_under_sanitizers():
    sys.path.insert(0, ROOT)
    from oracle import build
    try:
        lib = build.build(sanitize=True)
    except (subprocess.CalledProcessError, FileNotFoundError) as e:
        pytest.skip(f"no sanitizer toolchain: {e}")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("libasan not found")
    env = dict(os.environ, BOLE_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=97",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=98",
               OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
