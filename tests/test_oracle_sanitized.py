"""The oracle's pins with the oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; gcc), run in a child process that
preloads the sanitizer runtime.  Any out-of-bounds access, use after free or
undefined arithmetic in the oracle's C ends that process with a report."""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime() is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libgdn_oracle_asan.so")
    flags = ["-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    subprocess.run(["gcc", *flags, "-I", oracle.HERE, "-o", lib, oracle.SRC, "-lm"], check=True)
    script = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import oracle, oracle_pins\n"
        "m = oracle.Oracle(%r)\n"
        "for pin in oracle_pins.ALL_PINS:\n"
        "    pin(m)\n"
        "print('pins ok', len(oracle_pins.ALL_PINS))\n" % (ROOT, HERE, lib))
    env = dict(os.environ, LD_PRELOAD=_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and "pins ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
