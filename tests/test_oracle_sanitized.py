"""The CPU oracle's pins again, against its AddressSanitizer +
UndefinedBehaviorSanitizer build (oracle variant "san"), in a child process
started with the ASan runtime preloaded (the oracle is a library loaded into
Python, so the runtime must come first). Any out-of-bounds access, use after
free or undefined behaviour in the oracle aborts the child and fails here."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan():
    import oracle
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc has no libasan here")
    assert not oracle.stale("san")
    env = dict(os.environ, LD_PRELOAD=asan, MOE_ORACLE_VARIANT="san",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    probe = ("import numpy as np, oracle\n"
             "oracle.route_topk(np.zeros((2, 4), np.float32), 2)\n"
             "maps = open('/proc/self/maps').read()\n"
             "print(oracle.variant(), 'libmoeoracle_san.so' in maps, 'libasan' in maps)\n")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.stdout.split() == ["san", "True", "True"], (r.stdout + r.stderr)[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", "tests/test_oracle_pins.py",
                        "tests/test_oracle_gemm_pins.py",
                        # the all-patterns sweep runs on the OpenMP build, not this one
                        "-k", "not all_fp32_patterns"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
