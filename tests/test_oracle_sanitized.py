"""The oracle's pins, run once more against an AddressSanitizer +
UndefinedBehaviorSanitizer build of oracle.c (CPU only): every oracle
function the pins call must stay inside its buffers and be free of
undefined behaviour on the pins' inputs, which include the edge cases
(empty and partial blocks, ties, every fp8 code, poisoned pools)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    import oracle
    lib = oracle.build(sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env.update(ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:allocator_may_return_null=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_pins_decode.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-3000:] + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail


PLANTED = r'''
import numpy as np, ctypes, oracle
L = oracle.Layout(1, 2, 1, 64, 16, 8, 8, oracle.KV_F32)
kp = np.zeros((8, 1, 16, 64), np.float32)
table = np.arange(8, dtype=np.int32)[None, :]
lens = np.array([128], np.int32)
out = np.zeros(1 * 1 * 8 * 2 * 64 - 64, np.float64)  # one block's summary short
p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
oracle.lib().or_summaries(ctypes.byref(L.c()), p(kp), None, p(table), p(lens), None, 8, p(out))
print("no report")
'''


def test_sanitizer_build_reports_a_planted_overrun(tmp_path):
    """The harness above is live: the sanitized oracle, handed an output
    buffer one block short, aborts with an AddressSanitizer report."""
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    import oracle
    lib = oracle.build(sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env.update(ORACLE_LIB=lib, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", PLANTED], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0 and "no report" not in r.stdout
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
