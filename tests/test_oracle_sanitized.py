"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(host only): every oracle pin (tests/test_oracle_*.py and the datapath model
pin) runs again in a child process against a sanitized build of
oracle/fp8_oracle.c, with the ASan runtime preloaded and any report fatal."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    try:
        out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    except (OSError, subprocess.CalledProcessError):
        return None
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc's ASan runtime is not installed")
    env = dict(os.environ)
    env.update({
        "FP8_ORACLE_SANITIZE": "1",
        "LD_PRELOAD": rt,
        # Python and numpy are not instrumented: leak reports from them are noise
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "4",
    })
    pins = sorted(f for f in os.listdir(os.path.join(ROOT, "tests"))
                  if f.startswith("test_oracle_") and f.endswith(".py") and f != os.path.basename(__file__))
    pins.append("test_datapath_model.py")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + \
          [os.path.join("tests", f) for f in pins]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
