"""The oracle's CPU pins run once more against an AddressSanitizer +
UndefinedBehaviorSanitizer build of oracle/dspark_oracle.c (host code only),
in a child process: any out-of-bounds access, use after free or undefined
operation in the oracle (or its threaded request split) fails the run."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle_rng.py", "test_oracle_draft.py", "test_oracle_schedule.py", "test_oracle_verify.py",
        "test_oracle_threads.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc has no AddressSanitizer runtime here")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = oracle.build(out=str(tmp_path / "liboracle_asan.so"),
                       extra=["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                              "-g"])
    env = dict(os.environ)
    env.update({
        "DSPARK_ORACLE_LIB": lib,
        "LD_PRELOAD": _runtime("libasan.so"),  # the interpreter itself is not instrumented
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           *[os.path.join(ROOT, "tests", f) for f in PINS]]
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = p.stdout + p.stderr
    assert p.returncode == 0, log[-4000:]
    assert "runtime error" not in log and "AddressSanitizer" not in log, log[-4000:]
