"""CPU emulation of the persistent draft's device-wide barrier protocol
(csrc/dspark_gridsync.hpp, compiled unchanged with std::atomic operations,
one thread per workgroup): ordering across many barriers, and the bounded
give-up paths (an arrival that never comes, a workgroup that stops)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "draft_verify_sampling_prev_amd", "csrc")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("gridsync") / "gridsync_emulation")
    subprocess.run(["g++", "-std=c++17", "-O2", "-pthread", "-Wall", "-Wextra", "-I", CSRC,
                    os.path.join(ROOT, "tests", "gridsync_emulation.cpp"), "-o", out], check=True)
    return out


def _run(exe, *args, timeout=120):
    p = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=timeout)
    assert p.returncode == 0, p.stderr
    return {k: v for k, v in re.findall(r"(\w+)=(\S+)", p.stdout)}


def test_every_group_passes_every_barrier_in_order(exe):
    r = _run(exe, "order", 64, 40)
    assert int(r["violations"]) == 0
    assert int(r["passed"]) == 64 * 40 and int(r["gave_up"]) == 0 and r["error"] == "0"
    assert int(r["counter"]) == 64 * 40


def test_missing_arrival_makes_every_group_give_up(exe):
    r = _run(exe, "phantom", 32, 20000)
    assert int(r["gave_up"]) == 32 and int(r["passed"]) == 0 and r["error"] == "1"


def test_stopped_group_makes_the_others_give_up(exe):
    r = _run(exe, "dead", 32, 20000)
    # barrier 0 completes for all 32; at barrier 1 group 0 is absent and the other 31 give up
    assert int(r["passed"]) == 32 and int(r["gave_up"]) == 31 and r["error"] == "1"
    assert int(r["violations"]) == 0
