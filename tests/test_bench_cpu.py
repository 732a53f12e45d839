"""Host-side arithmetic of bench.py's roofline report (no GPU)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402
from draft_verify_sampling_prev_amd import synth  # noqa: E402


def test_draft_tile_bytes_and_flops_at_headline_shape():
    """Method bytes (L rows, Bm, A rows) apart from the kernel's own partials; 2*B*r*V flops."""
    wl = synth.dsv4()
    method, impl, flops = bench.draft_tiles_bytes_flops(wl)
    nT = (129280 + 63) // 64
    assert method == 2 * (256 * 129280 + 256 * 129280 + 256 * 256) == 132_513_792
    assert impl == 256 * nT * 8 + 256 * 4
    assert flops == 2.0 * 256 * 256 * 129280
    # the fused kernel's intensity: ~128 flop per method byte, so at 8 TB/s it would run the MFMA at
    # ~1.02 PFLOP/s, 0.41 of the 2.5 PFLOP/s bf16 peak
    assert flops / method == pytest.approx(127.9, abs=0.1)
    assert flops / (method / 8.0e12) / 2.5e15 == pytest.approx(0.409, abs=0.001)


def test_acceptance_by_position():
    acc = [0, 1, 2, 2, 5, 3]
    ell = [5, 5, 5, 2, 5, 3]
    a = bench.acceptance_by_position(acc, ell, 5)
    # position 1: all six reach it, five accept; position 3: requests 2 and 4 (acc >= 2, ell >= 3)
    # and 5 (acc 3, ell 3) reach it, requests 4 and 5 accept it
    assert a["1"] == {"reached": 6, "accepted": round(5 / 6, 4)}
    assert a["3"] == {"reached": 3, "accepted": round(2 / 3, 4)}
    assert a["5"] == {"reached": 1, "accepted": 1.0}


def test_vocab_passes_sums_and_rates():
    wl = synth.dsv4()
    kern = {"draft_tiles": {"avg_us": 40.0, "launches_per_step": 5},
            "target_partials": {"avg_us": 30.0, "launches_per_step": 1},
            "resid_tiles": {"avg_us": 25.0, "launches_per_step": 1},
            "bonus_partials": {"avg_us": 5.0, "launches_per_step": 1}}
    adm, rej = 768.0, 100.0
    v = bench.vocab_passes(wl, kern, adm, rej)
    s, V, r, B = 2, wl.V, wl.r, wl.B
    tile_b, _, _ = bench.draft_tiles_bytes_flops(wl)
    expect = {"draft_tiles": tile_b, "target_partials": s * V * adm,
              "resid_tiles": s * (r * V + 2 * rej * V), "bonus_partials": s * V * (B - rej)}
    for name, b in expect.items():
        assert v[name]["bytes_per_launch"] == int(b)
        assert v[name]["GB/s"] == pytest.approx(b / (kern[name]["avg_us"] * 1e-6) / 1e9, rel=1e-3)
    tot_b = sum(expect[n] * kern[n]["launches_per_step"] for n in expect)
    tot_us = sum(kern[n]["avg_us"] * kern[n]["launches_per_step"] for n in expect)
    assert v["all"]["bytes_per_step"] == int(tot_b)
    assert v["all"]["us_per_step"] == pytest.approx(tot_us)
    assert v["all"]["frac"] == pytest.approx(tot_b / (tot_us * 1e-6) / 1e9 / 8000.0, rel=1e-3)
    flops = 2.0 * r * V * (wl.gamma * B + rej)
    assert v["markov_mfma"]["flops_per_step"] == flops
    assert v["markov_mfma"]["frac"] == pytest.approx(flops / (225.0 * 1e-6) / 1e12 / 2500.0, rel=1e-3)


def test_vocab_passes_skips_kernels_that_did_not_run():
    wl = synth.dsv4()
    kern = {"draft_tiles": {"avg_us": 40.0, "launches_per_step": 5},
            "target_partials": {"avg_us": 30.0, "launches_per_step": 1}}
    v = bench.vocab_passes(wl, kern, 768.0, 100.0)
    assert "bonus_partials" not in v and "resid_tiles" not in v and "markov_mfma" not in v
    assert v["all"]["us_per_step"] == pytest.approx(230.0)


def test_more_than_one_gpu_is_refused():
    import subprocess
    p = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode != 0
    assert "one GPU" in (p.stdout + p.stderr)


def test_tile_slots_match_the_library_rule():
    """The bench's copy of the slot rule (used to split the load-only ceiling kernel as the tile kernel splits its
    tiles): at most 12 tiles per slot, whole rounds of one workgroup per compute unit and row block."""
    assert bench.tile_slots(2020, 1, 256) == 256       # V = 129280, B <= 256: one round
    assert bench.tile_slots(2020, 4, 256) == 192       # 169 needed at 12 tiles per slot: three rounds of 64
    assert bench.tile_slots(2020, 4, 256, 36) == 64    # B = 1024 (full batch, up to 36 tiles): one round
    assert bench.tile_slots(1719, 2, 256, 36) == 128   # B = 512, V = 110000: 13-14 tiles per slot
    assert bench.tile_slots(16, 1, 256) == 16          # fewer tiles than compute units
    assert bench.tile_slots(3200, 1, 256) == 512       # 267 needed: two rounds


def test_probe_library_exports_its_timer():
    import ctypes
    path = os.path.join(os.path.dirname(bench.__file__), "draft_verify_sampling_prev_amd", "libdspark_probe.so")
    if not os.path.exists(path):
        pytest.skip("libdspark_probe.so not built")
    lib = ctypes.CDLL(path)
    assert hasattr(lib, "dspark_probe_time_tile_reads")
