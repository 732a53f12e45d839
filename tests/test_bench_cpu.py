"""Host-side arithmetic of bench.py's roofline report (no GPU)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402
from draft_verify_sampling_prev_amd import synth  # noqa: E402


def test_draft_tile_bytes_and_flops_at_headline_shape():
    wl = synth.dsv4()
    byts, flops = bench.draft_tiles_bytes_flops(wl)
    nT = (129280 + 63) // 64
    assert byts == 2 * (256 * 129280 + 256 * 129280 + 256 * 256) + 256 * nT * 8 + 256 * 4
    assert flops == 2.0 * 256 * 256 * 129280


def test_vocab_passes_sums_and_rates():
    wl = synth.dsv4()
    kern = {"draft_tiles": {"avg_us": 40.0, "launches_per_step": 5},
            "target_partials": {"avg_us": 30.0, "launches_per_step": 1},
            "resid_tiles": {"avg_us": 25.0, "launches_per_step": 1},
            "bonus_partials": {"avg_us": 5.0, "launches_per_step": 1}}
    adm, rej = 768.0, 100.0
    v = bench.vocab_passes(wl, kern, adm, rej)
    s, V, r, B = 2, wl.V, wl.r, wl.B
    tile_b, _ = bench.draft_tiles_bytes_flops(wl)
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
