"""Sequential temperature scaling and the calibration error (host tooling,
draft_verify_sampling_prev_amd/calibration.py), pinned by a hand-computed ECE,
its limits, agreement of the survival product with the oracle's, and the
recovery of planted per-position temperatures."""
import numpy as np
import pytest

import oracle
from draft_verify_sampling_prev_amd import calibration as cal
from draft_verify_sampling_prev_amd import synth


def test_ece_hand_computed():
    # 15 bins: 0.1 -> bin 1, 0.15 -> bin 2, 0.9 -> bin 13, 0.95 -> bin 14; one sample each
    assert cal.ece([0.1, 0.15, 0.9, 0.95], [0, 1, 1, 1]) == pytest.approx((0.1 + 0.85 + 0.1 + 0.05) / 4)
    # two samples sharing a bin are averaged before the difference is taken
    assert cal.ece([0.5, 0.52], [1, 0]) == pytest.approx(abs(0.5 - 0.51))
    # confidence 1 falls in the last (closed) bin; confidence 0 in the first
    assert cal.ece([1.0, 0.0], [1, 0]) == 0.0
    assert cal.ece([], []) == 0.0


def test_ece_limits():
    g = np.random.default_rng(1)
    c = g.uniform(0, 1, 400000)
    y = (g.uniform(0, 1, c.size) < c).astype(float)   # calibrated by construction
    assert cal.ece(c, y) < 0.01
    assert cal.ece(c, 1 - y) > 0.3                      # anti-calibrated
    assert cal.ece(np.full(1000, 0.7), np.r_[np.ones(700), np.zeros(300)]) == pytest.approx(0.0, abs=1e-12)


def test_survival_matches_the_oracle_product():
    g = np.random.default_rng(2)
    z = (g.standard_normal((500, 6)) * 2).astype(np.float32)
    t = np.array([0.5, 1.0, 1.3, 2.0, 4.0, 9.0], dtype=np.float32)
    assert np.allclose(cal.survival(z, t), oracle.survival(z, t), rtol=2e-6, atol=1e-37)


def test_survival_labels():
    assert cal.survival_labels([0, 2, 3], 3).tolist() == [[0, 0, 0], [1, 1, 0], [1, 1, 1]]


def test_fit_recovers_planted_temperatures():
    """Labels drawn from a prefix-survival process with known temperatures: s_k = s_{k-1} and
    Bernoulli(sigmoid(z_k / T*_k)).  The left-to-right fit recovers each T*_k (the later ones only because
    the fit multiplies onto the earlier positions' fitted survival)."""
    g = np.random.default_rng(3)
    n, t_true = 200000, np.array([0.7, 1.6, 3.0], dtype=np.float32)
    z = (g.normal(1.0, 1.5, (n, 3))).astype(np.float32)
    c = 1.0 / (1.0 + np.exp(-(z / t_true[None, :])))
    s = np.cumprod(g.uniform(0, 1, (n, 3)) < c, axis=1).astype(float)
    temps, errs = cal.fit_sts(z, s)
    assert np.allclose(temps, t_true, rtol=0.08), temps
    assert np.all(errs < 0.01)
    # the fitted product is calibrated where a fixed temperature of 1 is not
    base = cal.survival(z, np.ones(3, dtype=np.float32))
    assert all(cal.ece(base[:, k], s[:, k]) > 3 * errs[k] for k in range(3))


def test_fit_when_confidence_is_uninformative():
    """When z carries no information about acceptance (the synthetic workloads' case) a per-position
    temperature can only move the survivals towards the marginal survival rates: the fitted ECE is below that
    of temperature 1 at every position, and the mean survival lands near the marginal rate."""
    g = np.random.default_rng(4)
    n = 100000
    z = g.normal(2.0, 1.0, (n, 4)).astype(np.float32)
    s = np.cumprod(g.uniform(0, 1, (n, 4)) < np.array([0.8, 0.7, 0.6, 0.5]), axis=1).astype(float)
    temps, errs = cal.fit_sts(z, s)
    th = cal.survival(z, temps)
    base = cal.survival(z, np.ones(4, dtype=np.float32))
    for k in range(4):
        assert errs[k] == pytest.approx(cal.ece(th[:, k], s[:, k]))
        assert errs[k] < cal.ece(base[:, k], s[:, k])
    assert np.allclose(th.mean(0), s.mean(0), atol=0.05)


def test_workload_temperatures_are_positive_and_complete():
    wl = synth.load_sweep(1024)
    assert len(wl.temps) == wl.gamma and all(t > 0 for t in wl.temps)


def test_workload_constants_match_the_calibration_record():
    """synth's calibrated constants are the ones tests/calibrate_workloads.py wrote on the held-out seeds."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "workload_calibration.json")) as f:
        rec = json.load(f)
    assert tuple(rec["dsv4"]["sigma"]) == synth.DSV4_SIGMA == synth.dsv4().sigma
    assert rec["dsv4"]["held_out_seed"] == synth.dsv4().data_seed + 8000
    assert max(abs(a - t) for a, t in zip(rec["dsv4"]["expected_alpha"], rec["dsv4"]["target_alpha"])) < 2e-3
    assert tuple(rec["load_sweep"]["temps"]) == synth.LOAD_SWEEP_STS == synth.load_sweep(1024).temps
    assert all(a <= b + 1e-12 for a, b in zip(rec["load_sweep"]["ece_after"], rec["load_sweep"]["ece_before"]))
