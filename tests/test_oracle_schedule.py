"""Pins for the oracle's survival product and budget selection (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle


def test_survival_zero_logits_is_exact_halving():
    z = np.zeros((3, 6), dtype=np.float32)
    T = np.array([1.0, 1.1, 1.2, 1.3, 1.4, 1.5], dtype=np.float32)
    th = oracle.survival(z, T)
    expect = np.array([0.5 ** k for k in range(1, 7)], dtype=np.float32)
    assert np.array_equal(th, np.broadcast_to(expect, th.shape))


def test_survival_large_temperature_tends_to_half():
    z = np.full((2, 3), 5.0, dtype=np.float32)
    T = np.full(3, 1e30, dtype=np.float32)
    th = oracle.survival(z, T)
    assert np.array_equal(th[0], np.array([0.5, 0.25, 0.125], dtype=np.float32))


def test_survival_closed_form_against_library_sigmoid():
    g = np.random.default_rng(0)
    z = (g.standard_normal((64, 8)) * 3).astype(np.float32)
    T = (1.0 + 0.1 * np.arange(1, 9)).astype(np.float32)
    th = oracle.survival(z, T).astype(np.float64)
    zt = torch.from_numpy(z).double() / torch.from_numpy(T).double()
    ref = torch.cumprod(torch.sigmoid(zt), 1).numpy()
    # each float op adds at most half an ulp; 3 ops per position plus the product chain
    assert np.allclose(th, ref, rtol=4 * 8 * 2**-24, atol=0)


def test_survival_non_increasing():
    g = np.random.default_rng(1)
    z = (g.standard_normal((200, 16)) * 4 - 1).astype(np.float32)
    T = np.linspace(0.5, 3, 16).astype(np.float32)
    th = oracle.survival(z, T)
    assert np.all(np.diff(th, axis=1) <= 0)
    assert np.all(th[:, 0] <= 1.0) and np.all(th >= 0)


def _lexsort_reference(theta, budget):
    B, gamma = theta.shape
    idx_b, idx_k = np.meshgrid(np.arange(B), np.arange(gamma), indexing="ij")
    order = np.lexsort((idx_k.ravel(), idx_b.ravel(), -theta.astype(np.float64).ravel()))
    adm = np.zeros(B * gamma, dtype=bool)
    adm[order[:min(budget, B * gamma)]] = True
    return adm.reshape(B, gamma).sum(1)


def _rand_theta(g, B, gamma, ties=False):
    z = (g.standard_normal((B, gamma)) * 2 + 0.5).astype(np.float32)
    if ties:
        z = np.round(z)  # many equal survivals
    T = np.ones(gamma, dtype=np.float32)
    return oracle.survival(z, T)


@pytest.mark.parametrize("ties", [False, True])
def test_select_matches_lexsort_and_budget(ties):
    g = np.random.default_rng(2)
    for trial in range(40):
        B, gamma = int(g.integers(1, 40)), int(g.integers(1, 9))
        th = _rand_theta(g, B, gamma, ties)
        for budget in (0, 1, B, B * gamma // 2, B * gamma - 1, B * gamma, B * gamma + 7):
            ln = oracle.select(th, budget)
            assert ln.sum() == min(budget, B * gamma)
            assert np.array_equal(ln, _lexsort_reference(th, budget))


def test_select_extremes_and_errors():
    th = _rand_theta(np.random.default_rng(3), 5, 4)
    assert np.all(oracle.select(th, 0) == 0)
    assert np.all(oracle.select(th, 20) == 4)
    assert np.all(oracle.select(th, 10**12) == 4)
    with pytest.raises(RuntimeError):
        oracle.select(th, -1)


def test_select_is_optimal_among_prefix_sets():
    """Brute force over every verify-length vector with the same total."""
    g = np.random.default_rng(4)
    for trial in range(30):
        B, gamma = int(g.integers(1, 5)), int(g.integers(1, 5))
        th = _rand_theta(g, B, gamma).astype(np.float64)
        cum = np.concatenate([np.zeros((B, 1)), np.cumsum(th, 1)], 1)
        for budget in range(0, B * gamma + 1):
            ln = oracle.select(th.astype(np.float32), budget)
            got = sum(cum[b, ln[b]] for b in range(B))
            best = max(sum(cum[b, v[b]] for b in range(B))
                       for v in itertools.product(range(gamma + 1), repeat=B) if sum(v) == budget)
            assert got == pytest.approx(best, rel=1e-12, abs=1e-300)


def test_select_non_anticipating():
    """Changing survivals after position k never changes whether (b, k) is admitted."""
    g = np.random.default_rng(5)
    for trial in range(200):
        B, gamma = int(g.integers(1, 12)), int(g.integers(2, 8))
        th = _rand_theta(g, B, gamma)
        budget = int(g.integers(0, B * gamma + 1))
        ln = oracle.select(th, budget)
        b, k = int(g.integers(0, B)), int(g.integers(0, gamma - 1))
        th2 = th.copy()
        # any non-increasing continuation below Theta_{b,k}
        th2[b, k + 1:] = np.sort(g.uniform(0, th[b, k], gamma - k - 1).astype(np.float32))[::-1]
        ln2 = oracle.select(th2, budget)
        assert (ln[b] > k) == (ln2[b] > k)


def test_select_equal_survivals_break_by_request_then_position():
    th = np.full((3, 2), 0.5, dtype=np.float32)
    th[:, 1] = 0.5  # all six equal
    assert oracle.select(th, 1).tolist() == [1, 0, 0]
    assert oracle.select(th, 3).tolist() == [2, 1, 0]
    # -0.0 and +0.0 compare equal: ties again by request order
    th0 = np.array([[-0.0], [0.0]], dtype=np.float32)
    assert oracle.select(th0, 1).tolist() == [1, 0]


def test_select_rejects_nan():
    th = np.array([[0.5, np.nan]], dtype=np.float32)
    with pytest.raises(RuntimeError):
        oracle.select(th, 1)


def test_appendix_a_early_stop_reading():
    """Appendix A: with Theta_1 < Theta_0 = 1 the early-stopping scheduler
    returns length 0 before looking at c_2; the budget form never looks at a
    later position to decide an earlier one (covered by the test above).  Here:
    a one-request budget of 1 admits position 1 regardless of c_2."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "appendix_a.json")) as f:
        fx = json.load(f)
    a1 = fx["facts_from_the_page"]["first_position_acceptance_a1"]
    for c2 in (fx["facts_from_the_page"]["c2_high_confidence"], fx["facts_from_the_page"]["c2_low_confidence"]):
        th = np.array([[a1, a1 * c2]], dtype=np.float32)
        assert oracle.select(th, 1).tolist() == [1]
        assert oracle.select(th, 0).tolist() == [0]
