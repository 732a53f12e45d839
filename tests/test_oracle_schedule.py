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


# ----------------------------------------------------------------------------- objective-based admission
UNIT = 2**36


def _objective_brute(theta, t, max_admit):
    """The admission rule written with exact rationals: candidates in the order
    (Theta desc, request asc, position asc); admit while
    E(m+1) / t[B+m+1] >= E(m) / t[B+m], E in units of 2^-36 (each term
    floor(clamp(Theta) * 2^36)), every request contributing 1."""
    from fractions import Fraction
    B, gamma = theta.shape
    order = sorted(((float(theta[b, k]), b, k) for b in range(B) for k in range(gamma)),
                   key=lambda c: (-c[0], c[1], c[2]))
    cap = min(max_admit, B * gamma)
    E = B * UNIT
    m = 0
    while m < cap:
        th = min(max(order[m][0], 0.0), 1.0)
        E1 = E + int(Fraction(th) * UNIT)  # floor for non-negative values
        if Fraction(E1) / Fraction(float(t[B + m + 1])) < Fraction(E) / Fraction(float(t[B + m])):
            break
        E = E1
        m += 1
    adm = np.zeros((B, gamma), dtype=bool)
    for i in range(m):
        adm[order[i][1], order[i][2]] = True
    ln = np.array([next((k for k in range(gamma) if not adm[b, k]), gamma) for b in range(B)], dtype=np.int32)
    return ln, m


def test_objective_appendix_a_early_stop():
    """Appendix A of the paperlayer.ai summary: without early stopping the
    length chosen for the first draft depends on c_2 (length 2 when the
    continuation is confident, 0 otherwise); with early stopping the scan ends
    before c_2 matters.  The capacity curve is an instance chosen here (the
    page gives none) with J(1) < J(0) and, for c_2 = 0.9, J(2) > J(0)."""
    from fractions import Fraction
    with open(os.path.join(os.path.dirname(__file__), "golden", "appendix_a.json")) as f:
        fx = json.load(f)["facts_from_the_page"]
    a1 = fx["first_position_acceptance_a1"]
    t = np.array([0.0, 1.0, 1.9, 2.0], dtype=np.float32)  # t[n]: n = 1 + admitted (one request)
    global_best = {}
    for c2 in (fx["c2_high_confidence"], fx["c2_low_confidence"]):
        th = np.array([[a1, np.float32(a1) * np.float32(c2)]], dtype=np.float32)
        ln, m = oracle.select_objective(th, t, 2)
        assert ln.tolist() == [0] and m == 0
        # the search over every prefix length that the page shows to be biased
        J = [(1 + sum(Fraction(float(x)) for x in th[0, :l])) / Fraction(float(t[1 + l])) for l in range(3)]
        global_best[c2] = max(range(3), key=lambda l: J[l])
    assert global_best == {fx["c2_high_confidence"]: 2, fx["c2_low_confidence"]: 0}


@pytest.mark.parametrize("seed", range(12))
def test_objective_matches_exact_rule(seed):
    g = np.random.default_rng(100 + seed)
    B, gamma = int(g.integers(1, 7)), int(g.integers(1, 6))
    z = (g.standard_normal((B, gamma)) * 2).astype(np.float32)
    if seed % 3 == 0:
        z[:, :] = z[0, 0]  # equal survivals across requests
    theta = oracle.survival(z, (1.0 + 0.2 * np.arange(1, gamma + 1)).astype(np.float32))
    n = B + B * gamma + 1
    kind = seed % 4
    if kind == 0:    # concave: fixed cost plus a per-token cost
        t = (3.0 + 0.05 * np.arange(n)).astype(np.float32)
    elif kind == 1:  # irregular: steps every 4 tokens
        t = (1.0 + 0.5 * (np.arange(n) // 4) + 0.01 * np.arange(n)).astype(np.float32)
    elif kind == 2:  # random increasing
        t = np.cumsum(g.uniform(0.01, 1.0, n)).astype(np.float32)
    else:            # random, not monotone
        t = g.uniform(0.5, 2.0, n).astype(np.float32)
    for cap in (0, 1, B * gamma // 2, B * gamma, 10 * B * gamma):
        ln, m = oracle.select_objective(theta, t, cap)
        ref_ln, ref_m = _objective_brute(theta, t, cap)
        assert m == ref_m and ln.tolist() == ref_ln.tolist(), (kind, cap)
        assert int(ln.sum()) == m


def test_objective_linear_profile_admits_only_certain_tokens():
    """t[n] proportional to n: J(m) is the mean of 1 (per request) and the
    admitted Theta, so a candidate with Theta < 1 lowers it; Theta = 1 keeps
    it equal, which does not stop the scan."""
    theta = np.array([[1.0, 1.0, 0.9], [1.0, 0.99, 0.5], [0.7, 0.6, 0.1]], dtype=np.float32)
    t = (0.25 * np.arange(3 + 9 + 1)).astype(np.float32)
    ln, m = oracle.select_objective(theta, t, 9)
    assert ln.tolist() == [2, 1, 0] and m == 3


@pytest.mark.parametrize("K", [0, 1, 5, 17, 40])
def test_objective_flat_then_prohibitive_equals_budget(K):
    """A profile flat up to B + K tokens and prohibitive after it admits the
    K best candidates: the budget form with budget K (and a flat profile
    with cap K too)."""
    g = np.random.default_rng(7)
    B, gamma = 8, 5
    theta = oracle.survival((g.standard_normal((B, gamma)) * 2).astype(np.float32),
                            np.ones(gamma, dtype=np.float32))
    n = B + B * gamma + 1
    t = np.where(np.arange(n) <= B + K, 1.0, 1e30).astype(np.float32)
    ln, m = oracle.select_objective(theta, t, B * gamma)
    assert ln.tolist() == oracle.select(theta, K).tolist() and m == min(K, B * gamma)
    ln2, m2 = oracle.select_objective(theta, np.ones(n, dtype=np.float32), K)
    assert ln2.tolist() == oracle.select(theta, K).tolist() and m2 == min(K, B * gamma)


def test_objective_clamps_and_errors():
    theta = np.array([[1.5, -0.25]], dtype=np.float32)  # given survivals outside [0, 1]
    t = np.ones(4, dtype=np.float32)
    ln, m = oracle.select_objective(theta, t, 2)
    assert ln.tolist() == [2] and m == 2
    with pytest.raises(RuntimeError):
        oracle.select_objective(theta, np.ones(2, dtype=np.float32), 2)  # profile too short
    with pytest.raises(RuntimeError):
        oracle.select_objective(theta, t, -1)


def test_threshold_constructed_cases():
    """Static-threshold admission (paperlayer.ai summary, section 4.3) on rows whose answers are fixed in
    advance: a survival equal to tau is verified (>=), a NaN ends the run, and on non-monotone given
    survivals only the leading run counts (later positions above tau stay unverified)."""
    nan = np.float32(np.nan)
    f = np.float32
    below = np.nextafter(f(0.3), f(0))  # the largest float32 under 0.3
    theta = np.array([
        [0.9, 0.5, 0.3, 0.1],       # 0.3 == tau counts: 3
        [0.3, 0.3, 0.2, 0.2],       # ties at tau: 2
        [0.8, nan, 0.9, 0.9],       # NaN mid-row ends the run: 1
        [nan, 1.0, 1.0, 1.0],       # NaN first: 0
        [below, below, 0.0, 0.0],   # one ulp under tau: 0
        [0.5, 0.2, 0.6, 0.7],       # not monotone: only the leading run, 1
        [1.0, 1.0, 1.0, 1.0],       # 4
        [-0.0, 0.0, -0.0, 0.0],     # signed zeros: 0 (and all 4 at tau = 0)
    ], dtype=np.float32)
    assert oracle.select_threshold(theta, f(0.3)).tolist() == [3, 2, 1, 0, 0, 1, 4, 0]
    assert oracle.select_threshold(theta, f(0.0)).tolist() == [4, 4, 1, 0, 4, 4, 4, 4]
    assert oracle.select_threshold(theta, f(1.0)).tolist() == [0, 0, 0, 0, 0, 0, 4, 0]
    assert oracle.select_threshold(theta, below).tolist() == [3, 2, 1, 0, 2, 1, 4, 0]
    assert oracle.select_threshold(theta, nan).tolist() == [0] * 8  # no comparison with NaN holds
    # monotone survivals: the run is the number of positions at or above tau
    g = np.random.default_rng(3)
    th2 = oracle.survival((g.standard_normal((20, 5))).astype(np.float32), np.ones(5, dtype=np.float32))
    assert oracle.select_threshold(th2, 0.2).tolist() == (th2 >= np.float32(0.2)).sum(1).tolist()


# ----------------------------------------------------------------------------- Markov-conditioned confidence
def test_markov_confidence_one_hot_codes_select_weights():
    """With one-hot conditioning codes A[x] = e_{x mod r}, z[b][k] = z0[b][k] + wc[x_{k-1} mod r] exactly."""
    V, r, B, gamma = 12, 8, 3, 4
    A = np.zeros((V, r), dtype=np.float32)
    A[np.arange(V), np.arange(V) % r] = 1.0
    wc = np.arange(1, r + 1, dtype=np.float32) * 0.5
    x0 = np.array([3, 11, 0], dtype=np.int32)
    tok = np.array([[1, 2, 9, 4], [5, 5, 5, 5], [7, 0, 10, 6]], dtype=np.int32)
    z0 = np.array([[0.25, -1.0, 2.0, 0.0], [1.5, 1.5, -0.5, 3.0], [0.0, 0.125, 0.0, -2.0]], dtype=np.float32)
    z = oracle.markov_confidence(A, wc, x0, tok, z0)
    prev = np.concatenate([x0[:, None], tok[:, :-1]], axis=1)
    assert np.array_equal(z, z0 + wc[prev % r])


def test_markov_confidence_integer_exact_and_depends_on_previous_token():
    """Small-integer codes: the dot product is exact; z_k changes with x_{k-1}
    and with nothing later (Appendix A: c_2 depends on x_1)."""
    g = np.random.default_rng(5)
    V, r, B, gamma = 50, 24, 4, 5
    A = g.integers(-3, 4, (V, r)).astype(np.float32)
    wc = g.integers(-2, 3, r).astype(np.float32)
    x0 = g.integers(0, V, B).astype(np.int32)
    tok = g.integers(0, V, (B, gamma)).astype(np.int32)
    z0 = g.integers(-5, 6, (B, gamma)).astype(np.float32)
    z = oracle.markov_confidence(A, wc, x0, tok, z0)
    ref = np.empty((B, gamma), dtype=np.int64)
    for b in range(B):
        for k in range(gamma):
            x = x0[b] if k == 0 else tok[b, k - 1]
            ref[b, k] = int(z0[b, k]) + int(A[x].astype(np.int64) @ wc.astype(np.int64))
    assert np.array_equal(z.astype(np.int64), ref)
    tok2 = tok.copy()
    tok2[:, 0] = (tok[:, 0] + 1) % V  # change x_1 only
    z2 = oracle.markov_confidence(A, wc, x0, tok2, z0)
    assert np.array_equal(z2[:, 0], z[:, 0]) and np.array_equal(z2[:, 2:], z[:, 2:])
    moved = (A[tok[:, 0]] @ wc) != (A[tok2[:, 0]] @ wc)
    assert np.array_equal(z2[:, 1] != z[:, 1], moved)
