"""Pins for the oracle's inverse-CDF sampler and Markov draft (CPU only)."""
import math

import numpy as np
import pytest
import torch
from scipy import stats

import oracle


def _exact_preimage_counts(w):
    """Grid points i in [0, 2^24) mapped to each token, from exact rationals.

    token j owns u = i/2^24 with C_{j-1} <= u*S < C_j (strict CDF rule), so its
    count is ceil(2^24 C_j / S) - ceil(2^24 C_{j-1} / S).
    """
    from fractions import Fraction
    wf = [Fraction(x) for x in w]
    S = sum(wf)
    counts = []
    c_prev = Fraction(0)
    for x in wf:
        c = c_prev + x
        hi = math.ceil(c / S * 2**24)
        lo = math.ceil(c_prev / S * 2**24)
        counts.append(hi - lo)
        c_prev = c
    return counts


@pytest.mark.parametrize("w", [
    [3 / 16, 1 / 16, 0.0, 4 / 16, 8 / 16],
    [1.0, 1.0, 1.0],
    [0.0, 5.0, 0.0, 0.0, 3.0, 0.0],
    [2.0**-10, 1.0, 2.0**-20, 0.5],
])
def test_inverse_cdf_brute_force_whole_grid(w):
    us = (np.arange(2**24, dtype=np.float64) / 2**24).astype(np.float32)
    toks = oracle.inverse_cdf_batch(np.array(w), us)
    got = np.bincount(toks, minlength=len(w)).tolist()
    assert got == _exact_preimage_counts(w)
    # zero-weight tokens are never drawn
    for j, x in enumerate(w):
        if x == 0.0:
            assert got[j] == 0


def test_inverse_cdf_boundaries_are_strict():
    w = np.array([1.0, 1.0, 2.0])  # C = 1, 2, 4 ; S = 4
    assert oracle.inverse_cdf(w, 0.0) == 0
    assert oracle.inverse_cdf(w, 0.25) == 1    # tau = 1 = C_0, not > C_0 -> next token
    assert oracle.inverse_cdf(w, 0.5) == 2     # tau = 2 = C_1
    assert oracle.inverse_cdf(w, 0.9999999) == 2


def _rand_problem(V, r, seed, scale_a=0.02):
    g = np.random.default_rng(seed)
    L = (g.standard_normal(V) * 2).astype(np.float32)
    A = (g.standard_normal((V, r)) * scale_a).astype(np.float32)
    Bm = (g.standard_normal((r, V)) * scale_a).astype(np.float32)
    return L, A, Bm


def test_draft_row_with_zero_bias_is_softmax():
    V, r = 1000, 16
    L, A, Bm = _rand_problem(V, r, 1)
    A[:] = 0.0
    o = oracle.draft_row(L, A, Bm, prev=5, u=0.37)
    ls = torch.log_softmax(torch.from_numpy(L).double(), 0)
    assert o["lse"] == pytest.approx(torch.logsumexp(torch.from_numpy(L).double(), 0).item(), rel=1e-14, abs=1e-12)
    assert o["p"] == pytest.approx(math.exp(ls[o["tok"]].item()), rel=1e-12)
    # the token is the inverse-CDF point of the library softmax
    cdf = torch.cumsum(ls.exp(), 0).numpy()
    assert cdf[o["tok"]] > 0.37 * cdf[-1] - 1e-12
    if o["tok"] > 0:
        assert cdf[o["tok"] - 1] <= 0.37 * cdf[-1] + 1e-12


def test_markov_logits_one_hot_rows_select_bm_rows():
    V, r = 64, 8
    L, A, Bm = _rand_problem(V, r, 2)
    A[:] = 0.0
    for prev, i in [(0, 0), (7, 5), (63, 7)]:
        A[prev, i] = 1.0
        f = oracle.markov_logits(L, A, Bm, prev)
        assert np.array_equal(f, L.astype(np.float64) + Bm[i].astype(np.float64))
        A[prev, i] = 0.0


def test_markov_logits_small_integers_exact():
    g = np.random.default_rng(3)
    V, r = 200, 256
    A = g.integers(-8, 9, size=(V, r)).astype(np.float32)
    Bm = g.integers(-8, 9, size=(r, V)).astype(np.float32)
    L = g.integers(-100, 100, size=V).astype(np.float32)
    for prev in (0, 17, 199):
        f = oracle.markov_logits(L, A, Bm, prev)
        ref = L.astype(np.int64) + A[prev].astype(np.int64) @ Bm.astype(np.int64)
        assert np.array_equal(f, ref.astype(np.float64))


def test_markov_logits_transposition_would_fail():
    # A non-symmetric case where A[prev] . Bm differs from Bm[:, prev] . A^T etc.
    V, r = 6, 3
    A = np.arange(V * r, dtype=np.float32).reshape(V, r)
    Bm = (np.arange(r * V, dtype=np.float32).reshape(r, V) * 0.5)
    L = np.zeros(V, dtype=np.float32)
    f = oracle.markov_logits(L, A, Bm, 4)
    assert np.array_equal(f, (A[4].astype(np.float64) @ Bm.astype(np.float64)))


def test_draft_chi_square_v8():
    """10^6 draws at V=8: x_k given x_{k-1} follows softmax(L_k + A[x_{k-1}] Bm)."""
    V, r, gamma, B = 8, 8, 8, 125000
    g = np.random.default_rng(4)
    Lk = (g.standard_normal((gamma, V)) * 1.5).astype(np.float32)
    A = (g.standard_normal((V, r)) * 0.5).astype(np.float32)
    Bm = (g.standard_normal((r, V)) * 0.5).astype(np.float32)
    L = np.broadcast_to(Lk, (B, gamma, V)).copy()
    x0 = g.integers(0, V, size=B).astype(np.int32)
    tok, p, lse = oracle.markov_draft(L, A, Bm, x0, seed=99)
    prev = np.concatenate([x0[:, None], tok[:, :-1]], axis=1)
    At, Bt, Lt = (torch.from_numpy(x).double() for x in (A, Bm, Lk))
    worst = 1.0
    for k in range(gamma):
        for pv in range(V):
            sel = prev[:, k] == pv
            n = int(sel.sum())
            if n < 200:
                continue
            probs = torch.softmax(Lt[k] + At[pv] @ Bt, 0).numpy()
            obs = np.bincount(tok[sel, k], minlength=V)
            pv_ = stats.chisquare(obs, probs * n).pvalue
            worst = min(worst, pv_)
            # reported p_d equals the model probability of the drawn token
            drawn = tok[sel, k]
            assert np.allclose(p[sel, k], probs[drawn], rtol=1e-6)
    # 64 tests: Bonferroni-style threshold
    assert worst > 1e-4 / 64


def test_logsumexp_matches_library():
    g = np.random.default_rng(5)
    row = (g.standard_normal(129280) * 2).astype(np.float32)
    ref = torch.logsumexp(torch.from_numpy(row).double(), 0).item()
    assert oracle.logsumexp(row) == pytest.approx(ref, rel=1e-14)


# ----------------------------------------------------------------------------- RNN head state update
def test_rnn_state_zero_weights_is_tanh_of_code():
    a = np.array([0.0, 0.5, -1.25, 3.0], dtype=np.float32)
    out = oracle.rnn_state(np.zeros((4, 4), dtype=np.float32), np.ones(4, dtype=np.float32), a)
    # tanh(0) = 0 exactly; tanh is odd; |tanh(x)| < 1; tanh(x) ~ x - x^3/3 near 0
    assert out[0] == 0.0 and abs(out[1] - (0.5 - 0.5**3 / 3 + 2 * 0.5**5 / 15)) < 0.5**7 * 17 / 315 + 1e-12
    assert np.array_equal(oracle.rnn_state(np.zeros((4, 4), np.float32), np.ones(4, np.float32), -a), -out)
    assert np.all(np.abs(out) < 1.0)


def test_rnn_state_one_hot_state_selects_a_column_of_w():
    """h_prev = e_j: the pre-activation is W[:, j] + a = Wt[j, :] + a (a transposed W would give Wt[:, j])."""
    g = np.random.default_rng(11)
    r = 6
    Wt = g.integers(-2, 3, (r, r)).astype(np.float32)
    a = g.integers(-1, 2, r).astype(np.float32)
    for j in range(r):
        h = np.zeros(r, dtype=np.float32)
        h[j] = 1.0
        out = oracle.rnn_state(Wt, h, a)
        pre = Wt[j].astype(np.float64) + a
        assert np.array_equal(np.round(np.arctanh(np.clip(out, -1 + 1e-15, 1 - 1e-15)), 9), np.round(pre, 9))


def test_rnn_state_diagonal_weights_act_elementwise():
    d = np.array([0.5, -2.0, 1.0, 0.0], dtype=np.float32)
    h = np.array([1.0, 0.25, -0.5, 7.0], dtype=np.float32)
    a = np.array([0.0, 0.5, 0.5, -0.25], dtype=np.float32)
    out = oracle.rnn_state(np.diag(d), h, a)
    pre = d.astype(np.float64) * h + a
    # tanh(x) = (e^{2x} - 1) / (e^{2x} + 1)
    assert np.allclose(out, (np.exp(2 * pre) - 1) / (np.exp(2 * pre) + 1), rtol=0, atol=1e-15)
