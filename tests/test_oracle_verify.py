"""Pins for the oracle's rejection-sampling verification (CPU only).

The pages fix the law of the output, not its realisation: every emitted token
must be distributed as the target's p_t at its position (exactness of the
acceptance rule), and with a draft that ignores its context the number of
accepted tokens follows the textbook 1 - TV acceptance rate.
"""
import json
import os

import numpy as np
import pytest
import torch
from scipy import stats

import oracle

SEED = 0x0123456789ABCDEF


def _softmax64(x):
    return torch.softmax(torch.from_numpy(np.asarray(x, dtype=np.float32)).double(), -1).numpy()


def _problem(B, gamma, V, r, g, t_scale=1.5, d_scale=1.5, a_scale=0.5):
    Tk = (g.standard_normal((gamma + 1, V)) * t_scale).astype(np.float32)
    Lk = (g.standard_normal((gamma, V)) * d_scale).astype(np.float32)
    A = (g.standard_normal((V, r)) * a_scale).astype(np.float32)
    Bm = (g.standard_normal((r, V)) * a_scale).astype(np.float32)
    T = np.broadcast_to(Tk, (B, gamma + 1, V)).copy()
    L = np.broadcast_to(Lk, (B, gamma, V)).copy()
    x0 = g.integers(0, V, size=B).astype(np.int32)
    return Tk, T, L, A, Bm, x0


def _emitted_by_position(out, n_out, gamma):
    res = []
    for k in range(gamma + 1):
        sel = n_out > k
        res.append(out[sel, k])
    return res


@pytest.mark.parametrize("ell_mode", ["full", "mixed"])
def test_emitted_tokens_follow_target_chi_square(ell_mode):
    """V=8, about 10^6 emitted tokens: token at position k ~ p_t,k given it is emitted."""
    g = np.random.default_rng(10)
    B, gamma, V, r = 700000, 3, 8, 8
    Tk, T, L, A, Bm, x0 = _problem(B, gamma, V, r, g)
    tok, pd, _ = oracle.markov_draft(L, A, Bm, x0, SEED)
    if ell_mode == "full":
        ell = np.full(B, gamma, dtype=np.int32)
    else:
        ell = (np.arange(B) % (gamma + 1)).astype(np.int32)
    acc, out, n_out, tp = oracle.verify(T, L, A, Bm, x0, tok, pd, ell, SEED)
    assert np.all(n_out == acc + 1) and np.all(acc <= ell)
    total = 0
    for k, toks in enumerate(_emitted_by_position(out, n_out, gamma)):
        if toks.size < 1000:
            continue
        total += toks.size
        p = _softmax64(Tk[k])
        pval = stats.chisquare(np.bincount(toks, minlength=V), p * toks.size).pvalue
        assert pval > 1e-4, (k, pval)
    assert total > 1e6 if ell_mode == "full" else total > 5e5


def test_accept_count_matches_textbook_rate_for_context_free_draft():
    """A = 0: acceptance at position j is alpha_j = sum_x min(p_t, p_d) independently,
    so E[a | ell] = sum_{k<=ell} prod_{j<=k} alpha_j."""
    g = np.random.default_rng(11)
    B, gamma, V, r = 60000, 4, 8, 8
    Tk, T, L, A, Bm, x0 = _problem(B, gamma, V, r, g, d_scale=1.0)
    A[:] = 0.0
    tok, pd, _ = oracle.markov_draft(L, A, Bm, x0, SEED)
    ell = np.full(B, gamma, dtype=np.int32)
    acc, out, n_out, tp = oracle.verify(T, L, A, Bm, x0, tok, pd, ell, SEED)
    alpha = np.array([np.minimum(_softmax64(Tk[j]), _softmax64(L[0, j])).sum() for j in range(gamma)])
    surv = np.cumprod(alpha)
    mean = surv.sum()
    # Var of a = sum_k P(a>=k) - mean^2 + 2 sum_{j<k} P(a>=k)
    pk = surv
    e2 = sum((2 * k + 1) * pk[k] for k in range(gamma))
    var = e2 - mean**2
    assert abs(acc.mean() - mean) < 4 * np.sqrt(var / B)
    # per-position survival frequencies as well
    for k in range(gamma):
        freq = (acc > k).mean()
        assert abs(freq - pk[k]) < 4 * np.sqrt(pk[k] * (1 - pk[k]) / B)


def test_identical_distributions_accept_everything():
    g = np.random.default_rng(12)
    B, gamma, V, r = 2000, 4, 50, 4
    Tk, T, L, A, Bm, x0 = _problem(B, gamma, V, r, g)
    A[:] = 0.0
    L = T[:, :gamma, :].copy()
    tok, pd, _ = oracle.markov_draft(L, A, Bm, x0, SEED)
    ell = (np.arange(B) % (gamma + 1)).astype(np.int32)
    acc, out, n_out, tp = oracle.verify(T, L, A, Bm, x0, tok, pd, ell, SEED)
    assert np.array_equal(acc, ell)


def test_disjoint_supports_reject_first_token_and_resample_target():
    g = np.random.default_rng(13)
    B, gamma, V, r = 20000, 3, 8, 4
    Tk, T, L, A, Bm, x0 = _problem(B, gamma, V, r, g)
    A[:] = 0.0
    L[:, :, 4:] = -1.0e4   # draft only proposes tokens 0..3
    T[:, :, :4] = -1.0e4   # target only allows tokens 4..7
    Tk = T[0]
    tok, pd, _ = oracle.markov_draft(L, A, Bm, x0, SEED)
    assert np.all(tok < 4)
    ell = np.full(B, gamma, dtype=np.int32)
    acc, out, n_out, tp = oracle.verify(T, L, A, Bm, x0, tok, pd, ell, SEED)
    assert np.all(acc == 0) and np.all(n_out == 1)
    first = out[:, 0]
    assert np.all(first >= 4)
    pval = stats.chisquare(np.bincount(first, minlength=V)[4:], _softmax64(Tk[0])[4:] * B).pvalue
    assert pval > 1e-4


def test_zero_length_emits_fresh_target_token():
    """Appendix A: a request with verify length 0 gets one token from p_t of position 1."""
    g = np.random.default_rng(14)
    B, gamma, V, r = 100000, 3, 8, 4
    Tk, T, L, A, Bm, x0 = _problem(B, gamma, V, r, g)
    tok, pd, _ = oracle.markov_draft(L, A, Bm, x0, SEED)
    ell = np.zeros(B, dtype=np.int32)
    acc, out, n_out, tp = oracle.verify(T, L, A, Bm, x0, tok, pd, ell, SEED)
    assert np.all(acc == 0) and np.all(n_out == 1)
    assert np.all(out[:, 1:] == -1)
    pval = stats.chisquare(np.bincount(out[:, 0], minlength=V), _softmax64(Tk[0]) * B).pvalue
    assert pval > 1e-4


def test_appendix_a_anticipation_biases_the_output():
    """The counterexample of Appendix A on a V=2 instance: choosing the verify length
    after seeing x_1 gives P(first token = A) = 0.45; a length fixed before x_1 gives p_t(A) = 0.3."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "appendix_a.json")) as f:
        fx = json.load(f)["instance_chosen_here"]
    pd_, pt_ = np.array(fx["p_d"]), np.array(fx["p_t"])
    B, gamma, V, r = 200000, 2, 2, 1
    T = np.broadcast_to(np.log(pt_).astype(np.float32), (B, gamma + 1, V)).copy()
    L = np.broadcast_to(np.log(pd_).astype(np.float32), (B, gamma, V)).copy()
    A = np.zeros((V, r), dtype=np.float32)
    Bm = np.zeros((r, V), dtype=np.float32)
    x0 = np.zeros(B, dtype=np.int32)
    tok, pd, _ = oracle.markov_draft(L, A, Bm, x0, SEED)
    # anticipating policy: length 2 when x_1 = A (confident continuation), else 0
    ell_ant = np.where(tok[:, 0] == 0, 2, 0).astype(np.int32)
    _, out_a, _, _ = oracle.verify(T, L, A, Bm, x0, tok, pd, ell_ant, SEED)
    p_ant = (out_a[:, 0] == 0).mean()
    se = np.sqrt(0.25 / B)
    assert abs(p_ant - fx["P_first_emitted_A_anticipating"]) < 5 * se
    for fixed in (0, 1, 2):
        ell = np.full(B, fixed, dtype=np.int32)
        _, out_f, _, _ = oracle.verify(T, L, A, Bm, x0, tok, pd, ell, SEED)
        assert abs((out_f[:, 0] == 0).mean() - fx["P_first_emitted_A_non_anticipating"]) < 5 * se


def test_final_token_query_brackets_contain_tau():
    g = np.random.default_rng(15)
    B, gamma, V, r = 4, 3, 300, 8
    Tk, T, L, A, Bm, x0 = _problem(B, gamma, V, r, g)
    tok, pd, _ = oracle.markov_draft(L, A, Bm, x0, SEED)
    for b in range(B):
        for a in range(gamma + 1):
            o = oracle.final_token(T[b], L[b], A, Bm, x0[b], tok[b], gamma, a, SEED, b)
            q = oracle.final_token(T[b], L[b], A, Bm, x0[b], tok[b], gamma, a, SEED, b, query=o["tok"])
            assert q["tok"] == o["tok"]
            assert q["cdf_before"] <= q["u"] < q["cdf_through"]


def test_target_p_reported_for_verified_positions_only():
    g = np.random.default_rng(16)
    B, gamma, V, r = 6, 4, 64, 4
    Tk, T, L, A, Bm, x0 = _problem(B, gamma, V, r, g)
    tok, pd, _ = oracle.markov_draft(L, A, Bm, x0, SEED)
    ell = np.array([0, 1, 2, 3, 4, 2], dtype=np.int32)
    acc, out, n_out, tp = oracle.verify(T, L, A, Bm, x0, tok, pd, ell, SEED)
    for b in range(B):
        for k in range(gamma):
            if k < ell[b]:
                ref = _softmax64(Tk[k])[tok[b, k]]
                assert tp[b, k] == pytest.approx(ref, rel=1e-6)
            else:
                assert tp[b, k] == 0.0


# ----------------------------------------------------------------------------- exact law by enumeration
def _exact_softmax(x):
    """Softmax of a float64 vector as exact rationals summing to 1: the float64 weights exp(x - max)
    taken as exact fractions and normalised exactly (the law the enumeration below assumes)."""
    from fractions import Fraction
    x = np.asarray(x, dtype=np.float64)
    w = [Fraction(float(v)) for v in np.exp(x - x.max())]
    s = sum(w)
    return [v / s for v in w]


def _enumerate_law(q, pd_of, ell, gamma):
    """Exact law of the emitted tuple for one request, by summing over every draft path and every
    accept / reject event with exact rationals (menfem.com note, Methodology: the k-th drafted token is
    kept with probability min(1, p_t/p_d) and the first rejection ends the step; the token after a
    rejection comes from normalise(max(0, p_t - p_d)) at that position, and after ell acceptances from
    p_t of position ell+1).
    q[k] is the target law at position k+1 (k = 0..gamma); pd_of(k, x) the draft law at position k+1 given
    the conditioning token x (x = -1 for the committed token x_0).  Returns {tuple: probability}."""
    from fractions import Fraction
    law = {}

    def add(t, pr):
        law[t] = law.get(t, Fraction(0)) + pr

    def walk(k, prev, prefix, pr):
        if pr == 0:
            return
        if k == ell:  # every verified token accepted: one token from the target at position ell+1
            for w, qw in enumerate(q[k]):
                add(prefix + (w,), pr * qw)
            return
        p = pd_of(k, prev)
        resid = [max(Fraction(0), q[k][w] - p[w]) for w in range(len(p))]
        rs = sum(resid)
        for x, px in enumerate(p):
            if px == 0:
                continue
            acc = min(Fraction(1), q[k][x] / px)
            walk(k + 1, x, prefix + (x,), pr * px * acc)
            if acc < 1:  # rejection at position k+1: the residual token ends the step
                for w, rw in enumerate(resid):
                    if rw:
                        add(prefix + (w,), pr * px * (1 - acc) * rw / rs)

    walk(0, -1, (), Fraction(1))
    return law


@pytest.mark.parametrize("V,gamma", [(3, 3), (4, 2), (4, 3)])
def test_verify_law_exact_by_enumeration(V, gamma):
    """For every verify length ell = 0..gamma: (i) the enumerated law satisfies the exactness identity of
    the acceptance rule with no rounding at all -- given the emitted prefix y_1..y_{j-1} and that a j-th token
    is emitted, y_j follows p_t at position j, so the law of the tuple is the product of the target
    probabilities along it times a stopping law; (ii) the oracle's realised tuples (draft + verify over
    many requests with identical rows, Markov-conditioned draft) follow the enumerated law (chi-square)."""
    from fractions import Fraction
    g = np.random.default_rng(100 + 10 * V + gamma)
    r = 3
    Tk = (g.standard_normal((gamma + 1, V)) * 1.2).astype(np.float32)
    Lk = (g.standard_normal((gamma, V)) * 1.2).astype(np.float32)
    A = (g.standard_normal((V, r)) * 0.8).astype(np.float32)
    Bm = (g.standard_normal((r, V)) * 0.8).astype(np.float32)
    x0v = int(g.integers(0, V))
    q = [_exact_softmax(Tk[k].astype(np.float64)) for k in range(gamma + 1)]
    pd_cache = {}

    def pd_of(k, prev):
        x = x0v if prev < 0 else prev
        if (k, x) not in pd_cache:
            f = Lk[k].astype(np.float64) + A[x].astype(np.float64) @ Bm.astype(np.float64)
            pd_cache[(k, x)] = _exact_softmax(f)
        return pd_cache[(k, x)]

    n_per = 120000
    ells = np.repeat(np.arange(gamma + 1, dtype=np.int32), n_per)
    B = ells.size
    T = np.broadcast_to(Tk, (B, gamma + 1, V)).copy()
    L = np.broadcast_to(Lk, (B, gamma, V)).copy()
    x0 = np.full(B, x0v, dtype=np.int32)
    tok, pd, _ = oracle.markov_draft(L, A, Bm, x0, SEED)
    acc, out, n_out, _ = oracle.verify(T, L, A, Bm, x0, tok, pd, ells, SEED)
    for ell in range(gamma + 1):
        law = _enumerate_law(q, pd_of, ell, gamma)
        assert sum(law.values()) == 1
        # (i) exactness: P(prefix, y_j = w, n >= j) = P(prefix, n >= j) * p_t,j(w) for every prefix and w
        for j in range(1, ell + 2):
            reach = {}
            emit = {}
            for t, pr in law.items():
                if len(t) >= j:
                    reach[t[:j - 1]] = reach.get(t[:j - 1], Fraction(0)) + pr
                    emit[t[:j]] = emit.get(t[:j], Fraction(0)) + pr
            for pre, pr in reach.items():
                for w in range(V):
                    assert emit.get(pre + (w,), Fraction(0)) == pr * q[j - 1][w]
        # (ii) the oracle's tuples against the law
        sel = ells == ell
        keys = [tuple(int(v) for v in out[i, :n_out[i]]) for i in np.nonzero(sel)[0]]
        cells = sorted(law, key=lambda t: (len(t), t))
        idx = {t: i for i, t in enumerate(cells)}
        counts = np.zeros(len(cells))
        for t in keys:
            assert t in idx, (ell, t)  # no tuple of probability zero
            counts[idx[t]] += 1
        expect = np.array([float(law[t]) for t in cells]) * len(keys)
        big = expect >= 5
        obs = np.append(counts[big], counts[~big].sum())
        exp = np.append(expect[big], expect[~big].sum())
        if exp[-1] == 0:
            obs, exp = obs[:-1], exp[:-1]
        pval = stats.chisquare(obs, exp * obs.sum() / exp.sum()).pvalue
        assert pval > 1e-4, (V, gamma, ell, pval)
