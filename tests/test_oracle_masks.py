"""Pins for the oracle with vocabulary masks (logits of -inf), CPU only.

A token whose draft or target logit is -inf has probability 0: the oracle
never drafts it, never emits it, and its probabilities are the softmax over
the finite logits only.  Checked against the closed form: the draft row's
p(x) and log-normaliser equal the masked softmax computed here in numpy
(float64), a row with one finite logit drafts that token with p = 1 for every
u, and a whole step with masked draft and target rows emits only unmasked
tokens, accepting every draft of the single-token rows (p_t = p_d = 1).
"""
import numpy as np
import pytest

import oracle


def _row(V, r, seed):
    g = np.random.default_rng(seed)
    L = g.normal(0, 2, V).astype(np.float32)
    A = (g.normal(0, 0.2, (V, r))).astype(np.float32)
    Bm = (g.normal(0, 0.2, (r, V))).astype(np.float32)
    return L, A, Bm


@pytest.mark.parametrize("keep", [1, 5, 40])
def test_masked_draft_row_is_the_softmax_over_the_finite_logits(keep):
    V, r = 96, 8
    L, A, Bm = _row(V, r, 3 + keep)
    g = np.random.default_rng(keep)
    allowed = np.sort(g.choice(V, size=keep, replace=False))
    Lm = np.full(V, -np.inf, dtype=np.float32)
    Lm[allowed] = L[allowed]
    prev = 7
    f = oracle.markov_logits(Lm, A, Bm, prev)
    assert np.all(np.isneginf(f[np.setdiff1d(np.arange(V), allowed)]))
    fin = f[allowed]
    lse = fin.max() + np.log(np.exp(fin - fin.max()).sum())
    for u in np.linspace(0.0, 1.0, 257, endpoint=False, dtype=np.float32):
        o = oracle.draft_row(Lm, A, Bm, prev, float(u))
        assert o["tok"] in allowed
        assert o["lse"] == pytest.approx(lse, rel=0, abs=1e-12)
        assert o["p"] == pytest.approx(np.exp(f[o["tok"]] - lse), rel=1e-12)
        if keep == 1:
            assert o["p"] == 1.0 and o["tok"] == allowed[0]


def test_masked_step_emits_only_finite_tokens():
    B, gamma, V, r = 8, 3, 64, 8
    g = np.random.default_rng(11)
    L = g.normal(0, 2, (B, gamma, V)).astype(np.float32)
    T = g.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    A = g.normal(0, 0.2, (V, r)).astype(np.float32)
    Bm = g.normal(0, 0.2, (r, V)).astype(np.float32)
    x0 = g.integers(0, V, B).astype(np.int32)
    allowed = []
    for b in range(B):
        keep = g.choice(V, size=1 if b % 2 == 0 else 6, replace=False)
        m = np.ones(V, dtype=bool)
        m[keep] = False
        L[b][:, m] = -np.inf
        T[b][:, m] = -np.inf
        allowed.append(set(int(x) for x in keep))
    for seed in range(20):
        tok, p, lse = oracle.markov_draft(L, A, Bm, x0, seed)
        ell = np.full(B, gamma, dtype=np.int32)
        acc, out, n_out, tp = oracle.verify(T, L, A, Bm, x0, tok, p, ell, seed)
        for b in range(B):
            assert set(int(x) for x in tok[b]) <= allowed[b]
            emitted = out[b][: n_out[b]]
            assert set(int(x) for x in emitted) <= allowed[b], (seed, b, emitted)
            if len(allowed[b]) == 1:
                assert np.all(p[b] == 1.0) and acc[b] == gamma and np.all(tp[b] == 1.0)
