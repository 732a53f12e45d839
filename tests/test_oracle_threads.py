"""The threaded oracle calls (requests split into contiguous ranges over POSIX
threads, used for the multi-thread CPU baseline) give the one-thread results
bit for bit, for thread counts that do and do not divide the batch."""
import numpy as np
import pytest

import oracle

SEED = 0x0123456789ABCDEF


@pytest.mark.parametrize("threads", [2, 3, 8, 64])
def test_threaded_draft_and_verify_equal_single_thread(threads):
    g = np.random.default_rng(40 + threads)
    B, gamma, V, r = 37, 4, 257 * 8, 16
    T = g.standard_normal((B, gamma + 1, V)).astype(np.float32) * 2
    L = (T[:, :gamma] + g.standard_normal((B, gamma, V)).astype(np.float32)).astype(np.float32)
    A = g.standard_normal((V, r)).astype(np.float32) * 0.3
    Bm = g.standard_normal((r, V)).astype(np.float32) * 0.3
    x0 = g.integers(0, V, B).astype(np.int32)
    one = oracle.markov_draft(L, A, Bm, x0, SEED)
    many = oracle.markov_draft(L, A, Bm, x0, SEED, threads=threads)
    for a, b in zip(one, many):
        assert np.array_equal(a, b)
    ell = g.integers(0, gamma + 1, B).astype(np.int32)
    v1 = oracle.verify(T, L, A, Bm, x0, one[0], one[1], ell, SEED)
    vn = oracle.verify(T, L, A, Bm, x0, one[0], one[1], ell, SEED, threads=threads)
    for a, b in zip(v1, vn):
        assert np.array_equal(a, b)


def test_threaded_calls_report_bad_input():
    B, gamma, V, r = 4, 2, 16, 2
    T = np.zeros((B, gamma + 1, V), np.float32)
    L = np.zeros((B, gamma, V), np.float32)
    A = np.zeros((V, r), np.float32)
    Bm = np.zeros((r, V), np.float32)
    x0 = np.array([0, 1, V, 2], np.int32)  # one committed token out of range
    with pytest.raises(RuntimeError):
        oracle.markov_draft(L, A, Bm, x0, SEED, threads=3)
    tok = np.zeros((B, gamma), np.int32)
    pd = np.full((B, gamma), 1.0 / V, np.float32)
    ell = np.array([0, 1, 3, 2], np.int32)  # a verify length beyond gamma
    with pytest.raises(RuntimeError):
        oracle.verify(T, L, A, Bm, np.zeros(B, np.int32), tok, pd, ell, SEED, threads=2)
