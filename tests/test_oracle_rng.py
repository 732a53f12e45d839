"""Pins for the oracle's Philox-4x32-10 and its uniform mapping (CPU only)."""
import os

import numpy as np
import pytest
from scipy import stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = [int(x, 16) for x in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat())
def test_philox_known_answers(ctr, key, expect):
    out = oracle.philox4x32_10(ctr, key)
    assert [int(x) for x in out] == expect


def test_uniform_matches_first_kat_word():
    # seed 0 -> key (0, 0); (b, k, d) = 0 -> counter (0, 0, 0, 0); word 0 is 0x6627e8d5.
    u = oracle.uniform(0, 0, 0, 0)
    assert u == (0x6627E8D5 >> 8) / 2.0**24


def test_uniform_keying_distinguishes_every_field():
    seed = 0x0123456789ABCDEF
    base = oracle.uniform(seed, 3, 2, 1)
    assert oracle.uniform(seed, 4, 2, 1) != base
    assert oracle.uniform(seed, 3, 3, 1) != base
    assert oracle.uniform(seed, 3, 2, 2) != base
    assert oracle.uniform(seed ^ (1 << 40), 3, 2, 1) != base  # high seed word is part of the key
    assert oracle.uniform(seed ^ 1, 3, 2, 1) != base


def test_uniform_grid_and_range():
    b = np.arange(4096)
    u = oracle.uniforms(7, b, 1, 0)
    assert u.dtype == np.float32
    assert np.all(u >= 0.0) and np.all(u < 1.0)
    scaled = u.astype(np.float64) * 2**24
    assert np.all(scaled == np.floor(scaled))  # on the 2^-24 grid


def test_uniform_chi_square():
    n = 1 << 20
    b = np.arange(n) % 4096
    k = np.arange(n) // 4096
    u = oracle.uniforms(0x0123456789ABCDEF, b, k, 1)
    counts = np.bincount((u * 256).astype(np.int64), minlength=256)
    p = stats.chisquare(counts).pvalue
    assert p > 1e-4
