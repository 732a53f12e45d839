"""Sequential temperature scaling (STS) of the confidence head, on the host.

The scheduler ranks draft positions by prefix survival
Theta_k = prod_{j<=k} sigmoid(z_j / T_j), one temperature per position shared
by all requests.  The temperatures are fitted offline, left to right, so that
the calibration error of the cumulative product at each position is smallest
(paperlayer.ai summary of arXiv 2607.05147, section 3.2: sequential
temperature scaling calibrates the confidence position by position against
the expected calibration error of the running product; menfem.com note,
"Key Contributions": post-hoc sequential temperature scaling).

Labels: s[b, k] = 1 when positions 1..k of request b were all accepted in a
step that verified every drafted token (the event Theta_k predicts).  The
pages give no binning; 15 equal-width bins is the convention used here.

This is calibration tooling that runs once per model, not part of the
per-step path (which takes the temperatures as an input); it is plain numpy.
The survival product is evaluated in float32 as the path evaluates it.
"""
from __future__ import annotations

import numpy as np

ECE_BINS = 15
# 400 temperatures, log-spaced over [0.05, 20].
DEFAULT_GRID = np.exp(np.linspace(np.log(0.05), np.log(20.0), 400)).astype(np.float32)


def ece(conf, labels, bins: int = ECE_BINS) -> float:
    """Expected calibration error: bin the confidences into `bins` equal-width bins over [0, 1] (the last
    bin closed), and sum |mean label - mean confidence| over the bins weighted by their share of the samples."""
    c = np.asarray(conf, dtype=np.float64).ravel()
    y = np.asarray(labels, dtype=np.float64).ravel()
    if c.size == 0:
        return 0.0
    idx = np.minimum((c * bins).astype(np.int64), bins - 1)
    idx = np.clip(idx, 0, bins - 1)
    cnt = np.bincount(idx, minlength=bins).astype(np.float64)
    sc = np.bincount(idx, weights=c, minlength=bins)
    sy = np.bincount(idx, weights=y, minlength=bins)
    nz = cnt > 0
    return float(np.sum(np.abs(sy[nz] - sc[nz])) / c.size)


def survival(z, temps) -> np.ndarray:
    """Theta[b, k] = prod_{j<=k} sigmoid(z[b, j] / temps[j]), in float32 left to right."""
    z = np.asarray(z, dtype=np.float32)
    t = np.asarray(temps, dtype=np.float32)
    with np.errstate(over="ignore"):  # exp overflow gives sigmoid 0, as intended
        c = (np.float32(1.0) / (np.float32(1.0) + np.exp(-(z / t[None, :])))).astype(np.float32)
    th = np.empty_like(c)
    run = np.ones(z.shape[0], dtype=np.float32)
    for k in range(z.shape[1]):
        run = (run * c[:, k]).astype(np.float32)
        th[:, k] = run
    return th


def survival_labels(accepted, gamma: int) -> np.ndarray:
    """s[b, k-1] = 1 when request b accepted at least k tokens (every token verified)."""
    a = np.asarray(accepted).reshape(-1, 1)
    return (a >= np.arange(1, gamma + 1)[None, :]).astype(np.float64)


def fit_sts(z, labels, grid=None, bins: int = ECE_BINS):
    """Fit one temperature per position, left to right: T_k is the grid value that minimises the ECE of
    Theta_k = Theta_{k-1} * sigmoid(z_k / T_k) against labels[:, k], with T_1 .. T_{k-1} already fixed
    (ties: the first grid value).  Returns (temps float32 [gamma], ece per position at the fit)."""
    z = np.asarray(z, dtype=np.float32)
    s = np.asarray(labels, dtype=np.float64)
    grid = DEFAULT_GRID if grid is None else np.asarray(grid, dtype=np.float32)
    n, gamma = z.shape
    prev = np.ones(n, dtype=np.float32)
    temps = np.zeros(gamma, dtype=np.float32)
    errs = np.zeros(gamma)
    for k in range(gamma):
        best, best_t, best_th = None, None, None
        for T in grid:
            with np.errstate(over="ignore"):  # exp overflow gives sigmoid 0, as intended
                c = (np.float32(1.0) / (np.float32(1.0) + np.exp(-(z[:, k] / T)))).astype(np.float32)
            th = (prev * c).astype(np.float32)
            e = ece(th, s[:, k], bins)
            if best is None or e < best:
                best, best_t, best_th = e, T, th
        temps[k], errs[k], prev = best_t, best, best_th
    return temps, errs
