"""GPU parity of the objective-based and static-threshold admission entry
points (through the C ABI) against the oracle: survivals within the survival
tolerance (device and host exp differ by ulps), and verify lengths exact
against the oracle run on the GPU's own survivals (the decision taken on the
same inputs on both sides)."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_prev_amd as dsp
import oracle
from oracle import check

pytestmark = pytest.mark.gpu


def _inputs(B, gamma, seed, ties=False):
    g = np.random.default_rng(seed)
    z = (g.standard_normal((B, gamma)) * 2.0).astype(np.float32)
    if ties:
        z[:] = z[0, 0]
    temps = (1.0 + 0.15 * np.arange(1, gamma + 1)).astype(np.float32)
    return z, temps


def _survival_ok(z, temps, theta_gpu):
    rep = check.Report()
    check.check_survival(z, temps, theta_gpu, rep)
    assert rep.ok(), rep.summary()


def _profile(kind, n, seed):
    g = np.random.default_rng(1000 + seed)
    x = np.arange(n, dtype=np.float64)
    if kind == "concave":      # fixed launch cost plus a per-token cost
        t = 40.0 + 0.05 * x
    elif kind == "steps":      # capacity quantised in blocks of 64 tokens
        t = 10.0 + 3.0 * np.floor(x / 64.0) + 0.001 * x
    elif kind == "increasing":
        t = np.cumsum(g.uniform(0.01, 1.0, n))
    elif kind == "random":     # not monotone
        t = g.uniform(0.5, 2.0, n)
    elif kind == "flat":
        t = np.ones(n)
    elif kind == "linear":
        t = 0.01 * x + 1e-3
    else:
        raise ValueError(kind)
    return t.astype(np.float32)


SHAPES = [(1, 1), (3, 5), (37, 4), (256, 5), (300, 16), (1024, 16), (4096, 4)]
KINDS = ["concave", "steps", "increasing", "random", "flat", "linear"]


@pytest.mark.parametrize("B,gamma", SHAPES)
@pytest.mark.parametrize("kind", KINDS)
def test_objective_matches_oracle(B, gamma, kind):
    dev = torch.device("cuda:0")
    seed = B * 31 + gamma
    z, temps = _inputs(B, gamma, seed, ties=(kind == "flat"))
    N = B * gamma
    t = _profile(kind, B + N + 1, seed)
    zt, tt, st = (torch.from_numpy(a).to(dev) for a in (z, temps, t))
    for cap in sorted({0, 1, N // 3, N, 4 * N}):
        theta, ln = dsp.dspark_schedule_objective(zt, tt, st, cap)
        torch.cuda.synchronize()
        theta_gpu = theta.cpu().numpy()
        _survival_ok(z, temps, theta_gpu)
        if cap == 0:
            theta_b, _ = dsp.dspark_schedule(zt, tt, 0)
            assert np.array_equal(theta_gpu.view(np.uint32), theta_b.cpu().numpy().view(np.uint32))
        ref_ln, ref_m = oracle.select_objective(theta_gpu, t, cap)
        got = ln.cpu().numpy()
        assert np.array_equal(got, ref_ln), (kind, cap, int(got.sum()), ref_m)
        assert int(got.sum()) == ref_m


def test_objective_stops_mid_stream_at_headline_shape():
    """A profile under which the early stop lands strictly inside the order,
    at the benchmarked shape (B = 256, gamma = 5): the stop rank is exact."""
    dev = torch.device("cuda:0")
    B, gamma = 256, 5
    z, temps = _inputs(B, gamma, 5)
    t = _profile("concave", B + B * gamma + 1, 5)
    zt, tt, st = (torch.from_numpy(a).to(dev) for a in (z, temps, t))
    theta, ln = dsp.dspark_schedule_objective(zt, tt, st, B * gamma)
    torch.cuda.synchronize()
    ref_ln, ref_m = oracle.select_objective(theta.cpu().numpy(), t, B * gamma)
    assert 0 < ref_m < B * gamma
    assert np.array_equal(ln.cpu().numpy(), ref_ln)


def test_objective_given_survivals_and_ties():
    """z = None: the survivals are the input; equal values order by request,
    then position."""
    dev = torch.device("cuda:0")
    B, gamma = 64, 6
    g = np.random.default_rng(9)
    theta = np.sort(g.choice(np.float32([0.9, 0.5, 0.5, 0.25, 0.0]), (B, gamma)), axis=1)[:, ::-1].copy()
    t = _profile("steps", B + B * gamma + 1, 9)
    surv = torch.from_numpy(theta).to(dev)
    for cap in (0, 7, 100, B * gamma):
        _, ln = dsp.dspark_schedule_objective(None, None, torch.from_numpy(t).to(dev), cap, survival=surv)
        torch.cuda.synchronize()
        ref_ln, _ = oracle.select_objective(theta, t, cap)
        assert np.array_equal(ln.cpu().numpy(), ref_ln)
        assert np.array_equal(surv.cpu().numpy(), theta)  # input left unchanged


@pytest.mark.parametrize("B,gamma", [(1, 1), (37, 4), (256, 5), (1000, 16)])
def test_threshold_matches_oracle(B, gamma):
    dev = torch.device("cuda:0")
    z, temps = _inputs(B, gamma, 77 + B)
    zt, tt = torch.from_numpy(z).to(dev), torch.from_numpy(temps).to(dev)
    theta_b, _ = dsp.dspark_schedule(zt, tt, 0)
    for tau in (0.0, 0.05, 0.3, 0.5, 0.9, 1.0):
        theta, ln = dsp.dspark_schedule_threshold(zt, tt, tau)
        torch.cuda.synchronize()
        theta_gpu = theta.cpu().numpy()
        _survival_ok(z, temps, theta_gpu)
        # the one-thread-per-request survival is the budget kernel's, bit for bit
        assert np.array_equal(theta_gpu.view(np.uint32), theta_b.cpu().numpy().view(np.uint32))
        assert np.array_equal(ln.cpu().numpy(), oracle.select_threshold(theta_gpu, tau))


# ----------------------------------------------------------------------------- budget admission (the benchmarked rule)
def _budget_given(theta: np.ndarray, budgets):
    """dspark_schedule in survival-input mode (z = None): verify lengths bit-exact against the oracle's
    sort-based selection on the same survivals for every budget, the admitted total exact, and the given
    survivals left untouched."""
    dev = torch.device("cuda:0")
    B, gamma = theta.shape
    N = B * gamma
    surv = torch.from_numpy(theta).to(dev)
    for budget in budgets:
        _, ln = dsp.dspark_schedule(None, None, int(budget), survival=surv)
        torch.cuda.synchronize()
        got = ln.cpu().numpy()
        ref = oracle.select(theta, int(budget))
        assert np.array_equal(got, ref), (B, gamma, int(budget), np.nonzero(got != ref)[0][:5])
        assert int(got.sum()) == min(int(budget), N)
    assert np.array_equal(surv.cpu().numpy().view(np.uint32), theta.view(np.uint32))


def _tie_budgets(theta: np.ndarray):
    """Budgets 0, 1, N-1, N, beyond N, and for each distinct survival value a cut just before, inside and
    just after its run of equal keys (so the admitted-th key is tied with keys on both sides of the cut)."""
    N = theta.size
    vals = np.sort(theta.ravel().astype(np.float64))[::-1]
    out = {0, 1, N - 1, N, N + 7}
    for v in np.unique(vals):
        above = int((vals > v).sum())
        eq = int((vals == v).sum())
        out |= {above, above + 1, above + eq // 2, above + eq - 1, above + eq}
    return sorted(b for b in out if b >= 0)


def _rows_from_levels(g, B, gamma, levels):
    """Non-increasing rows drawn from a few levels, so that many keys tie across requests."""
    return np.sort(g.choice(np.asarray(levels, dtype=np.float32), (B, gamma)), axis=1)[:, ::-1].copy()


@pytest.mark.parametrize("B,gamma", [(1, 1), (5, 3), (37, 4), (256, 5), (300, 16)])
def test_budget_ties_across_requests(B, gamma):
    g = np.random.default_rng(B + 17 * gamma)
    theta = _rows_from_levels(g, B, gamma, [1.0, 0.75, 0.5, 0.5, 0.25, 0.125, 0.0])
    _budget_given(theta, _tie_budgets(theta))


def test_budget_all_equal_survivals_admit_in_request_order():
    """Every key tied: the admitted set is the first `budget` candidates in (request, position) order."""
    B, gamma = 64, 6
    theta = np.full((B, gamma), 0.5, dtype=np.float32)
    for budget in (0, 1, 5, 6, 7, 100, 383, 384):
        _budget_given(theta, [budget])
        ln = oracle.select(theta, budget)
        assert ln.tolist() == [min(gamma, max(0, budget - gamma * b)) for b in range(B)]


def test_budget_signed_zeros_are_equal():
    """-0 and +0 are the same survival: a cut inside a run of mixed zeros follows (request, position)."""
    B, gamma = 40, 4
    g = np.random.default_rng(3)
    theta = _rows_from_levels(g, B, gamma, [0.5, 0.25, 0.0])
    zeros = theta == 0
    flip = zeros & (g.random((B, gamma)) < 0.5)
    theta[flip] = np.float32(-0.0)
    assert (theta.view(np.uint32) == 0x80000000).any() and (theta.view(np.uint32) == 0).any()
    _budget_given(theta, _tie_budgets(theta))


def test_budget_denormal_and_zero_survivals_at_gamma16():
    """gamma = 16 with survivals in the denormal range and exactly zero (given), then the same regime
    reached through the survival product itself (z strongly negative): the selection is exact on the
    GPU's own survivals, and survivals agree with the oracle's fp32 product."""
    B, gamma = 64, 16
    g = np.random.default_rng(16)
    # given: per row, a descending walk through normal, denormal and zero bit patterns
    bits = np.sort(g.choice(np.array([0x3F000000, 0x00800000, 0x007FFFFF, 0x00400000, 0x00000100, 0x00000001,
                                      0x00000000, 0x00000000], dtype=np.uint32), (B, gamma)), axis=1)[:, ::-1]
    theta = np.ascontiguousarray(bits).view(np.float32)
    assert np.isfinite(theta).all()
    _budget_given(theta, _tie_budgets(theta))
    # through the product: c = sigmoid(z) ~ 1e-5 per position drives Theta through the denormals to 0
    dev = torch.device("cuda:0")
    z = (g.standard_normal((B, gamma)) - 11.5).astype(np.float32)
    temps = np.ones(gamma, dtype=np.float32)
    zt, tt = torch.from_numpy(z).to(dev), torch.from_numpy(temps).to(dev)
    th, _ = dsp.dspark_schedule(zt, tt, 0)
    torch.cuda.synchronize()
    th_gpu = th.cpu().numpy()
    _survival_ok(z, temps, th_gpu)
    assert (th_gpu == 0).any() and ((th_gpu > 0) & (th_gpu < np.finfo(np.float32).tiny)).any()
    for budget in _tie_budgets(th_gpu):
        theta2, ln = dsp.dspark_schedule(zt, tt, budget)
        torch.cuda.synchronize()
        assert np.array_equal(theta2.cpu().numpy().view(np.uint32), th_gpu.view(np.uint32))
        assert np.array_equal(ln.cpu().numpy(), oracle.select(th_gpu, budget)), budget


@pytest.mark.parametrize("B,gamma", [(1024, 16), (4096, 4), (16384, 1)])
def test_budget_at_the_candidate_limit(B, gamma):
    """B * gamma = 16384, the largest selection the one-workgroup kernel takes: from z (random, no ties)
    and given survivals with many ties."""
    dev = torch.device("cuda:0")
    z, temps = _inputs(B, gamma, B + gamma)
    zt, tt = torch.from_numpy(z).to(dev), torch.from_numpy(temps).to(dev)
    N = B * gamma
    for budget in (0, 1, N // 7, N // 2, N - 1, N):
        theta, ln = dsp.dspark_schedule(zt, tt, budget)
        torch.cuda.synchronize()
        th = theta.cpu().numpy()
        _survival_ok(z, temps, th)
        assert np.array_equal(ln.cpu().numpy(), oracle.select(th, budget)), budget
    g = np.random.default_rng(B)
    theta = _rows_from_levels(g, B, gamma, [0.9, 0.6, 0.6, 0.3, 0.1, 0.0])
    _budget_given(theta, _tie_budgets(theta))


def test_budget_headline_shape_cuts():
    """B = 256, gamma = 5 from z: budgets around the benchmarked 768 and at the ends."""
    dev = torch.device("cuda:0")
    B, gamma = 256, 5
    z, temps = _inputs(B, gamma, 256)
    zt, tt = torch.from_numpy(z).to(dev), torch.from_numpy(temps).to(dev)
    for budget in (0, 1, 767, 768, 769, B * gamma - 1, B * gamma, 10**12):
        theta, ln = dsp.dspark_schedule(zt, tt, budget)
        torch.cuda.synchronize()
        th = theta.cpu().numpy()
        _survival_ok(z, temps, th)
        assert np.array_equal(ln.cpu().numpy(), oracle.select(th, budget)), budget
