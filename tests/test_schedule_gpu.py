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
