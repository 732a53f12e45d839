"""GPU parity of dspark_markov_draft_sched, the draft steps with the budget
schedule carried by a draft launch, through the C ABI.  The schedule rides in
the first tile launch when one slot fewer leaves every slot's tile count
unchanged (B <= 256), else in the last locate launch, else (fp32, B*gamma
above 7680) it is launched after the draft; cases cover all three.

Every output is compared bit for bit with dspark_markov_draft followed by
dspark_schedule on the same inputs (the two forms run the same selection code
on different workgroup sizes), and the schedule part against the oracle: the
survivals within the survival tolerance, the verify lengths exact against the
oracle's selection on the GPU's own survivals.  Cases cover the fused path
(bf16, B*gamma up to its 7680-key limit, budgets at 0, 1, a tie at the cut,
N - 1, N and above N, ties across requests) and the fallback paths (fp32
logits, B*gamma above the limit), and a whole step (verify included) checked
against the oracle.
"""
import numpy as np
import pytest
import torch

import draft_verify_sampling_prev_amd as dsp
import oracle
from draft_verify_sampling_prev_amd import synth
from gpu_util import check_step, host, structural_checks
from oracle import check

pytestmark = pytest.mark.gpu

FUSED_MAX_KEYS = 7680  # B*gamma a draft launch can carry (a 32 KB LDS tile buffer)


def _host(B, gamma, V, dtype="bf16"):
    """Which launch carries the schedule, by the library's rule (slot count as bench.tile_slots)."""
    import bench
    if dtype != "bf16" or B * gamma > FUSED_MAX_KEYS:
        return "separate"
    nT = (V + 63) // 64
    S = bench.tile_slots(nT, 1, torch.cuda.get_device_properties(0).multi_processor_count, 36 if B == 256 else 12)
    if B <= 256 and S > 1 and -(-nT // (S - 1)) == -(-nT // S):
        return "first tiles"
    return "last locate" if nT <= 64 * 64 else "separate"


def _bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint8)


def _both(g, budget: int, seed: int):
    """(fused outputs, separate-call outputs), each a dict of host arrays."""
    tok, p, lse, theta, ell = dsp.dspark_markov_draft_sched(g.L, g.A, g.Bm, g.x0, seed, g.z, g.temps, budget)
    torch.cuda.synchronize()
    fused = dict(tok=host(tok), p=host(p), lse=host(lse), theta=host(theta), ell=host(ell))
    tok2, p2, lse2 = dsp.dspark_markov_draft(g.L, g.A, g.Bm, g.x0, seed)
    theta2, ell2 = dsp.dspark_schedule(g.z, g.temps, budget)
    torch.cuda.synchronize()
    sep = dict(tok=host(tok2), p=host(p2), lse=host(lse2), theta=host(theta2), ell=host(ell2))
    return fused, sep


def _compare(fused, sep, z, temps, budget, what):
    for k in ("tok", "p", "lse", "theta", "ell"):
        assert np.array_equal(_bits(fused[k]), _bits(sep[k])), (what, k)
    rep = check.Report()
    check.check_survival(z, temps, fused["theta"], rep)
    assert rep.ok(), (what, rep.summary())
    assert np.array_equal(fused["ell"], oracle.select(fused["theta"], int(budget))), (what, budget)


@pytest.mark.parametrize("B,gamma,V,r,where", [(64, 5, 8192, 256, "last locate"), (37, 4, 3000, 256, "last locate"),
                                              (300, 3, 1000, 24, "last locate"),
                                              (1536, 5, 2048, 256, "last locate"),
                                              (64, 5, 40000, 256, "first tiles"), (200, 5, 40000, 24, "first tiles"),
                                              (256, 1, 40000, 256, "first tiles")])
def test_fused_schedule_matches_separate_calls(B, gamma, V, r, where):
    dev = torch.device("cuda:0")
    wl = synth.tiny(B=B, gamma=gamma, V=V, r=r, budget=1, dtype="bf16")
    inp = synth.make_inputs(wl)
    g = inp.to(dev)
    z, temps = inp.z.numpy(), inp.temps.numpy()
    N = B * gamma
    assert _host(B, gamma, V) == where
    print(f"case B={B} gamma={gamma} V={V} r={r} N={N} ({where})", flush=True)
    for budget in sorted({0, 1, N // 3, N - 1, N, N + 5}):
        fused, sep = _both(g, budget, wl.philox_seed + budget)
        _compare(fused, sep, z, temps, budget, f"budget {budget}")


@pytest.mark.parametrize("V,where", [(4096, "last locate"), (40000, "first tiles")])
def test_fused_schedule_ties_at_the_cut(V, where):
    """Confidence logits quantised to four values, so whole groups of candidates share a survival and the cut
    falls inside a group: the tie is broken in (request, position) order on both paths."""
    dev = torch.device("cuda:0")
    B, gamma = 200, 5
    assert _host(B, gamma, V) == where
    wl = synth.tiny(B=B, gamma=gamma, V=V, r=256, budget=1, dtype="bf16")
    inp = synth.make_inputs(wl)
    rng = np.random.default_rng(77)
    z = rng.choice(np.array([-1.0, 0.5, 2.0, 4.0], dtype=np.float32), size=(B, gamma))
    z[::7] = 2.0  # equal rows across requests
    inp.z = torch.from_numpy(z)
    g = inp.to(dev)
    temps = inp.temps.numpy()
    theta, _ = dsp.dspark_schedule(g.z, g.temps, 0)
    vals, counts = np.unique(host(theta), return_counts=True)
    # Budgets that cut inside the largest groups of equal survivals.
    order = np.sort(host(theta).ravel())[::-1]
    cuts = {1, B * gamma // 2}
    for v, c in zip(vals, counts):
        if c > 1:
            first = int(np.argmax(order == v))
            cuts.add(first + c // 2)
    for budget in sorted(cuts):
        fused, sep = _both(g, budget, 0xABCDEF + budget)
        _compare(fused, sep, z, temps, budget, f"tie cut {budget}")


@pytest.mark.parametrize("case", ["f32", "over_limit"])
def test_fallback_paths_match_separate_calls(case):
    """fp32 logits, and B*gamma above the fused limit, take the separate schedule launch inside the same call."""
    dev = torch.device("cuda:0")
    if case == "f32":
        wl = synth.tiny(B=96, gamma=5, V=2048, r=64, budget=1, dtype="f32")
    else:
        wl = synth.tiny(B=1600, gamma=5, V=1024, r=256, budget=1, dtype="bf16")
    assert _host(wl.B, wl.gamma, wl.V, wl.dtype) == "separate"
    inp = synth.make_inputs(wl)
    g = inp.to(dev)
    N = wl.B * wl.gamma
    for budget in (0, N // 4, N):
        fused, sep = _both(g, budget, 99 + budget)
        _compare(fused, sep, inp.z.numpy(), inp.temps.numpy(), budget, f"{case} budget {budget}")


def test_fused_step_against_the_oracle():
    """A whole step through the fused call and dspark_verify, every draft row and request checked against the
    oracle (teacher-forced), as the parity tests check the separate calls."""
    dev = torch.device("cuda:0")
    wl = synth.tiny(B=48, gamma=5, V=20000, r=256, budget=150, dtype="bf16")
    assert _host(wl.B, wl.gamma, wl.V) == "first tiles"
    inp = synth.make_inputs(wl)
    g = inp.to(dev)
    seed = wl.philox_seed
    tok, p, lse, theta, ell = dsp.dspark_markov_draft_sched(g.L, g.A, g.Bm, g.x0, seed, g.z, g.temps, wl.budget)
    acc, out_tok, n_out, tp = dsp.dspark_verify(g.T, g.L, g.A, g.Bm, g.x0, tok, p, lse, ell, seed)
    torch.cuda.synchronize()
    out = dict(tok=host(tok), p=host(p), lse=host(lse), theta=host(theta), ell=host(ell), acc=host(acc),
               out_tok=host(out_tok), n_out=host(n_out), tp=host(tp))
    structural_checks(out, wl.gamma)
    rep = check_step(inp, out, wl.budget, seed, threads=check.default_threads())
    print("  ", rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert check.flips_ok(rep), rep.summary()


def test_fused_schedule_at_the_headline_shape():
    """B = 256, gamma = 5, V = 129280, r = 256: the fused call against the separate calls, bit for bit."""
    dev = torch.device("cuda:0")
    wl = synth.dsv4()
    assert _host(wl.B, wl.gamma, wl.V) == "first tiles"
    inp = synth.make_inputs(wl)
    g = inp.to(dev)
    for budget in (wl.budget, 1, wl.B * wl.gamma - 1):
        fused, sep = _both(g, budget, wl.philox_seed + budget)
        _compare(fused, sep, inp.z.numpy(), inp.temps.numpy(), budget, f"headline budget {budget}")
