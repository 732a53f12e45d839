"""GPU parity of the draft step with the fused Markov-conditioned confidence
head (dspark_markov_draft_conf): draft outputs identical to
dspark_markov_draft, z within an fp32 dot-product bound of the oracle on the
GPU's own tokens, and the schedule driven by those z exact on the GPU's
survivals."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_prev_amd as dsp
import oracle
from draft_verify_sampling_prev_amd import synth

pytestmark = pytest.mark.gpu


def _f32(t):
    return np.ascontiguousarray(t.float().cpu().numpy())


CASES = [
    dict(B=3, gamma=4, V=1000, r=24, budget=8, dtype="bf16"),
    dict(B=5, gamma=3, V=777 * 8, r=16, budget=9, dtype="f32"),
    dict(B=37, gamma=4, V=3000, r=256, budget=100, dtype="bf16"),       # rank 256: A rows handed over in MFMA order
    dict(B=300, gamma=3, V=2048, r=256, budget=600, dtype="bf16"),      # two 256-row blocks
    dict(B=4, gamma=2, V=4224 * 64, r=64, budget=5, dtype="bf16"),      # more than 4096 tiles: the 256-thread locate
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c['B']}-g{c['gamma']}-V{c['V']}-r{c['r']}-{c['dtype']}")
def test_draft_conf_matches_oracle(case):
    dev = torch.device("cuda:0")
    wl = synth.tiny(**case)
    inp = synth.make_inputs(wl)
    g = inp.to(dev)
    B, gamma, r = wl.B, wl.gamma, wl.r
    rng = np.random.default_rng(17 + B)
    wc = torch.from_numpy((rng.standard_normal(r) * 0.5).astype(np.float32)).to(g.L.dtype).to(dev)
    z0 = g.z
    seed = 4242
    tok0, p0, lse0 = dsp.dspark_markov_draft(g.L, g.A, g.Bm, g.x0, seed)
    tok, p, lse, z = dsp.dspark_markov_draft_conf(g.L, g.A, g.Bm, g.x0, seed, z0, wc)
    torch.cuda.synchronize()
    # the confidence head does not touch the draft
    assert torch.equal(tok, tok0) and torch.equal(p.view(torch.int32), p0.view(torch.int32))
    assert torch.equal(lse.view(torch.int64), lse0.view(torch.int64))
    # z against the oracle on the GPU's tokens
    A, w, x0, t = _f32(g.A), _f32(wc), inp.x0.numpy(), tok.cpu().numpy()
    ref = oracle.markov_confidence(A, w, x0, t, inp.z.numpy()).astype(np.float64)
    prev = np.concatenate([x0[:, None], t[:, :-1]], axis=1)
    mag = np.abs(inp.z.numpy()).astype(np.float64) + np.abs(A[prev].astype(np.float64) * w.astype(np.float64)).sum(-1)
    err = np.abs(z.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= 2.0**-24 * (r + 2) * mag + 1e-30), float((err / (mag + 1e-30)).max())
    # the schedule on these z: exact on the GPU's survivals
    theta, ell = dsp.dspark_schedule(z, g.temps, wl.budget)
    torch.cuda.synchronize()
    assert np.array_equal(ell.cpu().numpy(), oracle.select(theta.cpu().numpy(), wl.budget))


def test_draft_conf_headline_shape():
    """B = 256, gamma = 5, V = 129280, r = 256: every z against the oracle."""
    dev = torch.device("cuda:0")
    wl = synth.dsv4()
    inp = synth.make_inputs(wl)
    g = inp.to(dev)
    rng = np.random.default_rng(99)
    wc = torch.from_numpy((rng.standard_normal(wl.r) * 0.5).astype(np.float32)).to(torch.bfloat16).to(dev)
    tok, p, lse, z = dsp.dspark_markov_draft_conf(g.L, g.A, g.Bm, g.x0, wl.philox_seed, g.z, wc)
    torch.cuda.synchronize()
    A, w, x0, t = _f32(g.A), _f32(wc), inp.x0.numpy(), tok.cpu().numpy()
    ref = oracle.markov_confidence(A, w, x0, t, inp.z.numpy()).astype(np.float64)
    prev = np.concatenate([x0[:, None], t[:, :-1]], axis=1)
    mag = np.abs(inp.z.numpy()).astype(np.float64) + np.abs(A[prev].astype(np.float64) * w.astype(np.float64)).sum(-1)
    err = np.abs(z.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= 2.0**-24 * (wl.r + 2) * mag + 1e-30)
    # z_k follows x_{k-1}: it differs from z0 by the token part
    assert not np.allclose(z.cpu().numpy(), inp.z.numpy())
