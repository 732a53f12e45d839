"""GPU parity of the RNN sequential head (dspark_rnn_draft + dspark_rnn_verify)
against the oracle, teacher-forced on the GPU's own states and tokens: each
state within half an ulp of its element type of tanh(W h_prev + A[x]), each
draft sample / residual from the GPU's state as the operand.  Near-boundary
flips are counted over sampling and accept decisions only (not state
elements) and held to the Markov path's rule (oracle/check.py flips_ok)."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_prev_amd as dsp
from draft_verify_sampling_prev_amd import synth
from oracle import check

pytestmark = pytest.mark.gpu



def _f32(t):
    return np.ascontiguousarray(t.float().cpu().numpy())


def _run(wl, seed=777, draft_rows=None, requests=None, state_rows=None):
    dev = torch.device("cuda:0")
    print(f"case rnn {wl.describe()} seed={seed}", flush=True)
    inp = synth.make_inputs(wl)
    g = inp.to(dev)
    r = wl.r
    gen = torch.Generator().manual_seed(wl.data_seed + 3)
    Wt = (torch.randn((r, r), generator=gen) / np.sqrt(r)).to(g.L.dtype).to(dev)
    tok, p, lse, H = dsp.dspark_rnn_draft(g.L, g.A, g.Bm, Wt, g.x0, seed)
    theta, ell = dsp.dspark_schedule(g.z, g.temps, wl.budget)
    acc, out_tok, n_out, tp = dsp.dspark_rnn_verify(g.T, g.L, H, g.Bm, tok, p, lse, ell, seed)
    torch.cuda.synchronize()
    Hh, tk = _f32(H), tok.cpu().numpy()
    A, Wh, Bm, L, T = _f32(g.A), _f32(Wt), _f32(g.Bm), _f32(g.L), _f32(g.T)
    rep = check.Report()
    check.check_rnn_states(A, Wh, inp.x0.numpy(), tk, Hh, rep, elem=wl.dtype, rows=state_rows)
    nt = check.default_threads()
    check.check_draft(L, A, Bm, inp.x0.numpy(), seed, tk, p.cpu().numpy(), lse.cpu().numpy(), rep, rows=draft_rows,
                      states=Hh, threads=nt)
    check.check_verify(T, L, A, Bm, inp.x0.numpy(), tk, p.cpu().numpy(), ell.cpu().numpy(), seed, acc.cpu().numpy(),
                       out_tok.cpu().numpy(), n_out.cpu().numpy(), tp.cpu().numpy(), rep, requests=requests,
                       states=Hh, threads=nt)
    print("  ", rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert check.flips_ok(rep), rep.summary()
    # the states really carry the prefix: they differ from tanh(A[x]) once W acts (k >= 2)
    if wl.gamma >= 2:
        assert not np.allclose(Hh[:, 1], np.tanh(A[tk[:, 0]]), atol=1e-4)
    return rep


CASES = [
    dict(B=3, gamma=4, V=1000, r=24, budget=8, dtype="bf16"),
    dict(B=5, gamma=3, V=777 * 8, r=16, budget=9, dtype="f32"),
    dict(B=37, gamma=4, V=3000, r=256, budget=100, dtype="bf16"),
    dict(B=300, gamma=3, V=2048, r=256, budget=600, dtype="bf16"),
    dict(B=4, gamma=2, V=4224 * 64, r=64, budget=5, dtype="bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c['B']}-g{c['gamma']}-V{c['V']}-r{c['r']}-{c['dtype']}")
def test_rnn_draft_verify_matches_oracle(case):
    _run(synth.tiny(**case))


def test_rnn_headline_shape_full():
    """B = 256, gamma = 5, V = 129280, r = 256, bf16: every state, every draft row and every request."""
    rep = _run(synth.dsv4())
    assert rep.decisions >= 256 * 5 + 256
