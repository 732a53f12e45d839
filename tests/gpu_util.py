"""Helpers for the GPU tests: run one draft -> schedule -> verify step through
the C ABI and bring the outputs back to the host."""
from __future__ import annotations

import numpy as np
import torch

import draft_verify_sampling_prev_amd as dsp
from oracle import check


def f32(t: torch.Tensor) -> np.ndarray:
    return np.ascontiguousarray(t.float().numpy())


def host(t):
    return None if t is None else t.cpu().numpy()


def run_step(inp, budget: int, seed: int, dev=None):
    dev = dev or torch.device("cuda:0")
    g = inp.to(dev)
    tok, p, lse = dsp.dspark_markov_draft(g.L, g.A, g.Bm, g.x0, seed)
    theta, ell = dsp.dspark_schedule(g.z, g.temps, budget)
    acc, out_tok, n_out, tp = dsp.dspark_verify(g.T, g.L, g.A, g.Bm, g.x0, tok, p, lse, ell, seed)
    torch.cuda.synchronize()
    return dict(tok=host(tok), p=host(p), lse=host(lse), theta=host(theta), ell=host(ell), acc=host(acc),
                out_tok=host(out_tok), n_out=host(n_out), tp=host(tp))


def check_step(inp, out, budget: int, seed: int, draft_rows=None, requests=None, threads: int = 1) -> check.Report:
    """Teacher-forced oracle check of one step: draft_rows / requests None = every row / request;
    threads > 1 spreads the oracle over host threads."""
    T, L, A, Bm = f32(inp.T), f32(inp.L), f32(inp.A), f32(inp.Bm)
    x0 = inp.x0.numpy()
    rep = check.Report()
    check.check_draft(L, A, Bm, x0, seed, out["tok"], out["p"], out["lse"], rep, rows=draft_rows, threads=threads)
    check.check_survival(inp.z.numpy(), inp.temps.numpy(), out["theta"], rep)
    check.check_select(out["theta"], budget, out["ell"], rep)
    check.check_verify(T, L, A, Bm, x0, out["tok"], out["p"], out["ell"], seed, out["acc"], out["out_tok"],
                       out["n_out"], out["tp"], rep, requests=requests, threads=threads)
    return rep


def structural_checks(out, gamma: int):
    """Properties that hold for every request at any size."""
    acc, ell, n_out, out_tok, tok = out["acc"], out["ell"], out["n_out"], out["out_tok"], out["tok"]
    assert np.all((ell >= 0) & (ell <= gamma))
    assert np.all((acc >= 0) & (acc <= ell))
    assert np.array_equal(n_out, acc + 1)
    for b in range(len(acc)):
        a = int(acc[b])
        assert np.array_equal(out_tok[b, :a], tok[b, :a])
        assert out_tok[b, a] >= 0
        assert np.all(out_tok[b, a + 1:] == -1)
