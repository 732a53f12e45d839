"""The outputs of a draft + verify step do not depend on what the workspace
held before the call, through the C ABI.

The verify's final kernel reads rows of the workspace that only one of its
two branches fills (the residual tile sums of a request with a rejection, and
at B = 300 its per-slot sums in the rows the draft's slot aggregates used;
the bonus-row chunk partials of a request without one), and the draft's tile
launches write and read the A-row hand-over and the tile partials there.  Each
case runs the same step on workspaces filled with all-ones bytes (NaN and -1
patterns), with zeros and with random bytes, and requires every output to be
bit-identical; the step itself is checked against the oracle elsewhere.
Cases: bf16 with the one-wave final kernel (B = 64 and B = 300, the latter
over two row blocks), fp32, and the RNN head (no x0)."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_prev_amd as dsp
from draft_verify_sampling_prev_amd.binding import workspace
from draft_verify_sampling_prev_amd import synth
from gpu_util import host

pytestmark = pytest.mark.gpu


def _fill(ws: torch.Tensor, how: str):
    if how == "ones":
        ws.fill_(255)
    elif how == "zeros":
        ws.zero_()
    else:
        gen = torch.Generator().manual_seed(1234)
        ws.copy_(torch.randint(0, 256, (ws.numel(),), dtype=torch.uint8, generator=gen))


def _bits(outs: dict) -> dict:
    """Every output as bytes (bfloat16 tensors through their 16-bit patterns)."""
    raw = {k: (t.view(torch.int16) if t.dtype == torch.bfloat16 else t) for k, t in outs.items() if t is not None}
    return {k: np.ascontiguousarray(host(t)).view(np.uint8).copy() for k, t in raw.items()}


def _markov_step(g, wl, ws):
    seed = wl.philox_seed
    tok, p, lse = dsp.dspark_markov_draft(g.L, g.A, g.Bm, g.x0, seed, ws=ws)
    _, ell = dsp.dspark_schedule(g.z, g.temps, wl.budget)
    acc, out_tok, n_out, tp = dsp.dspark_verify(g.T, g.L, g.A, g.Bm, g.x0, tok, p, lse, ell, seed, ws=ws)
    torch.cuda.synchronize()
    return dict(tok=tok, p=p, lse=lse, ell=ell, acc=acc, out_tok=out_tok, n_out=n_out, tp=tp)


def _rnn_step(g, wl, ws):
    seed = wl.philox_seed
    gen = torch.Generator().manual_seed(wl.data_seed + 3)
    Wt = (torch.randn((wl.r, wl.r), generator=gen) / np.sqrt(wl.r)).to(g.L.dtype).to(g.L.device)
    tok, p, lse, H = dsp.dspark_rnn_draft(g.L, g.A, g.Bm, Wt, g.x0, seed, ws=ws)
    _, ell = dsp.dspark_schedule(g.z, g.temps, wl.budget)
    acc, out_tok, n_out, tp = dsp.dspark_rnn_verify(g.T, g.L, H, g.Bm, tok, p, lse, ell, seed, ws=ws)
    torch.cuda.synchronize()
    return dict(tok=tok, p=p, lse=lse, H=H, ell=ell, acc=acc, out_tok=out_tok, n_out=n_out, tp=tp)


@pytest.mark.parametrize("B,gamma,V,r,dtype,head", [(64, 5, 40000, 256, "bf16", "markov"),
                                                   (300, 4, 9000, 64, "bf16", "markov"),
                                                   (48, 3, 3000, 32, "f32", "markov"),
                                                   (40, 4, 5000, 64, "bf16", "rnn")])
def test_outputs_do_not_depend_on_workspace_contents(B, gamma, V, r, dtype, head):
    dev = torch.device("cuda:0")
    # Budget about half the candidates: requests with and without a rejection.
    wl = synth.tiny(B=B, gamma=gamma, V=V, r=r, budget=B * gamma // 2, dtype=dtype)
    print(f"case workspace {head} B={B} gamma={gamma} V={V} r={r} {dtype}", flush=True)
    g = synth.make_inputs(wl).to(dev)
    ws = workspace(B, gamma, V, r, dev)
    step = _markov_step if head == "markov" else _rnn_step
    ref = None
    for how in ("ones", "zeros", "random"):
        _fill(ws, how)
        torch.cuda.synchronize()
        out = step(g, wl, ws)
        got = _bits(out)
        if ref is None:
            ref = got
            acc, ell = host(out["acc"]), host(out["ell"])
            # both branches of the final kernel are taken
            assert (acc < ell).any() and (acc == ell).any(), (acc.tolist(), ell.tolist())
            continue
        for k in ref:
            assert np.array_equal(ref[k], got[k]), (how, k)
