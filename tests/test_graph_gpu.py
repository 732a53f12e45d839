"""HIP-graph capture of a whole draft -> schedule -> verify step: every replay
must reproduce the eager results (the library records no memset nodes and
allocates nothing, so the step is capturable)."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_prev_amd as dsp
from draft_verify_sampling_prev_amd import binding, synth

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    wl = synth.tiny(B=48, gamma=5, V=4096, r=64, budget=100, dtype="bf16")
    inp = synth.make_inputs(wl)
    dev = torch.device("cuda:0")
    g = inp.to(dev)
    B, gamma, V, r = wl.B, wl.gamma, wl.V, wl.r
    ws = binding.workspace(B, gamma, V, r, dev)
    tok = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    p = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    lse = torch.empty((B, gamma), dtype=torch.float64, device=dev)
    theta = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    ell = torch.empty((B,), dtype=torch.int32, device=dev)
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    out_tok = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    n_out = torch.empty((B,), dtype=torch.int32, device=dev)
    tp = torch.empty((B, gamma), dtype=torch.float32, device=dev)

    def step(seed):
        dsp.dspark_markov_draft(g.L, g.A, g.Bm, g.x0, seed, ws=ws, out=(tok, p, lse))
        dsp.dspark_schedule(g.z, g.temps, wl.budget, survival=theta, out_len=ell)
        dsp.dspark_verify(g.T, g.L, g.A, g.Bm, g.x0, tok, p, lse, ell, seed, ws=ws, out=(acc, out_tok, n_out, tp))

    def snap():
        return [t.clone().cpu() for t in (tok, p, lse, theta, ell, acc, out_tok, n_out, tp)]

    seed = 1234
    step(seed)
    torch.cuda.synchronize()
    ref = snap()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(seed)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(seed)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (tok, p, lse, theta, ell, acc, out_tok, n_out, tp):
            t.fill_(-7)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snap()
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"replay {rep} differs"
