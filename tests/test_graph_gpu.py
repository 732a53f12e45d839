"""HIP-graph capture of a whole draft -> schedule -> verify step: every replay
must reproduce the eager results (the library records no memset nodes and
allocates nothing, so the step is capturable)."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_prev_amd as dsp
from draft_verify_sampling_prev_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,fused", [(dict(B=48, gamma=5, V=4096, r=64, budget=100), False),
                                         (dict(B=48, gamma=5, V=4096, r=64, budget=100), True),
                                         (dict(B=300, gamma=3, V=9000, r=256, budget=450), False)],
                         ids=["B48", "B48-fused-schedule", "B300-two-level"])
def test_graph_replays_match_eager(shape, fused):
    """B = 300 at rank 256: the locate reads slot aggregates and hands over A rows; fused: the schedule runs
    inside the draft call (dspark_markov_draft_sched)."""
    wl = synth.tiny(**shape, dtype="bf16")
    print(f"case graph {wl.describe()} fused={fused}", flush=True)
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
        if fused:
            dsp.dspark_markov_draft_sched(g.L, g.A, g.Bm, g.x0, seed, g.z, g.temps, wl.budget, ws=ws,
                                          out=(tok, p, lse), survival=theta, out_len=ell)
        else:
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


def test_graph_replays_with_device_seed_draw_fresh_uniforms():
    """With the seed in device memory, a captured step replayed after each write of a new seed draws that
    seed's uniforms: every replay equals the eager step run with the same seed, replays with different
    seeds differ, and one replay is checked against the oracle."""
    from gpu_util import check_step, host
    from oracle import check

    wl = synth.tiny(B=48, gamma=5, V=4096, r=64, budget=100, dtype="bf16")
    inp = synth.make_inputs(wl)
    dev = torch.device("cuda:0")
    g = inp.to(dev)
    B, gamma, V, r = wl.B, wl.gamma, wl.V, wl.r
    ws = binding.workspace(B, gamma, V, r, dev)
    bufs = dict(tok=torch.empty((B, gamma), dtype=torch.int32, device=dev),
                p=torch.empty((B, gamma), dtype=torch.float32, device=dev),
                lse=torch.empty((B, gamma), dtype=torch.float64, device=dev),
                theta=torch.empty((B, gamma), dtype=torch.float32, device=dev),
                ell=torch.empty((B,), dtype=torch.int32, device=dev),
                acc=torch.empty((B,), dtype=torch.int32, device=dev),
                out_tok=torch.empty((B, gamma + 1), dtype=torch.int32, device=dev),
                n_out=torch.empty((B,), dtype=torch.int32, device=dev),
                tp=torch.empty((B, gamma), dtype=torch.float32, device=dev))
    b = bufs
    seed_t = torch.zeros((1,), dtype=torch.int64, device=dev)

    def step(seed):
        dsp.dspark_markov_draft(g.L, g.A, g.Bm, g.x0, seed, ws=ws, out=(b["tok"], b["p"], b["lse"]))
        dsp.dspark_schedule(g.z, g.temps, wl.budget, survival=b["theta"], out_len=b["ell"])
        dsp.dspark_verify(g.T, g.L, g.A, g.Bm, g.x0, b["tok"], b["p"], b["lse"], b["ell"], seed, ws=ws,
                          out=(b["acc"], b["out_tok"], b["n_out"], b["tp"]))

    def snap():
        return {k: host(v.clone()) for k, v in bufs.items()}

    seeds = [0x0123456789ABCDEF, 7, 2**63 + 12345, 99]
    eager = {}
    for sd in seeds:
        step(sd)
        torch.cuda.synchronize()
        eager[sd] = snap()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seed_t.fill_(5)
        step(seed_t)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(seed_t)
    torch.cuda.synchronize()
    replays = {}
    for sd in seeds + seeds[:1]:
        for v in bufs.values():
            v.fill_(-7)
        seed_t.fill_(sd - 2**64 if sd >= 2**63 else sd)  # the same 64 bits, as a signed int64
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snap()
        for k in got:
            assert np.array_equal(got[k].view(np.uint8), eager[sd][k].view(np.uint8)), (hex(sd), k)
        replays[sd] = got
    assert not np.array_equal(replays[seeds[0]]["tok"], replays[seeds[1]]["tok"])
    rep = check_step(inp, replays[seeds[2]], wl.budget, seeds[2])
    assert rep.ok(), rep.summary()
    assert check.flips_ok(rep), rep.summary()
