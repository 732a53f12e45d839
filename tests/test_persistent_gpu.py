"""The persistent draft (all gamma steps in one cooperative launch with Bm
held on chip, used at bf16 rank 256 when B <= compute units and
V <= 512 * compute units) against the per-step launches: bit-identical
tokens, p_d, lse_d (and confidence logits), oracle parity, and the
device-wide barrier's give-up path driven from the host."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_prev_amd as dsp
from draft_verify_sampling_prev_amd import binding, synth
from gpu_util import check_step, run_step
from oracle import check

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().numpy().view(np.uint8)


def _draft_both(wl, seed, conf=False):
    dev = torch.device("cuda:0")
    g = synth.make_inputs(wl).to(dev)
    print(f"case persistent {wl.describe()} seed={seed:#x} conf={conf}", flush=True)
    wc = (torch.randn(wl.r, generator=torch.Generator().manual_seed(5)) * 0.5).to(g.L.dtype).to(dev)

    def draft():
        ws = binding.workspace(wl.B, wl.gamma, wl.V, wl.r, dev)
        if conf:
            out = dsp.dspark_markov_draft_conf(g.L, g.A, g.Bm, g.x0, seed, g.z, wc, ws=ws)
        else:
            out = dsp.dspark_markov_draft(g.L, g.A, g.Bm, g.x0, seed, ws=ws)
        binding.dspark_draft_status(wl.B, wl.gamma, wl.V, wl.r, ws=ws)
        return out

    try:
        binding.debug_draft()  # the persistent draft (enabled for the test)
        persistent = draft()
        binding.debug_draft(per_step_only=True)
        per_step = draft()
    finally:
        binding.debug_draft(per_step_only=True)
    torch.cuda.synchronize()
    for a, b, name in zip(persistent, per_step, ("tok", "p", "lse", "z")):
        assert np.array_equal(_bits(a), _bits(b)), name
    return persistent


@pytest.mark.parametrize("case", [
    dict(B=37, gamma=4, V=3000, r=256, budget=100),      # ragged batch block and last tile, most waves idle
    dict(B=1, gamma=16, V=2048 * 8, r=256, budget=7),     # one request, the longest block
    dict(B=256, gamma=1, V=129280, r=256, budget=128),    # one step (a single device-wide barrier)
    dict(B=200, gamma=3, V=16384 * 8, r=256, budget=300),  # V = 131072: every wave of the chip owns a tile
], ids=lambda c: f"B{c['B']}-g{c['gamma']}-V{c['V']}")
def test_persistent_equals_per_step(case):
    _draft_both(synth.tiny(dtype="bf16", **case), 0x0123456789ABCDEF)


def test_persistent_equals_per_step_headline_and_oracle():
    wl = synth.dsv4()
    _draft_both(wl, wl.philox_seed)
    _draft_both(wl, 12345, conf=True)
    inp = synth.make_inputs(wl)
    out = run_step(inp, wl.budget, 777)  # the persistent path, checked against the oracle on every row
    rep = check_step(inp, out, wl.budget, 777, threads=check.default_threads())
    print("  ", rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert rep.flips <= 3


def test_barrier_give_up_is_reported_and_recovers():
    """A barrier told to wait for an arrival that never comes gives up after a few polls: every workgroup
    exits, the status reports it, and the next draft (normal again) is complete and correct."""
    wl = synth.tiny(B=64, gamma=3, V=8192, r=256, budget=100, dtype="bf16")
    dev = torch.device("cuda:0")
    g = synth.make_inputs(wl).to(dev)
    ws = binding.workspace(wl.B, wl.gamma, wl.V, wl.r, dev)
    ref = dsp.dspark_markov_draft(g.L, g.A, g.Bm, g.x0, 99, ws=ws)
    binding.dspark_draft_status(wl.B, wl.gamma, wl.V, wl.r, ws=ws)
    try:
        binding.debug_draft(phantom_arrivals=1, poll_limit=2000)
        dsp.dspark_markov_draft(g.L, g.A, g.Bm, g.x0, 99, ws=ws)
        with pytest.raises(dsp.DsparkError, match="gave up"):
            binding.dspark_draft_status(wl.B, wl.gamma, wl.V, wl.r, ws=ws)
    finally:
        binding.debug_draft()
    again = dsp.dspark_markov_draft(g.L, g.A, g.Bm, g.x0, 99, ws=ws)
    binding.dspark_draft_status(wl.B, wl.gamma, wl.V, wl.r, ws=ws)
    for a, b in zip(ref, again):
        assert np.array_equal(_bits(a), _bits(b))
