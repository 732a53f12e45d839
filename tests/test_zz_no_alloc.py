"""dspark_markov_draft_noalloc (the allocation-free draft entry point, whose
tile partials, A-row hand-over and slot aggregates live in the library's
static device scratch) against dspark_markov_draft with a caller workspace: bit-identical
outputs on two calls in a row, the second with a smaller input, and the
shape-ragged and headline cases; the first call on a fresh device looks the
scratch up."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_prev_amd as dsp
from draft_verify_sampling_prev_amd import synth

pytestmark = pytest.mark.gpu


def _pair(wl, seed):
    dev = torch.device("cuda:0")
    g = synth.make_inputs(wl).to(dev)
    print(f"case noalloc {wl.describe()} seed={seed:#x}", flush=True)
    ref = dsp.dspark_markov_draft(g.L, g.A, g.Bm, g.x0, seed)
    B, gamma = wl.B, wl.gamma
    out = (torch.full((B, gamma), -5, dtype=torch.int32, device=dev),
           torch.full((B, gamma), -5.0, dtype=torch.float32, device=dev),
           torch.full((B, gamma), -5.0, dtype=torch.float64, device=dev))
    got = dsp.dspark_markov_draft_noalloc(g.L, g.A, g.Bm, g.x0, seed, out=out)
    torch.cuda.synchronize()
    for a, b, name in zip(ref, got, ("tok", "p", "lse")):
        assert np.array_equal(a.cpu().numpy().view(np.uint8), b.cpu().numpy().view(np.uint8)), name


def test_noalloc_two_calls_second_smaller():
    # headline shape (rank 256: the A-row hand-over region is used), then a smaller, ragged one
    _pair(synth.dsv4(), 0x0123456789ABCDEF)
    _pair(synth.tiny(B=37, gamma=4, V=3000, r=256, budget=100, dtype="bf16"), 7)


def test_noalloc_small_then_fp32_and_ragged_rank():
    _pair(synth.tiny(B=300, gamma=3, V=1000, r=24, budget=450, dtype="bf16"), 11)
    _pair(synth.tiny(B=5, gamma=3, V=777 * 8, r=16, budget=9, dtype="f32"), 12)


def test_noalloc_two_row_blocks_rank256():
    # B above one 256-row block at rank 256: the locate reads the tile launch's slot aggregates, which the
    # static scratch holds after the A-row hand-over
    _pair(synth.tiny(B=512, gamma=3, V=20000, r=256, budget=700, dtype="bf16"), 13)
    _pair(synth.tiny(B=300, gamma=2, V=9000, r=256, budget=300, dtype="bf16"), 14)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    dev = torch.device("cuda:0")
    B, gamma, V, r = 2048, 8, 129280, 8
    L = torch.zeros((B, gamma, V), dtype=torch.bfloat16, device=dev)
    A = torch.zeros((V, r), dtype=torch.bfloat16, device=dev)
    Bm = torch.zeros((r, V), dtype=torch.bfloat16, device=dev)
    x0 = torch.zeros((B,), dtype=torch.int32, device=dev)
    with pytest.raises(dsp.DsparkError, match="scratch"):
        dsp.dspark_markov_draft_noalloc(L, A, Bm, x0, 1)
