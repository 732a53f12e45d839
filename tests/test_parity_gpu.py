"""GPU parity: the HIP path through the C ABI against the oracle, teacher-forced.

Bit-exact: verify lengths (given the GPU's own survivals), accepted counts and
token ids, except counted near-boundary flips: |u - boundary| < 1e-5 by the
parity protocol, and in addition every flip within 1e-6 of its boundary and
at most max(3, decisions / 250) flips per case (oracle/check.py flips_ok).
Probabilities within 1e-5 relative, log-normalisers within 1e-5, survivals
within 1e-5 relative.
"""
import time

import numpy as np
import pytest
import torch

from draft_verify_sampling_prev_amd import synth
from gpu_util import check_step, run_step, structural_checks
from oracle import check

pytestmark = pytest.mark.gpu



def _run_and_check(wl, seed=None, draft_rows=None, requests=None, data_seed=None, inp=None):
    seed = wl.philox_seed if seed is None else seed
    inp = synth.make_inputs(wl, seed=data_seed) if inp is None else inp
    print(f"case {wl.describe()} seed={seed:#x}", flush=True)
    out = run_step(inp, wl.budget, seed)
    structural_checks(out, wl.gamma)
    t0 = time.perf_counter()
    rep = check_step(inp, out, wl.budget, seed, draft_rows=draft_rows, requests=requests,
                     threads=check.default_threads())
    print("  ", rep.summary(), f"(oracle {time.perf_counter() - t0:.1f} s)", flush=True)
    assert rep.ok(), rep.summary()
    assert check.flips_ok(rep), rep.summary()
    return out, rep


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seed", [0x0123456789ABCDEF, 7, 2**63 + 12345])
def test_tiny_full_parity(dtype, seed):
    _run_and_check(synth.tiny(dtype=dtype), seed=seed)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_tiles_and_rank(dtype):
    # V = 1000 is not a multiple of the 128-column tile nor of the 8192 chunk;
    # r = 24 is not a multiple of the 32-wide k step; B = 300 spans two
    # 256-row blocks, the second ragged.
    wl = synth.tiny(B=300, gamma=3, V=1000, r=24, budget=450, dtype=dtype)
    _run_and_check(wl)


def test_rank256_ragged_batch_and_vocab():
    # r = 256: each draft step hands the next one its A rows in MFMA order.
    # B = 37 leaves a partial 16-row block, V = 3000 a partial 64-column tile.
    _run_and_check(synth.tiny(B=37, gamma=4, V=3000, r=256, budget=100, dtype="bf16"))


def test_rank256_two_row_blocks():
    # B = 300 at r = 256: two 256-row blocks in the tile kernels, the second ragged.
    wl = synth.tiny(B=300, gamma=3, V=2048, r=256, budget=600, dtype="bf16")
    _run_and_check(wl, requests=range(0, 300, 5))


@pytest.mark.parametrize("B,budget,rej_lo,rej_hi", [(512, 900, 129, 512), (256, 1280, 129, 256), (256, 100, 0, 111)])
def test_full_row_blocks_all_residual_paths(B, budget, rej_lo, rej_hi):
    """B a multiple of 256 at r = 256: the draft tile kernel's branch-free variant (every wave has rows), with
    one and two 256-row blocks, checked in full against the oracle.  The budgets put the residual tile pass in
    its different per-wave pipelines: with many verified drafts most requests reject and waves hold two blocks
    of rejected rows; with budget 100 only a few requests can reject, so most waves hold none."""
    wl = synth.tiny(B=B, gamma=5, V=3000, r=256, budget=budget, dtype="bf16")
    out, rep = _run_and_check(wl)
    n_rej = int((out["acc"] < out["ell"]).sum())
    print(f"  rejected requests: {n_rej}", flush=True)
    # more than 128 rejected rows: some waves of the residual pass hold two blocks of them; fewer than 112: some
    # waves hold none
    assert rej_lo <= n_rej <= rej_hi


@pytest.mark.parametrize("B,gamma,budget", [(1, 1, 1), (1, 16, 7), (3, 16, 48), (17, 2, 0), (9, 4, 10**9),
                                            (257, 3, 400)])  # 257: a second row block of one row
def test_edge_shapes_and_budgets(B, gamma, budget):
    wl = synth.tiny(B=B, gamma=gamma, V=256, r=8, budget=budget, dtype="bf16")
    out, _ = _run_and_check(wl)
    if budget == 0:
        assert np.all(out["ell"] == 0) and np.all(out["n_out"] == 1)
    if budget >= B * gamma:
        assert np.all(out["ell"] == gamma)


def test_many_vocab_chunks_and_row_blocks():
    # B = 600 -> three 256-row blocks in the Markov tiles; V = 20000 -> 3 chunks, ragged.
    wl = synth.tiny(B=600, gamma=4, V=20000, r=64, budget=1200, dtype="bf16")
    rows = [(b, k) for b in range(0, 600, 37) for k in (1, 2, 3, 4)]
    _run_and_check(wl, draft_rows=rows, requests=range(0, 600, 7))


def test_two_row_blocks_more_slots_than_slot_sums():
    """B = 300, V = 240000 (3750 tiles): two row blocks with more than 256 tile slots each, so the draft locate
    and the final kernel scan the tile sums in one level, as below B = 257 (with at most 256 slots they first
    pick a slot from per-slot sums; the load-sweep, mask and B = 300 cases cover that)."""
    import bench
    wl = synth.tiny(B=300, gamma=3, V=240000, r=64, budget=450, dtype="bf16")
    nT = (wl.V + 63) // 64
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert bench.tile_slots(nT, 2, cus, 12) > 256
    rows = [(b, k) for b in range(0, 300, 13) for k in (1, 2, 3)]
    out, _ = _run_and_check(wl, draft_rows=rows, requests=range(0, 300, 3))
    assert (out["acc"] < out["ell"]).sum() > 50  # many residual samples


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_long_vocabulary_generic_paths(dtype):
    # V = 600000: 74 target chunks (> 64, the accept kernel's per-lane chunk loop)
    # and 9375 bf16 tiles (> 64 * 64, the workgroup locate and final kernels).
    wl = synth.tiny(B=3, gamma=2, V=600000, r=16, budget=4, dtype=dtype)
    _run_and_check(wl)


def test_zero_markov_factors_reduce_to_plain_softmax():
    wl = synth.tiny(B=8, gamma=3, V=4096, r=32, budget=12, dtype="bf16")
    inp = synth.make_inputs(wl)
    inp.A.zero_()
    inp.Bm.zero_()
    out = run_step(inp, wl.budget, wl.philox_seed)
    rep = check_step(inp, out, wl.budget, wl.philox_seed)
    assert rep.ok(), rep.summary()


_HEADLINE = {}


def _headline_inputs():
    if not _HEADLINE:
        _HEADLINE["inp"] = synth.make_inputs(synth.dsv4())
    return _HEADLINE["inp"]


def test_headline_shape_full():
    """B=256, gamma=5, V=129280, r=256, bf16, budget 768, in the launch configuration the benchmark times:
    every one of the 1280 draft rows and every one of the 256 requests against the oracle."""
    wl = synth.dsv4()
    out, rep = _run_and_check(wl, inp=_headline_inputs())
    assert rep.decisions >= wl.B * wl.gamma + wl.B


def test_headline_shape_run_to_run_bitwise():
    """Two runs of the benchmarked step give identical bits in every output (the residual-row list is filled
    by an atomic slot counter in no fixed order; no result may depend on that order)."""
    wl = synth.dsv4()
    inp = _headline_inputs()
    a = run_step(inp, wl.budget, wl.philox_seed)
    b = run_step(inp, wl.budget, wl.philox_seed)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


def test_qwen_shape_sampled():
    wl = synth.qwen3_4b()
    g = np.random.default_rng(6)
    rows = [(int(b), int(k)) for b, k in zip(g.integers(0, wl.B, 24), g.integers(1, wl.gamma + 1, 24))]
    _run_and_check(wl, draft_rows=rows, requests=range(0, wl.B, 3))


def _sample(wl, rng_seed, n=16):
    g = np.random.default_rng(rng_seed)
    rows = [(int(b), int(k)) for b, k in zip(g.integers(0, wl.B, n), g.integers(1, wl.gamma + 1, n))]
    rows += [(0, 1), (wl.B - 1, wl.gamma)]
    reqs = sorted(set(int(b) for b in g.integers(0, wl.B, n)) | {0, wl.B - 1})
    return rows, reqs


@pytest.mark.parametrize("gamma", [4, 8, 12, 16])
def test_long_block_sampled(gamma):
    """Long-block sweep point: B=128, V=151936, r=256, bf16, every drafted token verified."""
    wl = synth.long_block(gamma)
    rows, reqs = _sample(wl, 100 + gamma)
    out, _ = _run_and_check(wl, draft_rows=rows, requests=reqs)
    assert np.all(out["ell"] == gamma)  # unbounded budget


_LOAD_SWEEP_INPUTS = {}


@pytest.mark.parametrize("mult", [1, 2, 4, 8])
def test_load_sweep_sampled(mult):
    """Load-sweep point: B=1024, gamma=8, V=129280, r=256, bf16, budget mult*B (four 256-row blocks)."""
    wl = synth.load_sweep(1024 * mult)
    if not _LOAD_SWEEP_INPUTS:  # the inputs do not depend on the budget
        _LOAD_SWEEP_INPUTS["inp"] = synth.make_inputs(wl)
    inp = _LOAD_SWEEP_INPUTS["inp"]
    print(f"case {wl.describe()} seed={wl.philox_seed:#x}", flush=True)
    out = run_step(inp, wl.budget, wl.philox_seed)
    structural_checks(out, wl.gamma)
    assert int(out["ell"].sum()) == min(wl.budget, wl.B * wl.gamma)
    rows, reqs = _sample(wl, 200 + mult, n=160)
    rep = check_step(inp, out, wl.budget, wl.philox_seed, draft_rows=rows, requests=reqs,
                     threads=check.default_threads())
    print("  ", rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert check.flips_ok(rep), rep.summary()
    if mult == 8:  # run to run, bitwise, at the B = 1024 shape (four row blocks, ~32 tiles per slot)
        again = run_step(inp, wl.budget, wl.philox_seed)
        for k in out:
            assert np.array_equal(out[k].view(np.uint8), again[k].view(np.uint8)), k


def test_full_batch_slots_past_the_staging():
    """B = 512, V = 110000 (1719 tiles): a full-batch launch gives each of 128 slots per row block 13-14 tiles,
    more than the 12 whose partials the LDS staging holds, so the staging is written out mid-launch.  Every draft
    row's sample depends on all of its tiles' partials, so sampled rows check every write-out; plus bitwise run
    to run."""
    wl = synth.tiny(B=512, gamma=2, V=110000, r=256, budget=700, dtype="bf16")
    inp = synth.make_inputs(wl)
    rows, reqs = _sample(wl, 321, n=96)
    out, _ = _run_and_check(wl, draft_rows=rows, requests=reqs, inp=inp)
    again = run_step(inp, wl.budget, wl.philox_seed)
    for k in out:
        assert np.array_equal(out[k].view(np.uint8), again[k].view(np.uint8)), k


def test_run_to_run_determinism():
    wl = synth.tiny(B=64, gamma=5, V=8192, r=64, budget=200, dtype="bf16")
    inp = synth.make_inputs(wl)
    a = run_step(inp, wl.budget, 11)
    b = run_step(inp, wl.budget, 11)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
