"""GPU parity with vocabulary masks: logits of -inf in the draft and target
rows, as constrained decoding sets them, through the C ABI against the oracle.

Per request (the same mask at every position of its draft and target rows):
half the vocabulary masked in one contiguous range (whole tiles, tile slots
and target chunks without a finite value), all but five tokens masked, all but
one token masked (the draft then samples it with probability 1 and every
verified draft is accepted), or no mask.  Masked tiles carry the partial
(-inf, 0) and weigh nothing in the draft's two-level and one-level locates,
the target normalisers, the residual and the bonus samples.  Every draft row
and every request is checked, teacher-forced, as the other parity tests do.
Cases: B = 300 (two 256-row blocks: the locate reads slot aggregates),
B = 64 at rank 256 (one row block, the one-level locate, the A-row hand-over),
fp32 logits, a 270000-token vocabulary (more than 4096 tiles: the generic
locate and final kernels) and B = 512 at V = 129280 (full-batch launches that write their staged
partials out every 12 tiles and fold the slot aggregates there; sampled rows
and requests, every mask kind among them).
"""
import numpy as np
import pytest
import torch

from draft_verify_sampling_prev_amd import synth
from gpu_util import check_step, run_step, structural_checks
from oracle import check

pytestmark = pytest.mark.gpu


def _mask(inp, V: int, seed: int):
    """Applies the per-request masks in place (bf16 -inf in L and T); returns the kinds."""
    rng = np.random.default_rng(seed)
    B = inp.L.shape[0]
    kinds = []
    ninf = float("-inf")
    for b in range(B):
        kind = b % 4
        if kind == 0:
            lo, hi = V // 4, 3 * V // 4
            inp.L[b, :, lo:hi] = ninf
            inp.T[b, :, lo:hi] = ninf
        elif kind in (1, 2):
            keep = rng.choice(V, size=5 if kind == 1 else 1, replace=False)
            m = torch.ones(V, dtype=torch.bool)
            m[torch.from_numpy(keep)] = False
            inp.L[b][:, m] = ninf
            inp.T[b][:, m] = ninf
        kinds.append(kind)
    return np.array(kinds)


@pytest.mark.parametrize("B,gamma,V,r,dtype", [(300, 3, 24000, 64, "bf16"), (64, 4, 24000, 256, "bf16"),
                                                (48, 3, 3000, 32, "f32"), (8, 2, 270000, 64, "bf16")])
def test_vocabulary_masks_match_the_oracle(B, gamma, V, r, dtype):
    wl = synth.tiny(B=B, gamma=gamma, V=V, r=r, budget=B * gamma // 2, dtype=dtype)
    inp = synth.make_inputs(wl)
    kinds = _mask(inp, V, seed=5 + B)
    print(f"case masks B={B} gamma={gamma} V={V} r={r} {dtype}", flush=True)
    out = run_step(inp, wl.budget, wl.philox_seed)
    structural_checks(out, gamma)
    # the single-token requests draft that token with probability 1 (up to the rounding of the normaliser)
    # and accept their verified drafts (a rejection needs u within ~1e-6 of 1)
    one = kinds == 2
    assert np.allclose(out["p"][one], 1.0, rtol=0.0, atol=1e-6), out["p"][one]
    assert (out["acc"][one] == out["ell"][one]).mean() > 0.99
    rep = check_step(inp, out, wl.budget, wl.philox_seed, threads=check.default_threads())
    print("  ", rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert check.flips_ok(rep), rep.summary()


def test_vocabulary_masks_full_batch_sampled():
    B, gamma, V, r = 512, 2, 129280, 256
    wl = synth.tiny(B=B, gamma=gamma, V=V, r=r, budget=B * gamma // 2, dtype="bf16")
    inp = synth.make_inputs(wl)
    kinds = _mask(inp, V, seed=17)
    print(f"case masks B={B} gamma={gamma} V={V} r={r} (sampled)", flush=True)
    out = run_step(inp, wl.budget, wl.philox_seed)
    structural_checks(out, gamma)
    g = np.random.default_rng(23)
    reqs = sorted(set(int(b) for b in g.integers(0, B, 24)) | {0, 1, 2, 3, B - 1})
    rows = [(b, k) for b in reqs for k in range(1, gamma + 1)]
    assert set(kinds[reqs]) == {0, 1, 2, 3}
    rep = check_step(inp, out, wl.budget, wl.philox_seed, draft_rows=rows, requests=reqs,
                     threads=check.default_threads())
    print("  ", rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert check.flips_ok(rep), rep.summary()
