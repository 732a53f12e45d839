"""Calibrate the synthetic workloads on their held-out seeds (run by hand; it
writes tests/golden/workload_calibration.json, and the constants it prints are
the ones draft_verify_sampling_prev_amd/synth.py holds).

1. dsv4-serving-shaped (B=256, gamma=5, V=129280): the draft-noise level
   sigma_k of each position is set so that the expected conditional acceptance
   alpha_k = E[ sum_j min(p_t,k(j), p_d,k(j)) ] -- the acceptance probability
   of the rejection rule for a draft drawn from p_d -- equals the suffix-decay
   example's 0.85/0.78/0.68/0.54/0.38 (llm-wiki.hwlabs.dev explainer).  The
   expectation is over the held-out batch's 256 rows, with the rows' noise
   draws fixed, the bf16 rounding of the draft logits included, and the Markov
   bias of the token the oracle's draft sampled (the bias is ~0.006 in size).
   sigma_k is found by bisection (alpha decreases with sigma).  The realised
   acceptance of an oracle step that verifies every drafted token is reported
   beside it.
2. load-sweep (B=1024, gamma=8): sequential temperature scaling
   (calibration.fit_sts) on the survival labels of one oracle step of the
   held-out batch with every drafted token verified.

Held-out seed = data seed + 8000 (the data seeds are 1000 + workload index).
Uses the oracle (CPU) only; nothing here comes from the GPU path.
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from draft_verify_sampling_prev_amd import calibration as cal  # noqa: E402
from draft_verify_sampling_prev_amd import synth  # noqa: E402

HELD_OUT = 8000
THREADS = max(1, min(16, os.cpu_count() or 1))


def _f32(t):
    return np.ascontiguousarray(t.float().numpy())


def alpha_of_sigma(T32_k, eps_k, delta_k, sigma):
    """Mean over rows of sum_j min(softmax(T), softmax(L + Delta)), L = bf16(eps * sigma + T32) as synth draws it."""
    L = (eps_k * np.float32(sigma) + T32_k).to(torch.bfloat16).double() + delta_k
    pt = torch.softmax(T32_k.to(torch.bfloat16).double(), -1)
    pd = torch.softmax(L, -1)
    return float(torch.minimum(pt, pd).sum(-1).mean())


def calibrate_dsv4():
    wl = synth.dsv4()
    seed = wl.data_seed + HELD_OUT
    B, gamma, V, r = wl.B, wl.gamma, wl.V, wl.r
    # the draws of synth.make_inputs, in its order
    g = torch.Generator().manual_seed(seed)
    T32 = torch.randn((B, gamma + 1, V), generator=g, dtype=torch.float32).mul_(2.0)
    eps = torch.randn((B, gamma, V), generator=g, dtype=torch.float32)
    inp = synth.make_inputs(wl, seed=seed)
    A, Bm = _f32(inp.A), _f32(inp.Bm)
    # Markov bias of the tokens an oracle draft at the current sigma conditions on
    tok, _, _ = oracle.markov_draft(_f32(inp.L), A, Bm, inp.x0.numpy(), wl.philox_seed, threads=THREADS)
    prev = np.concatenate([inp.x0.numpy()[:, None], tok[:, :-1]], axis=1)
    targets = synth.SUFFIX_DECAY[:gamma]
    sigmas = []
    for k in range(gamma):
        delta = torch.from_numpy(A[prev[:, k]].astype(np.float64) @ Bm.astype(np.float64))
        lo, hi = 0.01, 4.0
        for _ in range(22):
            mid = 0.5 * (lo + hi)
            if alpha_of_sigma(T32[:, k], eps[:, k], delta, mid) > targets[k]:
                lo = mid
            else:
                hi = mid
        sigmas.append(round(0.5 * (lo + hi), 4))
        print(f"dsv4 k={k + 1}: sigma {sigmas[-1]} (target alpha {targets[k]})", flush=True)
    # check: expected and realised acceptance at the calibrated sigmas
    wl2 = synth.Workload(**{**wl.__dict__, "sigma": tuple(sigmas)})
    inp2 = synth.make_inputs(wl2, seed=seed)
    L2, T2 = _f32(inp2.L), _f32(inp2.T)
    tok2, p2, _ = oracle.markov_draft(L2, A, Bm, inp2.x0.numpy(), wl.philox_seed, threads=THREADS)
    prev2 = np.concatenate([inp2.x0.numpy()[:, None], tok2[:, :-1]], axis=1)
    expected = []
    for k in range(gamma):
        delta = torch.from_numpy(A[prev2[:, k]].astype(np.float64) @ Bm.astype(np.float64))
        expected.append(round(alpha_of_sigma(T32[:, k], eps[:, k], delta, sigmas[k]), 4))
    ell = np.full(B, gamma, dtype=np.int32)
    acc, _, _, _ = oracle.verify(T2, L2, A, Bm, inp2.x0.numpy(), tok2, p2, ell, wl.philox_seed, threads=THREADS)
    realised = []
    for k in range(1, gamma + 1):
        reach = acc >= k - 1
        realised.append(round(float((acc[reach] >= k).mean()), 4))
    return {"workload": wl.name, "held_out_seed": seed, "target_alpha": list(targets), "sigma": sigmas,
            "expected_alpha": expected, "realised_alpha_one_step": realised,
            "previous_sigma": list(synth.DSV4_SIGMA)}


def fit_load_sweep():
    wl = synth.load_sweep(1024, temps=tuple(1.0 + 0.1 * k for k in range(1, 9)))
    seed = wl.data_seed + HELD_OUT
    inp = synth.make_inputs(wl, seed=seed)
    B, gamma = wl.B, wl.gamma
    L, T, A, Bm = _f32(inp.L), _f32(inp.T), _f32(inp.A), _f32(inp.Bm)
    x0 = inp.x0.numpy()
    t0 = time.time()
    tok, p, _ = oracle.markov_draft(L, A, Bm, x0, wl.philox_seed, threads=THREADS)
    ell = np.full(B, gamma, dtype=np.int32)
    acc, _, _, _ = oracle.verify(T, L, A, Bm, x0, tok, p, ell, wl.philox_seed, threads=THREADS)
    print(f"load-sweep held-out oracle step: {time.time() - t0:.1f} s", flush=True)
    labels = cal.survival_labels(acc, gamma)
    z = inp.z.numpy()
    temps, errs = cal.fit_sts(z, labels)
    before = cal.survival(z, np.asarray(wl.temps, dtype=np.float32))
    ece_before = [round(cal.ece(before[:, k], labels[:, k]), 4) for k in range(gamma)]
    return {"workload": "load-sweep", "held_out_seed": seed, "temps_before": [round(t, 4) for t in wl.temps],
            "temps": [round(float(t), 4) for t in temps], "ece_before": ece_before,
            "ece_after": [round(float(e), 4) for e in errs],
            "survival_rate": [round(float(v), 4) for v in labels.mean(0)]}


def main():
    out = {"dsv4": calibrate_dsv4(), "load_sweep": fit_load_sweep(),
           "script": "tests/calibrate_workloads.py (oracle on the held-out seeds)"}
    path = os.path.join(ROOT, "tests", "golden", "workload_calibration.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
