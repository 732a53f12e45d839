"""Teacher-forced parity checks of the GPU path against the oracle.

Test infrastructure only (used by ``tests/``, ``__graft_entry__.smoke()``).
Inputs are host numpy arrays: the synthetic inputs (widened to float32) and
the GPU path's outputs copied back.  Every GPU decision is recomputed by the
oracle from the GPU's own previous decisions (its previous draft token, its
verify lengths, its accepted count), so one near-boundary flip does not
cascade.  A disagreement is an *allowed flip* only when the oracle's own
uniform lies within ``FLIP_TOL`` of the decision boundary:
  accept test  |u - ratio| < 1e-5;
  sampling     the GPU token y differs from the oracle's x and the oracle's
               CDF boundary between them is within 1e-5 of u (in units of
               the total mass).
Anything else is a hard failure.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os
from typing import Iterable, List, Optional, Tuple

import numpy as np

from . import accept_scan, draft_row, final_token, rnn_state, select, survival, uniform

FLIP_TOL = 1e-5
# Flips observed between the GPU path and the oracle lie within 1e-7 of their boundary (the GPU sums fp32
# exponentials per tile and combines tiles in fp64; the oracle sums in fp64), at about one per 500 decisions at
# V = 129280, where a token's CDF interval is itself ~1e-5 wide.  The tests require every flip within
# MAX_FLIP_GAP, and at most max(3, decisions / 250) flips per case.
MAX_FLIP_GAP = 1e-6
P_RTOL = 1e-5       # probabilities, relative
LSE_ATOL = 1e-5     # log-normalisers, absolute
THETA_RTOL = 1e-5   # survivals, relative


@dataclasses.dataclass
class Report:
    checked: int = 0     # values compared (decisions, probabilities, states, survivals, lengths)
    decisions: int = 0   # sampling and accept decisions compared (the events a flip can occur in)
    draft_flips: int = 0
    accept_flips: int = 0
    final_flips: int = 0
    failures: List[str] = dataclasses.field(default_factory=list)
    flip_gaps: List[float] = dataclasses.field(default_factory=list)  # |u - boundary| of every allowed flip

    def fail(self, msg: str):
        if len(self.failures) < 50:
            self.failures.append(msg)

    def ok(self) -> bool:
        return not self.failures

    @property
    def flips(self) -> int:
        return self.draft_flips + self.accept_flips + self.final_flips

    def merge(self, other: "Report"):
        self.checked += other.checked
        self.decisions += other.decisions
        self.draft_flips += other.draft_flips
        self.accept_flips += other.accept_flips
        self.final_flips += other.final_flips
        self.flip_gaps.extend(other.flip_gaps)
        for f in other.failures:
            self.fail(f)

    def summary(self) -> str:
        gaps = f" max_flip_gap={max(self.flip_gaps):.2e}" if self.flip_gaps else ""
        return (f"checked={self.checked} decisions={self.decisions} draft_flips={self.draft_flips} "
                f"accept_flips={self.accept_flips} final_flips={self.final_flips}{gaps} failures={len(self.failures)}"
                + ("" if self.ok() else "\n  " + "\n  ".join(self.failures[:10])))


def flip_cap(rep: "Report") -> int:
    """Largest number of near-boundary flips a case may have: 3, or one per 250 decisions if more."""
    return max(3, -(-rep.decisions // 250))


def flips_ok(rep: "Report") -> bool:
    return rep.flips <= flip_cap(rep) and all(g < MAX_FLIP_GAP for g in rep.flip_gaps)


def default_threads() -> int:
    """Host threads for the oracle side of a check (the oracle's C calls release the GIL)."""
    return max(1, min(16, os.cpu_count() or 1))


def _parallel(fn, items: list, rep: Report, threads: int):
    """Run fn(chunk, report) over contiguous chunks of items on a thread pool and merge the reports in order."""
    if threads <= 1 or len(items) < 2 * threads:
        fn(items, rep)
        return
    n = threads * 4
    chunks = [items[len(items) * i // n: len(items) * (i + 1) // n] for i in range(n)]
    reps = [Report() for _ in chunks]
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda cr: fn(cr[0], cr[1]), zip(chunks, reps)))
    for r in reps:
        rep.merge(r)


def _sample_flip_gap(o_tok: int, y: int, o: dict) -> float:
    """Distance of u from the oracle's CDF boundary between the oracle token and the GPU token y
    (o: oracle row result queried at y: cdf_before = C_{y-1}/S, cdf_through = C_y/S)."""
    u = o["u"]
    return o["cdf_before"] - u if y > o_tok else u - o["cdf_through"]


def _sample_flip_allowed(o_tok: int, y: int, o: dict) -> bool:
    return _sample_flip_gap(o_tok, y, o) < FLIP_TOL


def check_draft(L, A, Bm, x0, seed, tok, p, lse, rep: Report, rows: Optional[Iterable[Tuple[int, int]]] = None,
                states=None, threads: int = 1):
    """L [B][g][V] f32, tok/p/lse GPU outputs [B][g].  rows: (b, k) pairs with k 1-based; default all.
    states [B][g][r] (RNN head): the operand of (b, k) is states[b][k-1] instead of A[x_{k-1}].
    threads > 1 spreads the rows over a thread pool."""
    B, gamma, V = L.shape
    if rows is None:
        rows = [(b, k) for b in range(B) for k in range(1, gamma + 1)]
    _parallel(lambda part, r: _check_draft_rows(L, A, Bm, x0, seed, tok, p, lse, r, part, states), list(rows), rep,
              threads)


def _check_draft_rows(L, A, Bm, x0, seed, tok, p, lse, rep: Report, rows, states):
    V = L.shape[2]
    for b, k in rows:
        if states is not None:
            A, prev = states[b], k - 1
        else:
            prev = int(x0[b]) if k == 1 else int(tok[b, k - 2])
        y = int(tok[b, k - 1])
        if not (0 <= y < V):
            rep.fail(f"draft b={b} k={k}: token {y} out of range")
            continue
        u = uniform(seed, b, k, 0)
        o = draft_row(L[b, k - 1], A, Bm, prev, u, query=y)
        rep.checked += 1
        rep.decisions += 1
        if o["tok"] != y:
            if _sample_flip_allowed(o["tok"], y, o):
                rep.draft_flips += 1
                rep.flip_gaps.append(_sample_flip_gap(o["tok"], y, o))
                continue
            rep.fail(f"draft b={b} k={k}: gpu token {y} oracle {o['tok']} (u={u:.8f}, "
                     f"C_before={o['cdf_before']:.8f}, C_through={o['cdf_through']:.8f})")
            continue
        if abs(float(p[b, k - 1]) - o["p"]) > P_RTOL * o["p"]:
            rep.fail(f"draft b={b} k={k}: p_d gpu {float(p[b, k - 1]):.9g} oracle {o['p']:.9g}")
        if abs(float(lse[b, k - 1]) - o["lse"]) > LSE_ATOL:
            rep.fail(f"draft b={b} k={k}: lse gpu {float(lse[b, k - 1]):.9g} oracle {o['lse']:.9g}")


def check_rnn_states(A, Wt, x0, tok, H_gpu, rep: Report, elem: str = "bf16",
                     rows: Optional[Iterable[Tuple[int, int]]] = None):
    """RNN-head states, teacher-forced: H_gpu[b][k-1] (widened to float) against
    tanh(W H_gpu[b][k-2] + A[x_{k-1}]) (h_0 = 0) from the oracle in double.  The GPU sums in fp32 and rounds
    each state to its element type, so the bound is half an ulp of that type (2^-8 relative for bf16, 2^-24
    for fp32), plus the fp32 error of the sum (tanh' <= 1) and a few fp32 ulps for tanh."""
    B, gamma, r = H_gpu.shape
    half_ulp = 2.0 ** -8 if elem == "bf16" else 2.0 ** -24
    if rows is None:
        rows = [(b, k) for b in range(B) for k in range(1, gamma + 1)]
    for b, k in rows:
        x = int(x0[b]) if k == 1 else int(tok[b, k - 2])
        h_prev = np.zeros(r, dtype=np.float32) if k == 1 else H_gpu[b, k - 2].astype(np.float32)
        ref = rnn_state(Wt, h_prev, A[x])
        pre_mag = np.abs(A[x].astype(np.float64)) + np.abs(Wt.astype(np.float64)).T @ np.abs(h_prev.astype(np.float64))
        got = H_gpu[b, k - 1].astype(np.float64)
        tol = half_ulp * np.abs(ref) + 2.0 ** -24 * (r + 4) * pre_mag + 2.0 ** -21
        rep.checked += r
        bad = np.abs(got - ref) > tol
        if bad.any():
            i = int(np.argmax(bad))
            rep.fail(f"rnn state b={b} k={k} i={i}: gpu {got[i]:.9g} oracle {ref[i]:.9g} (tol {tol[i]:.3g})")


def check_survival(z, temps, theta_gpu, rep: Report):
    ref = survival(z, temps).astype(np.float64)
    g = theta_gpu.astype(np.float64)
    bad = np.abs(g - ref) > THETA_RTOL * np.abs(ref) + 1e-38
    rep.checked += ref.size
    if bad.any():
        i = np.argwhere(bad)[0]
        rep.fail(f"survival mismatch at {tuple(i)}: gpu {g[tuple(i)]:.9g} oracle {ref[tuple(i)]:.9g}")


def check_select(theta_gpu, budget, len_gpu, rep: Report):
    """Bit-exact verify lengths given the GPU's own survivals."""
    ref = select(theta_gpu, budget)
    rep.checked += ref.size
    if not np.array_equal(ref, len_gpu.astype(np.int32)):
        i = int(np.argmax(ref != len_gpu))
        rep.fail(f"verify length mismatch at b={i}: gpu {int(len_gpu[i])} oracle {int(ref[i])}")


def check_verify(T, L, A, Bm, x0, tok, pd, ell, seed, acc, out_tok, n_out, target_p, rep: Report,
                 requests: Optional[Iterable[int]] = None, states=None, threads: int = 1):
    """Teacher-forced on the GPU's draft outputs, verify lengths and accepted counts.
    states [B][g][r] (RNN head): residual draft rows use states[b][k-1] as the operand.
    threads > 1 spreads the requests over a thread pool."""
    B = L.shape[0]
    if requests is None:
        requests = range(B)
    _parallel(lambda part, r: _check_verify_requests(T, L, A, Bm, x0, tok, pd, ell, seed, acc, out_tok, n_out,
                                                     target_p, r, part, states), [int(b) for b in requests], rep,
              threads)


def _check_verify_requests(T, L, A, Bm, x0, tok, pd, ell, seed, acc, out_tok, n_out, target_p, rep: Report,
                           requests, states):
    B, gamma, V = L.shape
    for b in requests:
        b = int(b)
        l = int(ell[b])
        a_g = int(acc[b])
        rep.checked += 1
        if not (0 <= a_g <= l):
            rep.fail(f"verify b={b}: accepted {a_g} outside [0, {l}]")
            continue
        a_o, pt, ratio, us = accept_scan(T[b], tok[b], pd[b], l, seed, b)
        if target_p is not None:
            for k in range(l):
                if abs(float(target_p[b, k]) - pt[k]) > P_RTOL * pt[k] + 1e-30:
                    rep.fail(f"verify b={b} k={k + 1}: p_t gpu {float(target_p[b, k]):.9g} oracle {pt[k]:.9g}")
            for k in range(l, gamma):
                if float(target_p[b, k]) != 0.0:
                    rep.fail(f"verify b={b} k={k + 1}: p_t beyond the verify length is {float(target_p[b, k])}")
        # GPU decisions: accept at positions < a_g, reject at a_g (if a_g < l)
        for k in range(min(a_g + 1, l)):
            rep.decisions += 1
            gpu_acc = k < a_g
            orc_acc = bool(us[k] < np.float32(ratio[k]))
            if gpu_acc != orc_acc:
                if abs(float(us[k]) - ratio[k]) < FLIP_TOL:
                    rep.accept_flips += 1
                    rep.flip_gaps.append(abs(float(us[k]) - ratio[k]))
                else:
                    rep.fail(f"verify b={b} k={k + 1}: gpu {'accept' if gpu_acc else 'reject'} but "
                             f"u={us[k]:.8f} ratio={ratio[k]:.8f}")
        if int(n_out[b]) != a_g + 1:
            rep.fail(f"verify b={b}: n_out {int(n_out[b])} != accepted + 1 = {a_g + 1}")
        for k in range(a_g):
            if int(out_tok[b, k]) != int(tok[b, k]):
                rep.fail(f"verify b={b}: out_tok[{k}] {int(out_tok[b, k])} != draft token {int(tok[b, k])}")
        for k in range(a_g + 1, gamma + 1):
            if int(out_tok[b, k]) != -1:
                rep.fail(f"verify b={b}: out_tok[{k}] = {int(out_tok[b, k])}, expected -1")
        y = int(out_tok[b, a_g])
        if not (0 <= y < V):
            rep.fail(f"verify b={b}: final token {y} out of range")
            continue
        if states is not None:  # operand rows states[b][0..g-1], addressed as "tokens" 0..g-1
            o = final_token(T[b], L[b], states[b], Bm, 0, np.arange(1, gamma + 1, dtype=np.int32), l, a_g, seed, b,
                            query=y)
        else:
            o = final_token(T[b], L[b], A, Bm, int(x0[b]), tok[b], l, a_g, seed, b, query=y)
        rep.decisions += 1
        if o["tok"] != y:
            if _sample_flip_allowed(o["tok"], y, o):
                rep.final_flips += 1
                rep.flip_gaps.append(_sample_flip_gap(o["tok"], y, o))
            else:
                kind = "residual" if a_g < l else "bonus"
                rep.fail(f"verify b={b} ({kind}, a={a_g}, l={l}): gpu token {y} oracle {o['tok']} "
                         f"(u={o['u']:.8f}, C_before={o['cdf_before']:.8f}, C_through={o['cdf_through']:.8f})")
