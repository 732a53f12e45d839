"""CPU oracle of the DSpark per-step token path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it.  The arithmetic lives in ``dspark_oracle.c`` (plain sequential C,
double precision); this module only compiles it with gcc and marshals numpy
arrays through ctypes.

Every function takes host numpy arrays.  Logits and Markov factors are passed
as float32 (bf16 values widen to float32 exactly).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dspark_oracle.c")
# DSPARK_ORACLE_LIB selects another build of the same source (the sanitizer
# build of the CPU tests); it is then loaded as given, never rebuilt.
_LIB_OVERRIDE = os.environ.get("DSPARK_ORACLE_LIB")
_LIB = _LIB_OVERRIDE or os.path.join(_HERE, "liboracle.so")

ORC_OK = 0


class RowOut(ctypes.Structure):
    _fields_ = [
        ("tok", ctypes.c_int32),
        ("degenerate", ctypes.c_int32),
        ("p", ctypes.c_double),
        ("lse", ctypes.c_double),
        ("mass", ctypes.c_double),
        ("cdf_before", ctypes.c_double),
        ("cdf_through", ctypes.c_double),
        ("u", ctypes.c_float),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


GCC_FLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-pthread"]


def build(out: str = None, extra=()) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction) into `out`
    (default: the in-tree liboracle.so); `extra` adds flags (e.g. sanitizers)."""
    out = out or os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", *GCC_FLAGS, *extra, _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not _LIB_OVERRIDE and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p


def _declare(L):
    L.orc_philox4x32_10.argtypes = [_P, _P, _P]
    L.orc_philox4x32_10.restype = None
    L.orc_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
    L.orc_uniform.restype = ctypes.c_float
    L.orc_uniform_batch.argtypes = [ctypes.c_uint64, _P, _P, _P, ctypes.c_int, _P]
    L.orc_uniform_batch.restype = None
    L.orc_inverse_cdf.argtypes = [_P, ctypes.c_int, ctypes.c_float, _P]
    L.orc_inverse_cdf.restype = ctypes.c_int
    L.orc_inverse_cdf_batch.argtypes = [_P, ctypes.c_int, _P, ctypes.c_int, _P]
    L.orc_inverse_cdf_batch.restype = None
    L.orc_logsumexp.argtypes = [_P, ctypes.c_int]
    L.orc_logsumexp.restype = ctypes.c_double
    L.orc_markov_logits.argtypes = [_P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P]
    L.orc_markov_logits.restype = None
    L.orc_draft_row.argtypes = [_P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                ctypes.c_int, ctypes.POINTER(RowOut)]
    L.orc_draft_row.restype = ctypes.c_int
    L.orc_markov_draft.argtypes = [_P, _P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_uint64, _P, _P, _P]
    L.orc_markov_draft.restype = ctypes.c_int
    L.orc_survival.argtypes = [_P, _P, ctypes.c_int, ctypes.c_int, _P]
    L.orc_survival.restype = None
    L.orc_rnn_state.argtypes = [_P, _P, _P, ctypes.c_int, _P]
    L.orc_rnn_state.restype = None
    L.orc_markov_confidence.argtypes = [_P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P]
    L.orc_markov_confidence.restype = ctypes.c_int
    L.orc_select.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int64, _P]
    L.orc_select.restype = ctypes.c_int
    L.orc_select_objective.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, ctypes.c_int, ctypes.c_int64, _P,
                                       ctypes.POINTER(ctypes.c_int64)]
    L.orc_select_objective.restype = ctypes.c_int
    L.orc_select_threshold.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_float, _P]
    L.orc_select_threshold.restype = None
    L.orc_accept_scan.argtypes = [_P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_int,
                                  _P, _P, _P]
    L.orc_accept_scan.restype = ctypes.c_int
    L.orc_final_token.argtypes = [_P, _P, _P, _P, ctypes.c_int32, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                  ctypes.POINTER(RowOut)]
    L.orc_final_token.restype = ctypes.c_int
    L.orc_verify.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             ctypes.c_int, ctypes.c_uint64, _P, _P, _P, _P]
    L.orc_verify.restype = ctypes.c_int
    L.orc_markov_draft_mt.argtypes = L.orc_markov_draft.argtypes + [ctypes.c_int]
    L.orc_markov_draft_mt.restype = ctypes.c_int
    L.orc_verify_mt.argtypes = L.orc_verify.argtypes + [ctypes.c_int]
    L.orc_verify_mt.restype = ctypes.c_int


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _u32(a):
    return np.ascontiguousarray(a, dtype=np.uint32)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != ORC_OK:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


# ----------------------------------------------------------------------------- Philox / uniforms
def philox4x32_10(ctr, key):
    c = _u32(ctr)
    k = _u32(key)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed: int, b: int, k: int, d: int) -> float:
    return float(lib().orc_uniform(ctypes.c_uint64(seed), b, k, d))


def uniforms(seed: int, b, k, d) -> np.ndarray:
    b, k, d = np.broadcast_arrays(np.asarray(b), np.asarray(k), np.asarray(d))
    bb, kk, dd = _u32(b.ravel()), _u32(k.ravel()), _u32(d.ravel())
    out = np.zeros(bb.size, dtype=np.float32)
    lib().orc_uniform_batch(ctypes.c_uint64(seed), _ptr(bb), _ptr(kk), _ptr(dd), bb.size, _ptr(out))
    return out.reshape(b.shape)


# ----------------------------------------------------------------------------- sampler
def inverse_cdf(w, u: float) -> int:
    ww = _f64(w)
    return int(lib().orc_inverse_cdf(_ptr(ww), ww.size, ctypes.c_float(u), None))


def inverse_cdf_batch(w, us) -> np.ndarray:
    ww = _f64(w)
    uu = _f32(us)
    out = np.zeros(uu.size, dtype=np.int32)
    lib().orc_inverse_cdf_batch(_ptr(ww), ww.size, _ptr(uu), uu.size, _ptr(out))
    return out


# ----------------------------------------------------------------------------- draft
def logsumexp(row) -> float:
    r = _f32(row)
    return float(lib().orc_logsumexp(_ptr(r), r.size))


def markov_logits(L_row, A, Bm, prev: int) -> np.ndarray:
    Lr, Aa, Bb = _f32(L_row), _f32(A), _f32(Bm)
    V, r = Lr.size, Aa.shape[1]
    f = np.zeros(V, dtype=np.float64)
    lib().orc_markov_logits(_ptr(Lr), _ptr(Aa), _ptr(Bb), V, r, int(prev), _ptr(f))
    return f


def draft_row(L_row, A, Bm, prev: int, u: float, query: int = -1) -> dict:
    Lr, Aa, Bb = _f32(L_row), _f32(A), _f32(Bm)
    V, r = Lr.size, Aa.shape[1]
    o = RowOut()
    _check(lib().orc_draft_row(_ptr(Lr), _ptr(Aa), _ptr(Bb), V, r, int(prev), ctypes.c_float(u), int(query),
                               ctypes.byref(o)), "draft_row")
    return o.as_dict()


def markov_draft(L, A, Bm, x0, seed: int, threads: int = 1):
    """Free-running draft.  L [B][gamma][V], A [V][r], Bm [r][V], x0 [B].
    threads > 1 splits the requests over that many POSIX threads (same results)."""
    Ll, Aa, Bb, xx = _f32(L), _f32(A), _f32(Bm), _i32(x0)
    B, gamma, V = Ll.shape
    r = Aa.shape[1]
    tok = np.zeros((B, gamma), dtype=np.int32)
    p = np.zeros((B, gamma), dtype=np.float32)
    lse = np.zeros((B, gamma), dtype=np.float64)
    args = (_ptr(Ll), _ptr(Aa), _ptr(Bb), _ptr(xx), B, gamma, V, r, ctypes.c_uint64(seed), _ptr(tok), _ptr(p),
            _ptr(lse))
    if threads > 1:
        _check(lib().orc_markov_draft_mt(*args, int(threads)), "markov_draft_mt")
    else:
        _check(lib().orc_markov_draft(*args), "markov_draft")
    return tok, p, lse


# ----------------------------------------------------------------------------- schedule
def survival(z, T) -> np.ndarray:
    zz, TT = _f32(z), _f32(T)
    B, gamma = zz.shape
    th = np.zeros((B, gamma), dtype=np.float32)
    lib().orc_survival(_ptr(zz), _ptr(TT), B, gamma, _ptr(th))
    return th


def rnn_state(Wt, h_prev, a) -> np.ndarray:
    """One RNN-head update in double: tanh(Wt^T h_prev + a) (Wt[j][i] multiplies h_prev[j] into output i)."""
    W, h, aa = _f32(Wt), _f32(h_prev), _f32(a)
    r = aa.shape[0]
    out = np.zeros(r, dtype=np.float64)
    lib().orc_rnn_state(_ptr(W), _ptr(h), _ptr(aa), r, _ptr(out))
    return out


def markov_confidence(A, wc, x0, tok, z0) -> np.ndarray:
    """z[b][k] = z0[b][k] + <A[x_{k-1}], wc> (x_0 = x0[b], x_{k-1} = tok[b][k-2])."""
    AA, ww, xx, tt, zz = _f32(A), _f32(wc), _i32(x0), _i32(tok), _f32(z0)
    V, r = AA.shape
    B, gamma = zz.shape
    z = np.zeros((B, gamma), dtype=np.float32)
    _check(lib().orc_markov_confidence(_ptr(AA), _ptr(ww), _ptr(xx), _ptr(tt), _ptr(zz), B, gamma, V, r, _ptr(z)),
           "markov_confidence")
    return z


def select(theta, budget: int) -> np.ndarray:
    th = _f32(theta)
    B, gamma = th.shape
    ln = np.zeros(B, dtype=np.int32)
    _check(lib().orc_select(_ptr(th), B, gamma, ctypes.c_int64(int(budget)), _ptr(ln)), "select")
    return ln


def select_objective(theta, step_time, max_admit: int):
    """Objective-based admission (greedy order, early stop); returns (len, admitted)."""
    th, st = _f32(theta), _f32(step_time)
    B, gamma = th.shape
    ln = np.zeros(B, dtype=np.int32)
    adm = ctypes.c_int64(0)
    _check(lib().orc_select_objective(_ptr(th), B, gamma, _ptr(st), int(st.shape[0]), ctypes.c_int64(int(max_admit)),
                                      _ptr(ln), ctypes.byref(adm)), "select_objective")
    return ln, int(adm.value)


def select_threshold(theta, tau: float) -> np.ndarray:
    th = _f32(theta)
    B, gamma = th.shape
    ln = np.zeros(B, dtype=np.int32)
    lib().orc_select_threshold(_ptr(th), B, gamma, ctypes.c_float(float(tau)), _ptr(ln))
    return ln


# ----------------------------------------------------------------------------- verify
def accept_scan(T_b, tok_b, pd_b, ell: int, seed: int, b: int):
    """Returns (a, pt[ell], ratio[ell], u[ell]) for one request."""
    Tb, tb, pb = _f32(T_b), _i32(tok_b), _f32(pd_b)
    V = Tb.shape[-1]
    n = max(int(ell), 1)
    pt = np.zeros(n, dtype=np.float64)
    ratio = np.zeros(n, dtype=np.float64)
    us = np.zeros(n, dtype=np.float32)
    a = lib().orc_accept_scan(_ptr(Tb), _ptr(tb), _ptr(pb), int(ell), V, ctypes.c_uint64(seed), int(b), _ptr(pt),
                              _ptr(ratio), _ptr(us))
    if a < 0:
        raise RuntimeError(f"oracle accept_scan failed with code {a}")
    return a, pt[:ell], ratio[:ell], us[:ell]


def final_token(T_b, L_b, A, Bm, x0_b: int, tok_b, ell: int, a: int, seed: int, b: int, query: int = -1) -> dict:
    Tb, Lb, Aa, Bb, tb = _f32(T_b), _f32(L_b), _f32(A), _f32(Bm), _i32(tok_b)
    V = Tb.shape[-1]
    r = Aa.shape[1]
    o = RowOut()
    _check(lib().orc_final_token(_ptr(Tb), _ptr(Lb), _ptr(Aa), _ptr(Bb), int(x0_b), _ptr(tb), int(ell), int(a), V,
                                 r, ctypes.c_uint64(seed), int(b), int(query), ctypes.byref(o)), "final_token")
    return o.as_dict()


def verify(T, L, A, Bm, x0, tok, pd, ell, seed: int, threads: int = 1):
    """Full verification.  T [B][gamma+1][V], L [B][gamma][V].
    threads > 1 splits the requests over that many POSIX threads (same results)."""
    TT, Ll, Aa, Bb = _f32(T), _f32(L), _f32(A), _f32(Bm)
    xx, tt, pp, ll = _i32(x0), _i32(tok), _f32(pd), _i32(ell)
    B, gamma, V = Ll.shape
    r = Aa.shape[1]
    acc = np.zeros(B, dtype=np.int32)
    out = np.zeros((B, gamma + 1), dtype=np.int32)
    n_out = np.zeros(B, dtype=np.int32)
    tp = np.zeros((B, gamma), dtype=np.float32)
    args = (_ptr(TT), _ptr(Ll), _ptr(Aa), _ptr(Bb), _ptr(xx), _ptr(tt), _ptr(pp), _ptr(ll), B, gamma, V, r,
            ctypes.c_uint64(seed), _ptr(acc), _ptr(out), _ptr(n_out), _ptr(tp))
    if threads > 1:
        _check(lib().orc_verify_mt(*args, int(threads)), "verify_mt")
    else:
        _check(lib().orc_verify(*args), "verify")
    return acc, out, n_out, tp
