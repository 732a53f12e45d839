"""ctypes binding of libdspark (C ABI declared in include/dspark.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs and the workspace are allocated with torch, and raw
device pointers plus torch's current HIP stream are passed to the library.
Every step of the path runs in the library's kernels; there is no CPU
fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

DSPARK_F32 = 0
DSPARK_BF16 = 1

_PKG = os.path.dirname(os.path.abspath(__file__))
# DSPARK_LIB may point at another build of the same library (for A/B timing).
_LIB_PATH = os.environ.get("DSPARK_LIB") or os.path.join(_PKG, "libdspark.so")

# Kernel ids for dspark_profile_query.
KERNELS = ("draft_tiles", "draft_locate", "schedule", "target_partials", "accept", "resid_tiles",
           "bonus_partials", "final")


class DsparkError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int


def load_library():
    """Load libdspark.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise DsparkError(f"{_LIB_PATH} is missing: build it with draft_verify_sampling_prev_amd.build.build() "
                          "(or __graft_entry__.build())")
    L = ctypes.CDLL(_LIB_PATH)
    L.dspark_version.restype = ctypes.c_char_p
    L.dspark_version.argtypes = []
    L.dspark_last_error.restype = ctypes.c_char_p
    L.dspark_last_error.argtypes = []
    L.dspark_workspace_size.restype = ctypes.c_size_t
    L.dspark_workspace_size.argtypes = [_I, _I, _I, _I]
    L.dspark_markov_draft.restype = _I
    L.dspark_markov_draft.argtypes = [_I, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_uint64, _P, _P, _P, _P, _P,
                                      ctypes.c_size_t, _P]
    L.dspark_markov_draft_noalloc.restype = _I
    L.dspark_markov_draft_noalloc.argtypes = [_I, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_uint64, _P, _P, _P, _P, _P]
    L.dspark_markov_draft_conf.restype = _I
    L.dspark_markov_draft_conf.argtypes = [_I, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_uint64, _P, _P, _P, _P, _P,
                                           _P, _P, _P, ctypes.c_size_t, _P]
    L.dspark_markov_draft_sched.restype = _I
    L.dspark_markov_draft_sched.argtypes = [_I, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_uint64, _P, _P, _P,
                                            ctypes.c_int64, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.dspark_rnn_draft.restype = _I
    L.dspark_rnn_draft.argtypes = [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_uint64, _P, _P, _P, _P, _P, _P,
                                   ctypes.c_size_t, _P]
    L.dspark_rnn_verify.restype = _I
    L.dspark_rnn_verify.argtypes = [_I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_uint64, _P, _P, _P,
                                    _P, _P, _P, ctypes.c_size_t, _P]
    L.dspark_schedule.restype = _I
    L.dspark_schedule.argtypes = [_P, _P, _I, _I, ctypes.c_int64, _P, _P, _P]
    L.dspark_schedule_objective.restype = _I
    L.dspark_schedule_objective.argtypes = [_P, _P, _I, _I, _P, _I, ctypes.c_int64, _P, _P, _P]
    L.dspark_schedule_threshold.restype = _I
    L.dspark_schedule_threshold.argtypes = [_P, _P, _I, _I, ctypes.c_float, _P, _P, _P]
    L.dspark_verify.restype = _I
    L.dspark_verify.argtypes = [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_uint64, _P, _P, _P,
                                _P, _P, _P, ctypes.c_size_t, _P]
    L.dspark_profile_start.restype = _I
    L.dspark_profile_start.argtypes = [_I, ctypes.c_uint]
    L.dspark_profile_stop.restype = _I
    L.dspark_profile_stop.argtypes = []
    L.dspark_profile_query.restype = _I
    L.dspark_profile_query.argtypes = [_I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
    _lib = L
    return L


def _check(rc: int, what: str):
    if rc != 0:
        msg = load_library().dspark_last_error().decode()
        raise DsparkError(f"{what} failed ({rc}): {msg}")


def dspark_version() -> str:
    return load_library().dspark_version().decode()


def dspark_workspace_size(B: int, gamma: int, V: int, r: int) -> int:
    return int(load_library().dspark_workspace_size(B, gamma, V, r))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSPARK_BF16
    if t.dtype == torch.float32:
        return DSPARK_F32
    raise DsparkError(f"unsupported logits dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str, device, dtype=None, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise DsparkError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise DsparkError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise DsparkError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise DsparkError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise DsparkError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise DsparkError(f"{name} must be contiguous")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _seed(seed, device):
    """(by-value seed, device seed pointer) for the C calls.  `seed` is an int (fixed when the call is
    enqueued) or a one-element int64 tensor on the call's device, whose bits the kernels read as the
    unsigned 64-bit seed when they run (so a captured graph draws new uniforms after the tensor changes)."""
    if isinstance(seed, torch.Tensor):
        _dev(seed, "seed", device, torch.int64, (1,))
        return ctypes.c_uint64(0), ctypes.c_void_p(seed.data_ptr())
    return ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), None


def workspace(B: int, gamma: int, V: int, r: int, device) -> torch.Tensor:
    n = dspark_workspace_size(B, gamma, V, r)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def dspark_markov_draft(L: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor, x0: torch.Tensor, seed,
                        ws: Optional[torch.Tensor] = None, out: Optional[Tuple] = None,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Draft gamma tokens per request.  seed: int, or a one-element int64 device tensor read when the kernels run.
    Returns (draft_tok int32 [B][g], draft_p f32 [B][g], draft_lse f64 [B][g])."""
    dev = L.device
    _dev(L, "L", None)
    B, gamma, V = L.shape
    r = A.shape[1]
    _dev(A, "A", dev, L.dtype, (V, r))
    _dev(Bm, "Bm", dev, L.dtype, (r, V))
    _dev(x0, "x0", dev, torch.int32, (B,))
    if out is None:
        tok = torch.empty((B, gamma), dtype=torch.int32, device=dev)
        p = torch.empty((B, gamma), dtype=torch.float32, device=dev)
        lse = torch.empty((B, gamma), dtype=torch.float64, device=dev)
    else:
        tok, p, lse = out
    if ws is None:
        ws = workspace(B, gamma, V, r, dev)
    rc = load_library().dspark_markov_draft(_dtype_code(L), _ptr(L), _ptr(A), _ptr(Bm), _ptr(x0), B, gamma, V, r,
                                            *_seed(seed, dev), _ptr(tok), _ptr(p),
                                            _ptr(lse), _ptr(ws), ws.numel(), _stream(dev, stream))
    _check(rc, "dspark_markov_draft")
    return tok, p, lse


def dspark_markov_draft_sched(L: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor, x0: torch.Tensor, seed,
                              z: torch.Tensor, temps: torch.Tensor, budget: int, ws: Optional[torch.Tensor] = None,
                              out: Optional[Tuple] = None, survival: Optional[torch.Tensor] = None,
                              out_len: Optional[torch.Tensor] = None, stream=None):
    """dspark_markov_draft then dspark_schedule(z, temps, budget) in one call (the schedule runs beside the last
    draft step where it can).  Returns (draft_tok, draft_p, draft_lse, survival f32 [B][g], verify_len int32 [B])."""
    dev = L.device
    _dev(L, "L", None)
    B, gamma, V = L.shape
    r = A.shape[1]
    _dev(A, "A", dev, L.dtype, (V, r))
    _dev(Bm, "Bm", dev, L.dtype, (r, V))
    _dev(x0, "x0", dev, torch.int32, (B,))
    _dev(z, "z", dev, torch.float32, (B, gamma))
    _dev(temps, "temps", dev, torch.float32, (gamma,))
    if out is None:
        tok = torch.empty((B, gamma), dtype=torch.int32, device=dev)
        p = torch.empty((B, gamma), dtype=torch.float32, device=dev)
        lse = torch.empty((B, gamma), dtype=torch.float64, device=dev)
    else:
        tok, p, lse = out
    if survival is None:
        survival = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    _dev(survival, "survival", dev, torch.float32, (B, gamma))
    if out_len is None:
        out_len = torch.empty((B,), dtype=torch.int32, device=dev)
    _dev(out_len, "verify_len", dev, torch.int32, (B,))
    if ws is None:
        ws = workspace(B, gamma, V, r, dev)
    rc = load_library().dspark_markov_draft_sched(_dtype_code(L), _ptr(L), _ptr(A), _ptr(Bm), _ptr(x0), B, gamma, V,
                                                  r, *_seed(seed, dev), _ptr(z), _ptr(temps),
                                                  ctypes.c_int64(int(budget)), _ptr(tok), _ptr(p), _ptr(lse),
                                                  _ptr(survival), _ptr(out_len), _ptr(ws), ws.numel(),
                                                  _stream(dev, stream))
    _check(rc, "dspark_markov_draft_sched")
    return tok, p, lse, survival, out_len


def dspark_markov_draft_noalloc(L: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor, x0: torch.Tensor, seed,
                                out: Optional[Tuple] = None, stream=None):
    """dspark_markov_draft without a workspace (the library's static device scratch); allocates nothing when
    `out` is given.  Returns (draft_tok int32 [B][g], draft_p f32 [B][g], draft_lse f64 [B][g])."""
    dev = L.device
    _dev(L, "L", None)
    B, gamma, V = L.shape
    r = A.shape[1]
    _dev(A, "A", dev, L.dtype, (V, r))
    _dev(Bm, "Bm", dev, L.dtype, (r, V))
    _dev(x0, "x0", dev, torch.int32, (B,))
    if out is None:
        tok = torch.empty((B, gamma), dtype=torch.int32, device=dev)
        p = torch.empty((B, gamma), dtype=torch.float32, device=dev)
        lse = torch.empty((B, gamma), dtype=torch.float64, device=dev)
    else:
        tok, p, lse = out
        _dev(tok, "draft_tok", dev, torch.int32, (B, gamma))
        _dev(p, "draft_p", dev, torch.float32, (B, gamma))
        _dev(lse, "draft_lse", dev, torch.float64, (B, gamma))
    rc = load_library().dspark_markov_draft_noalloc(_dtype_code(L), _ptr(L), _ptr(A), _ptr(Bm), _ptr(x0), B, gamma, V,
                                                    r, *_seed(seed, dev), _ptr(tok), _ptr(p), _ptr(lse),
                                                    _stream(dev, stream))
    _check(rc, "dspark_markov_draft_noalloc")
    return tok, p, lse


def dspark_markov_draft_conf(L: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor, x0: torch.Tensor, seed,
                             z0: torch.Tensor, wc: torch.Tensor, ws: Optional[torch.Tensor] = None,
                             out: Optional[Tuple] = None, stream=None):
    """Draft gamma tokens per request and the Markov-conditioned confidence
    logits z[b][k-1] = z0[b][k-1] + <A[x_{k-1}], wc>.  Returns (draft_tok int32,
    draft_p f32, draft_lse f64, z f32), each [B][g]."""
    dev = L.device
    _dev(L, "L", None)
    B, gamma, V = L.shape
    r = A.shape[1]
    _dev(A, "A", dev, L.dtype, (V, r))
    _dev(Bm, "Bm", dev, L.dtype, (r, V))
    _dev(x0, "x0", dev, torch.int32, (B,))
    _dev(z0, "z0", dev, torch.float32, (B, gamma))
    _dev(wc, "wc", dev, L.dtype, (r,))
    if out is None:
        tok = torch.empty((B, gamma), dtype=torch.int32, device=dev)
        p = torch.empty((B, gamma), dtype=torch.float32, device=dev)
        lse = torch.empty((B, gamma), dtype=torch.float64, device=dev)
        z = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    else:
        tok, p, lse, z = out
    if ws is None:
        ws = workspace(B, gamma, V, r, dev)
    rc = load_library().dspark_markov_draft_conf(_dtype_code(L), _ptr(L), _ptr(A), _ptr(Bm), _ptr(x0), B, gamma, V,
                                                 r, *_seed(seed, dev), _ptr(z0), _ptr(wc),
                                                 _ptr(tok), _ptr(p), _ptr(lse), _ptr(z), _ptr(ws), ws.numel(),
                                                 _stream(dev, stream))
    _check(rc, "dspark_markov_draft_conf")
    return tok, p, lse, z


def dspark_rnn_draft(L: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor, Wt: torch.Tensor, x0: torch.Tensor, seed,
                     ws: Optional[torch.Tensor] = None, out: Optional[Tuple] = None, stream=None):
    """Draft gamma tokens per request with the RNN head.  Returns (draft_tok int32 [B][g], draft_p f32,
    draft_lse f64, H [B][g][r] in the logits' dtype)."""
    dev = L.device
    _dev(L, "L", None)
    B, gamma, V = L.shape
    r = A.shape[1]
    _dev(A, "A", dev, L.dtype, (V, r))
    _dev(Bm, "Bm", dev, L.dtype, (r, V))
    _dev(Wt, "Wt", dev, L.dtype, (r, r))
    _dev(x0, "x0", dev, torch.int32, (B,))
    if out is None:
        tok = torch.empty((B, gamma), dtype=torch.int32, device=dev)
        p = torch.empty((B, gamma), dtype=torch.float32, device=dev)
        lse = torch.empty((B, gamma), dtype=torch.float64, device=dev)
        H = torch.empty((B, gamma, r), dtype=L.dtype, device=dev)
    else:
        tok, p, lse, H = out
    _dev(H, "H", dev, L.dtype, (B, gamma, r))
    if ws is None:
        ws = workspace(B, gamma, V, r, dev)
    rc = load_library().dspark_rnn_draft(_dtype_code(L), _ptr(L), _ptr(A), _ptr(Bm), _ptr(Wt), _ptr(x0), B, gamma, V,
                                         r, *_seed(seed, dev), _ptr(tok), _ptr(p), _ptr(lse),
                                         _ptr(H), _ptr(ws), ws.numel(), _stream(dev, stream))
    _check(rc, "dspark_rnn_draft")
    return tok, p, lse, H


def dspark_schedule(z: Optional[torch.Tensor], temps: Optional[torch.Tensor], budget: int,
                    survival: Optional[torch.Tensor] = None, out_len: Optional[torch.Tensor] = None,
                    B: Optional[int] = None, gamma: Optional[int] = None,
                    stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Survival product and budget selection.  With z=None, `survival` is the input Theta.
    Returns (survival f32 [B][g], verify_len int32 [B])."""
    ref = z if z is not None else survival
    if ref is None:
        raise DsparkError("either z or survival must be given")
    dev = ref.device
    if B is None or gamma is None:
        B, gamma = ref.shape
    if z is not None:
        _dev(z, "z", dev, torch.float32, (B, gamma))
        _dev(temps, "temps", dev, torch.float32, (gamma,))
        if survival is None:
            survival = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    _dev(survival, "survival", dev, torch.float32, (B, gamma))
    if out_len is None:
        out_len = torch.empty((B,), dtype=torch.int32, device=dev)
    rc = load_library().dspark_schedule(_ptr(z), _ptr(temps), B, gamma, ctypes.c_int64(int(budget)), _ptr(survival),
                                        _ptr(out_len), _stream(dev, stream))
    _check(rc, "dspark_schedule")
    return survival, out_len


def _schedule_args(z, temps, survival, out_len, B, gamma):
    ref = z if z is not None else survival
    if ref is None:
        raise DsparkError("either z or survival must be given")
    dev = ref.device
    if B is None or gamma is None:
        B, gamma = ref.shape
    if z is not None:
        _dev(z, "z", dev, torch.float32, (B, gamma))
        _dev(temps, "temps", dev, torch.float32, (gamma,))
        if survival is None:
            survival = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    _dev(survival, "survival", dev, torch.float32, (B, gamma))
    if out_len is None:
        out_len = torch.empty((B,), dtype=torch.int32, device=dev)
    return dev, B, gamma, survival, out_len


def dspark_schedule_objective(z: Optional[torch.Tensor], temps: Optional[torch.Tensor], step_time: torch.Tensor,
                              max_admit: int, survival: Optional[torch.Tensor] = None,
                              out_len: Optional[torch.Tensor] = None, B: Optional[int] = None,
                              gamma: Optional[int] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Survival product and objective-based admission against the engine
    profile `step_time` (f32 [n_time], time of a batch of n tokens).
    Returns (survival f32 [B][g], verify_len int32 [B])."""
    dev, B, gamma, survival, out_len = _schedule_args(z, temps, survival, out_len, B, gamma)
    if step_time.dim() != 1:
        raise DsparkError("step_time must be one-dimensional")
    _dev(step_time, "step_time", dev, torch.float32, (step_time.shape[0],))
    rc = load_library().dspark_schedule_objective(_ptr(z), _ptr(temps), B, gamma, _ptr(step_time),
                                                  int(step_time.shape[0]), ctypes.c_int64(int(max_admit)),
                                                  _ptr(survival), _ptr(out_len), _stream(dev, stream))
    _check(rc, "dspark_schedule_objective")
    return survival, out_len


def dspark_schedule_threshold(z: Optional[torch.Tensor], temps: Optional[torch.Tensor], tau: float,
                              survival: Optional[torch.Tensor] = None, out_len: Optional[torch.Tensor] = None,
                              B: Optional[int] = None, gamma: Optional[int] = None,
                              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Survival product and static-threshold admission (leading run of Theta >= tau).
    Returns (survival f32 [B][g], verify_len int32 [B])."""
    dev, B, gamma, survival, out_len = _schedule_args(z, temps, survival, out_len, B, gamma)
    rc = load_library().dspark_schedule_threshold(_ptr(z), _ptr(temps), B, gamma, ctypes.c_float(float(tau)),
                                                  _ptr(survival), _ptr(out_len), _stream(dev, stream))
    _check(rc, "dspark_schedule_threshold")
    return survival, out_len


def dspark_verify(Tgt: torch.Tensor, L: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor, x0: torch.Tensor,
                  draft_tok: torch.Tensor, draft_p: torch.Tensor, draft_lse: torch.Tensor, verify_len: torch.Tensor,
                  seed, ws: Optional[torch.Tensor] = None, out: Optional[Tuple] = None, want_target_p: bool = True,
                  stream=None):
    """Rejection-sampling verification.
    Returns (accepted int32 [B], out_tok int32 [B][g+1], n_out int32 [B], target_p f32 [B][g] or None)."""
    dev = L.device
    _dev(L, "L", None)
    B, gamma, V = L.shape
    r = A.shape[1]
    _dev(Tgt, "Tgt", dev, L.dtype, (B, gamma + 1, V))
    _dev(A, "A", dev, L.dtype, (V, r))
    _dev(Bm, "Bm", dev, L.dtype, (r, V))
    _dev(x0, "x0", dev, torch.int32, (B,))
    _dev(draft_tok, "draft_tok", dev, torch.int32, (B, gamma))
    _dev(draft_p, "draft_p", dev, torch.float32, (B, gamma))
    _dev(draft_lse, "draft_lse", dev, torch.float64, (B, gamma))
    _dev(verify_len, "verify_len", dev, torch.int32, (B,))
    if out is None:
        acc = torch.empty((B,), dtype=torch.int32, device=dev)
        out_tok = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
        n_out = torch.empty((B,), dtype=torch.int32, device=dev)
        tp = torch.empty((B, gamma), dtype=torch.float32, device=dev) if want_target_p else None
    else:
        acc, out_tok, n_out, tp = out
    if ws is None:
        ws = workspace(B, gamma, V, r, dev)
    rc = load_library().dspark_verify(_dtype_code(L), _ptr(Tgt), _ptr(L), _ptr(A), _ptr(Bm), _ptr(x0), _ptr(draft_tok),
                                      _ptr(draft_p), _ptr(draft_lse), _ptr(verify_len), B, gamma, V, r,
                                      *_seed(seed, dev), _ptr(acc), _ptr(out_tok),
                                      _ptr(n_out), _ptr(tp), _ptr(ws), ws.numel(), _stream(dev, stream))
    _check(rc, "dspark_verify")
    return acc, out_tok, n_out, tp


def dspark_rnn_verify(Tgt: torch.Tensor, L: torch.Tensor, H: torch.Tensor, Bm: torch.Tensor, draft_tok: torch.Tensor,
                      draft_p: torch.Tensor, draft_lse: torch.Tensor, verify_len: torch.Tensor, seed,
                      ws: Optional[torch.Tensor] = None, out: Optional[Tuple] = None, want_target_p: bool = True,
                      stream=None):
    """Verification of an RNN-head draft (the residual rebuilds draft rows from the states H [B][g][r]).
    Returns (accepted int32 [B], out_tok int32 [B][g+1], n_out int32 [B], target_p f32 [B][g] or None)."""
    dev = L.device
    _dev(L, "L", None)
    B, gamma, V = L.shape
    r = H.shape[2]
    _dev(Tgt, "Tgt", dev, L.dtype, (B, gamma + 1, V))
    _dev(H, "H", dev, L.dtype, (B, gamma, r))
    _dev(Bm, "Bm", dev, L.dtype, (r, V))
    _dev(draft_tok, "draft_tok", dev, torch.int32, (B, gamma))
    _dev(draft_p, "draft_p", dev, torch.float32, (B, gamma))
    _dev(draft_lse, "draft_lse", dev, torch.float64, (B, gamma))
    _dev(verify_len, "verify_len", dev, torch.int32, (B,))
    if out is None:
        acc = torch.empty((B,), dtype=torch.int32, device=dev)
        out_tok = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
        n_out = torch.empty((B,), dtype=torch.int32, device=dev)
        tp = torch.empty((B, gamma), dtype=torch.float32, device=dev) if want_target_p else None
    else:
        acc, out_tok, n_out, tp = out
    if ws is None:
        ws = workspace(B, gamma, V, r, dev)
    rc = load_library().dspark_rnn_verify(_dtype_code(L), _ptr(Tgt), _ptr(L), _ptr(H), _ptr(Bm), _ptr(draft_tok),
                                          _ptr(draft_p), _ptr(draft_lse), _ptr(verify_len), B, gamma, V, r,
                                          *_seed(seed, dev), _ptr(acc), _ptr(out_tok),
                                          _ptr(n_out), _ptr(tp), _ptr(ws), ws.numel(), _stream(dev, stream))
    _check(rc, "dspark_rnn_verify")
    return acc, out_tok, n_out, tp


# ----------------------------------------------------------------------------- timing (measurement tools)
def profile_start(max_launches: int = 100000, kernels=KERNELS):
    """Start timing the named kernels (default: all)."""
    mask = 0
    for k in kernels:
        mask |= 1 << KERNELS.index(k)
    _check(load_library().dspark_profile_start(max_launches, mask), "dspark_profile_start")


def profile_stop():
    _check(load_library().dspark_profile_stop(), "dspark_profile_stop")


def profile_query(kernel: str):
    """Returns (total_ms, launches) of one kernel since profile_start."""
    kid = KERNELS.index(kernel)
    ms = ctypes.c_double()
    n = ctypes.c_int()
    _check(load_library().dspark_profile_query(kid, ctypes.byref(ms), ctypes.byref(n)), "dspark_profile_query")
    return ms.value, n.value
