"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest
import torch

import draft_verify_sampling_prev_amd as dsp
from draft_verify_sampling_prev_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsp.library_path()):
        from draft_verify_sampling_prev_amd import build
        build.build()
    return dsp.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"dspark_markov_draft", "dspark_schedule", "dspark_verify", "dspark_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        getattr(lib, n)


def test_python_binding_has_the_same_names():
    for n in ("dspark_markov_draft", "dspark_markov_draft_conf", "dspark_markov_draft_noalloc",
              "dspark_markov_draft_sched", "dspark_rnn_draft",
              "dspark_rnn_verify",
              "dspark_schedule", "dspark_schedule_objective",
              "dspark_schedule_threshold",
              "dspark_verify", "dspark_workspace_size", "dspark_version"):
        assert callable(getattr(dsp, n))


def test_version(lib):
    assert "gfx950" in dsp.dspark_version()


def test_workspace_size_grows_with_shape(lib):
    a = dsp.dspark_workspace_size(4, 5, 1024, 16)
    b = dsp.dspark_workspace_size(256, 5, 129280, 256)
    assert 0 < a < b
    assert dsp.dspark_workspace_size(-1, 5, 1024, 16) == 0


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)


def _draft(lib, dtype=1, B=4, gamma=5, V=1024, r=16, L=FAKE, ws_bytes=1 << 30, ptr=FAKE):
    return lib.dspark_markov_draft(dtype, L, ptr, ptr, ptr, B, gamma, V, r, ctypes.c_uint64(1), None, ptr, ptr, ptr, ptr,
                                   ws_bytes, None)


def test_draft_argument_errors(lib):
    assert _draft(lib, dtype=7) == UNSUPPORTED
    assert _draft(lib, gamma=0) == UNSUPPORTED
    assert _draft(lib, gamma=17) == UNSUPPORTED
    assert _draft(lib, V=1001) == UNSUPPORTED
    assert _draft(lib, r=12) == UNSUPPORTED
    assert _draft(lib, r=264) == UNSUPPORTED
    assert _draft(lib, B=-1) == INVALID
    assert _draft(lib, B=5000, gamma=4) == UNSUPPORTED     # B*gamma > 16384
    assert _draft(lib, ptr=None) == INVALID
    assert _draft(lib, L=MISALIGNED) == INVALID
    assert _draft(lib, ws_bytes=16) == WORKSPACE
    assert b"workspace" in lib.dspark_last_error()
    # B == 0 is a no-op, even with null pointers
    assert _draft(lib, B=0, ptr=None, L=None) == OK


def test_draft_conf_argument_errors(lib):
    f = lib.dspark_markov_draft_conf

    def call(z0=FAKE, wc=FAKE, z=FAKE, B=4, dtype=1):
        return f(dtype, FAKE, FAKE, FAKE, FAKE, B, 5, 1024, 16, ctypes.c_uint64(1), None, z0, wc, FAKE, FAKE, FAKE, z, FAKE,
                 1 << 30, None)

    assert call(z0=None) == INVALID
    assert call(wc=None) == INVALID
    assert call(z=None) == INVALID
    assert call(dtype=5) == UNSUPPORTED
    assert call(B=0, z0=None, wc=None, z=None) == OK


def test_rnn_argument_errors(lib):
    fd = lib.dspark_rnn_draft

    def draft(Wt=FAKE, H=FAKE, B=4, dtype=1):
        return fd(dtype, FAKE, FAKE, FAKE, Wt, FAKE, B, 5, 1024, 16, ctypes.c_uint64(1), None, FAKE, FAKE, FAKE, H, FAKE,
                  1 << 30, None)

    assert draft(Wt=None) == INVALID
    assert draft(H=None) == INVALID
    assert draft(H=MISALIGNED) == INVALID
    assert draft(Wt=MISALIGNED) == INVALID
    assert draft(dtype=9) == UNSUPPORTED
    assert draft(B=0, Wt=None, H=None) == OK
    fv = lib.dspark_rnn_verify

    def verify(H=FAKE, B=4, ws_bytes=1 << 30):
        return fv(1, FAKE, FAKE, H, FAKE, FAKE, FAKE, FAKE, FAKE, B, 5, 1024, 16, ctypes.c_uint64(1), None, FAKE, FAKE, FAKE,
                  None, FAKE, ws_bytes, None)

    assert verify(H=None) == INVALID
    assert verify(H=MISALIGNED) == INVALID
    assert verify(ws_bytes=0) == WORKSPACE
    assert verify(B=0, H=None) == OK


def test_schedule_argument_errors(lib):
    f = lib.dspark_schedule
    assert f(FAKE, FAKE, 4, 5, ctypes.c_int64(-1), FAKE, FAKE, None) == INVALID
    assert f(FAKE, None, 4, 5, ctypes.c_int64(3), FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 4, 0, ctypes.c_int64(3), FAKE, FAKE, None) == UNSUPPORTED
    assert f(FAKE, FAKE, 4, 5, ctypes.c_int64(3), None, FAKE, None) == INVALID
    assert f(None, None, 0, 5, ctypes.c_int64(3), None, None, None) == OK


def test_schedule_objective_argument_errors(lib):
    f = lib.dspark_schedule_objective

    def call(z=FAKE, temps=FAKE, B=4, gamma=5, st=FAKE, n_time=64, cap=3, surv=FAKE, ln=FAKE):
        return f(z, temps, B, gamma, st, n_time, ctypes.c_int64(cap), surv, ln, None)

    assert call(cap=-1) == INVALID
    assert call(temps=None) == INVALID
    assert call(st=None) == INVALID
    assert call(surv=None) == INVALID
    assert call(gamma=0) == UNSUPPORTED
    assert call(B=5000, gamma=4) == UNSUPPORTED
    assert call(n_time=7) == INVALID            # needs B + min(cap, B*gamma) + 1 = 8 entries
    assert b"step_time" in lib.dspark_last_error()
    assert call(n_time=24, cap=1000) == INVALID  # cap clamps to 20: needs 25
    assert call(B=0, z=None, temps=None, st=None, surv=None, ln=None) == OK


def test_schedule_threshold_argument_errors(lib):
    f = lib.dspark_schedule_threshold
    assert f(FAKE, None, 4, 5, ctypes.c_float(0.5), FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 4, 17, ctypes.c_float(0.5), FAKE, FAKE, None) == UNSUPPORTED
    assert f(FAKE, FAKE, 4, 5, ctypes.c_float(0.5), FAKE, None, None) == INVALID
    assert f(None, None, 0, 5, ctypes.c_float(0.5), None, None, None) == OK


def test_verify_argument_errors(lib):
    f = lib.dspark_verify
    args = dict(dtype=1, Tgt=FAKE, B=4, gamma=5, V=1024, r=16, ws_bytes=1 << 30, acc=FAKE)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["dtype"], a["Tgt"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["B"], a["gamma"], a["V"],
                 a["r"], ctypes.c_uint64(1), None, a["acc"], FAKE, FAKE, None, FAKE, a["ws_bytes"], None)

    assert call(dtype=3) == UNSUPPORTED
    assert call(Tgt=None) == INVALID
    assert call(acc=None) == INVALID
    assert call(Tgt=MISALIGNED) == INVALID
    assert call(ws_bytes=0) == WORKSPACE
    assert call(V=12) == UNSUPPORTED
    assert call(B=0, Tgt=None) == OK


def test_binding_refuses_host_tensors(lib):
    L = torch.zeros((2, 3, 64), dtype=torch.bfloat16)
    A = torch.zeros((64, 8), dtype=torch.bfloat16)
    Bm = torch.zeros((8, 64), dtype=torch.bfloat16)
    x0 = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(binding.DsparkError):
        dsp.dspark_markov_draft(L, A, Bm, x0, 1)


def test_no_cpu_fallback_in_product_path():
    """The package never imports the oracle."""
    pkg = os.path.join(ROOT, "draft_verify_sampling_prev_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "dspark_oracle" not in text, fn


def test_noalloc_draft_argument_errors(lib):
    """The allocation-free draft validates everything, including the size of its static scratch (32 MiB),
    before touching the device."""
    f = lib.dspark_markov_draft_noalloc

    def call(B=4, gamma=5, V=1024, r=16, dtype=1, ptr=FAKE, L=FAKE):
        return f(dtype, L, ptr, ptr, ptr, B, gamma, V, r, ctypes.c_uint64(1), None, ptr, ptr, ptr, None)

    assert call(dtype=3) == UNSUPPORTED
    assert call(gamma=17) == UNSUPPORTED
    assert call(V=1001) == UNSUPPORTED
    assert call(B=-1) == INVALID
    # B * ceil(V/64) * 8 bytes of partials beyond 32 MiB: B = 1024 at V = 600000 needs ~73 MiB
    assert call(B=1024, gamma=8, V=600000, r=256) == WORKSPACE
    assert b"scratch" in lib.dspark_last_error()
    assert call(B=2048, gamma=8, V=129280, r=256) == WORKSPACE  # 2048 * 2020 * 8 bytes > 32 MiB
    assert call(ptr=None) == INVALID
    assert call(B=0, ptr=None, L=None) == OK
