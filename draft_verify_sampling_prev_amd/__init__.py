"""MI355X-native DSpark per-step draft -> schedule -> verify token path.

The compute path is the HIP library ``libdspark.so`` (hand-written gfx950
kernels behind a C ABI, declared in ``include/dspark.h``).  This package holds
the thin ctypes binding with the same entry-point names, the build step, and
the seeded synthetic-input generator.  Importing it does not load the
library; the first call does, and raises if the library is missing.
"""
from .binding import (  # noqa: F401
    DsparkError,
    dspark_markov_draft,
    dspark_markov_draft_conf,
    dspark_markov_draft_noalloc,
    dspark_markov_draft_sched,
    dspark_rnn_draft,
    dspark_rnn_verify,
    dspark_schedule,
    dspark_schedule_objective,
    dspark_schedule_threshold,
    dspark_verify,
    dspark_workspace_size,
    dspark_version,
    library_path,
    load_library,
)

__all__ = [
    "DsparkError",
    "dspark_markov_draft",
    "dspark_markov_draft_conf",
    "dspark_markov_draft_noalloc",
    "dspark_markov_draft_sched",
    "dspark_rnn_draft",
    "dspark_rnn_verify",
    "dspark_schedule",
    "dspark_schedule_objective",
    "dspark_schedule_threshold",
    "dspark_verify",
    "dspark_workspace_size",
    "dspark_version",
    "library_path",
    "load_library",
]
