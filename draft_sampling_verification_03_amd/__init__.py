"""DSpark per-round speculative-decoding hot path on AMD MI355X (gfx950).

Python binding of the C ABI in ``include/dspark.h`` (``libdspark.so``, built
in-tree by ``build.py``).  The functions ``dspark_*`` mirror the C entry points
one to one and only marshal arguments; every step of the path runs in the HIP
kernels.  Importing this package does not load the library; the first call
does, and raises if it is missing (there is no CPU fallback).
"""
from ._abi import (  # noqa: F401
    DSPARK_BF16, DSPARK_F32, DSPARK_SCHED_ASYNC_TOPK, DSPARK_SCHED_EARLY_STOP,
    DSPARK_SCHED_FULL_SEARCH, DSPARK_SCHED_OFF, DSPARK_SCHED_THRESHOLD, DSparkError, LIB_PATH, STATUS_NAMES,
    dspark_clear_device_error, dspark_device_error, dspark_draft, dspark_draft_workspace,
    dspark_draft_noalloc, dspark_draft_noalloc_scratch, NOALLOC_SCRATCH_BYTES,
    dspark_schedule, dspark_schedule_workspace, dspark_status_string, dspark_tv_overlap,
    dspark_tv_overlap_workspace, dspark_trace_collect, dspark_trace_enable, dspark_trace_entry,
    dspark_train_losses, dspark_train_losses_workspace, dspark_draft_rnn, dspark_verify_rnn,
    dspark_verify, dspark_verify_workspace, library, trace_summary)
from .api import (draft, draft_rnn, schedule, train_losses, tv_overlap, verify, verify_rnn,
                  Workspace)  # noqa: F401
