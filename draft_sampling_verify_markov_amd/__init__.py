"""DSpark draft -> schedule -> verify round on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libdspark.so`` (include/dspark.h).
It only marshals arguments: it checks dtypes, devices, shapes and contiguity
of torch tensors, passes raw device pointers and the current HIP stream, and
turns negative status codes into exceptions.  Every step of the round runs in
the HIP kernels of the library; there is no fallback path.
"""

from ._binding import (  # noqa: F401
    DSPARK_W_BF16,
    DSPARK_W_F32,
    DERR_BITS,
    DSparkError,
    DSparkDeviceError,
    lib_path,
    load_library,
    workspace_size,
    new_workspace,
    workspace_init,
    device_error,
    draft,
    draft_noalloc,
    schedule,
    schedule_async,
    schedule_threshold,
    accept_rates,
    verify,
    run_round,
    draft_rnn,
    verify_rnn,
    verify_stream,
    sts_workspace_size,
    new_sts_workspace,
    sts_fit,
    sts_apply,
)

__all__ = [
    "DSPARK_W_BF16", "DSPARK_W_F32", "DERR_BITS", "DSparkError", "DSparkDeviceError", "lib_path", "load_library",
    "workspace_size", "new_workspace", "workspace_init", "device_error", "draft", "draft_noalloc", "schedule", "schedule_async", "schedule_threshold", "accept_rates",
    "verify", "run_round", "draft_rnn", "verify_rnn", "verify_stream", "sts_workspace_size", "new_sts_workspace", "sts_fit", "sts_apply",
]
