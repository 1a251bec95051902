"""MI355X (gfx950) decode paged attention.

A C-ABI shared library (``libpa_decode.so``, declared in
``include/pa_decode.h``) with hand-written HIP kernels, and this thin ctypes
binding that passes torch tensors and the current HIP stream to it.
"""
from ._binding import (  # noqa: F401
    LIB_PATH, PA_DTYPE_BF16, PA_DTYPE_F16, PA_DTYPE_FP32, PA_DTYPE_INT32, PA_EALIGN, PA_EHIP, PA_EINVAL,
    PA_ENODEV, PA_ENOMEM, PA_ENOTSUP, PA_MERGE_AUTO, PA_MERGE_FUSED, PA_MERGE_KERNEL, PA_NOALLOC_SCRATCH_BYTES, PA_OK, PA_WORKSPACE_ZERO_BYTES, PA_SCALE_DEFAULT, PA_SCHEDULE_AUTO, PA_SCHEDULE_BALANCED,
    PA_SCHEDULE_PARTITIONS, PA_SCHEDULE_STAGED, PA_SCHEDULE_FITTED, PA_VARIANT_AUTO, PA_VARIANT_MFMA, PA_VARIANT_VALU,
    PaError, PaOpts, PaStats, PaTensor, cache_append, decode, last_error, make_opts, pa_cache_append,
    pa_check_args, pa_decode, pa_decode_noalloc, pa_prefill, release_workspaces, pa_prefill_workspace_bytes, prefill,
    pa_decode_ex, pa_decode_workspace_bytes, pa_get_stats, pa_release, pa_reset_stats, strerror,
    PA_TRACE_WORDS, pa_trace_clock_khz, pa_trace_set,
    tensor_desc, version,
)

__version__ = "0.1.0"
