"""ctypes binding of ``libpa_decode.so`` (the C ABI in ``include/pa_decode.h``).

Argument marshalling only: torch tensors become ``pa_tensor`` descriptors
(data pointer, dtype, shape, strides) and the current HIP stream is passed
through.  Every step of the computation runs in the library's gfx950 kernels;
there is no fallback of any kind.  If the library is missing, importing the
package raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa_decode.so")

PA_OK, PA_EINVAL, PA_ENOTSUP, PA_EALIGN, PA_ENODEV, PA_ENOMEM, PA_EHIP = range(7)
# scale argument asking the library for 1/sqrt(head_dim)
PA_SCALE_DEFAULT = float("nan")
# static split-KV scratch of pa_decode_noalloc, per device
PA_NOALLOC_SCRATCH_BYTES = 32 << 20
PA_DTYPE_BF16, PA_DTYPE_INT32, PA_DTYPE_FP32, PA_DTYPE_F16 = 1, 2, 3, 4
PA_VARIANT_AUTO, PA_VARIANT_VALU, PA_VARIANT_MFMA = 0, 1, 2
VARIANTS = {"auto": PA_VARIANT_AUTO, "valu": PA_VARIANT_VALU, "mfma": PA_VARIANT_MFMA}
PA_SCHEDULE_AUTO, PA_SCHEDULE_PARTITIONS, PA_SCHEDULE_BALANCED, PA_SCHEDULE_STAGED, PA_SCHEDULE_FITTED = \
    0, 1, 2, 3, 4
SCHEDULES = {"auto": PA_SCHEDULE_AUTO, "partitions": PA_SCHEDULE_PARTITIONS,
             "balanced": PA_SCHEDULE_BALANCED, "staged": PA_SCHEDULE_STAGED, "fitted": PA_SCHEDULE_FITTED}
PA_MERGE_AUTO, PA_MERGE_KERNEL, PA_MERGE_FUSED = 0, 1, 2
MERGES = {"auto": PA_MERGE_AUTO, "kernel": PA_MERGE_KERNEL, "fused": PA_MERGE_FUSED}
PA_WORKSPACE_ZERO_BYTES = 65536


class PaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class PaOpts(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("partition_tokens", ctypes.c_int32),
                ("schedule", ctypes.c_int32), ("shares", ctypes.c_int32),
                ("window", ctypes.c_int32), ("merge", ctypes.c_int32), ("reserved", ctypes.c_int32 * 2)]


class PaStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "calls", "valu_launches", "mfma_launches", "split_calls", "merge_launches",
        "last_partition_tokens", "last_num_partitions", "last_variant", "balanced_calls",
        "last_schedule", "append_launches", "prefill_launches", "fused_calls")]


class PaError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code}): {detail}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m paged_attention_decode_04_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    T = ctypes.POINTER(PaTensor)
    args12 = [T, T, T, T, T, ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
              ctypes.c_int, T]
    lib.pa_decode.argtypes = args12 + [ctypes.c_void_p]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_ex.argtypes = args12 + [ctypes.c_void_p, ctypes.POINTER(PaOpts),
                                          ctypes.c_void_p, ctypes.c_size_t]
    lib.pa_decode_ex.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = args12 + [ctypes.c_void_p, ctypes.POINTER(PaOpts)]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_check_args.argtypes = args12 + [ctypes.POINTER(PaOpts)]
    lib.pa_check_args.restype = ctypes.c_int
    lib.pa_decode_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                              ctypes.POINTER(PaOpts)]
    lib.pa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_get_stats.argtypes = [ctypes.POINTER(PaStats)]
    lib.pa_get_stats.restype = ctypes.c_int
    lib.pa_reset_stats.argtypes = []
    lib.pa_reset_stats.restype = None
    lib.pa_trace_set.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.pa_trace_set.restype = ctypes.c_int
    lib.pa_trace_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int)]
    lib.pa_trace_clock_khz.restype = ctypes.c_int
    lib.pa_strerror.argtypes = [ctypes.c_int]
    lib.pa_strerror.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_release.argtypes = []
    lib.pa_release.restype = ctypes.c_int
    lib.pa_version.argtypes = []
    lib.pa_version.restype = ctypes.c_char_p
    T = ctypes.POINTER(PaTensor)
    lib.pa_cache_append.argtypes = [T, T, T, T, T, T, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    lib.pa_cache_append.restype = ctypes.c_int
    lib.pa_prefill.argtypes = [T, T, T, T, T, T, ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, T, ctypes.c_void_p, ctypes.POINTER(PaOpts), ctypes.c_void_p,
                               ctypes.c_size_t]
    lib.pa_prefill.restype = ctypes.c_int
    lib.pa_prefill_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                               ctypes.POINTER(PaOpts)]
    lib.pa_prefill_workspace_bytes.restype = ctypes.c_size_t
    return lib


class _Library:
    """The shared library, loaded on first use: importing the package (for
    instance to build the library) does not need it, and every call through
    the binding fails loudly with ImportError if it is missing or stale."""
    _lib = None

    def __getattr__(self, name):
        if _Library._lib is None:
            _Library._lib = _load()
        return getattr(_Library._lib, name)


LIB = _Library()


def strerror(code: int) -> str:
    return LIB.pa_strerror(code).decode()


def last_error() -> str:
    return LIB.pa_last_error().decode()


def version() -> str:
    return LIB.pa_version().decode()


def _check(rc: int, where: str):
    if rc != PA_OK:
        raise PaError(rc, where, last_error())


# ------------------------------------------------------------------ marshalling
def _dtype_code(t) -> int:
    import torch
    return {torch.bfloat16: PA_DTYPE_BF16, torch.int32: PA_DTYPE_INT32,
            torch.float32: PA_DTYPE_FP32, torch.float16: PA_DTYPE_F16}.get(t.dtype, 0)


def tensor_desc(t) -> PaTensor:
    """pa_tensor describing a torch tensor (no copy; shape/strides in elements)."""
    d = PaTensor()
    d.data = t.data_ptr()
    d.dtype = _dtype_code(t)
    d.ndim = t.dim()
    for i, (n, s) in enumerate(zip(t.shape, t.stride())):
        if i < 4:
            d.shape[i] = n
            d.stride[i] = s
    return d


def _require_device(*ts):
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all tensors must live on the same GPU device")


def make_opts(variant="auto", partition_tokens: int = 0, schedule="auto", shares: int = 0,
              window: int = 0, merge="auto") -> PaOpts:
    o = PaOpts()
    o.shares = int(shares)
    o.window = int(window)
    o.merge = MERGES[merge] if isinstance(merge, str) else int(merge)
    o.variant = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    o.partition_tokens = int(partition_tokens)
    o.schedule = SCHEDULES[schedule] if isinstance(schedule, str) else int(schedule)
    return o


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _torch_stream(stream, device):
    """The torch stream the call's work goes to (a torch.cuda.Stream, or a
    raw hipStream_t handle wrapped as an external stream)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


# Workspaces of the convenience calls, one per (device, stream): zeroed once
# when made (every call leaves the balanced schedule's counters zero, and the
# rest is written before it is read), grown when a call needs more.  Calls on
# one stream are ordered, so sharing a workspace there is safe; calls on
# different streams get different workspaces.
_WORKSPACES = {}


def _workspace(nbytes, device, tstream):
    """A 256-byte-aligned uint8 device buffer of at least nbytes for work on
    tstream, allocated (and zero-filled) on that stream so the caching
    allocator orders its reuse after that stream's work."""
    import torch
    capturing = torch.cuda.is_current_stream_capturing()
    key = (device.index, tstream.cuda_stream)
    have = None if capturing else _WORKSPACES.get(key)
    if have is not None and have.numel() >= nbytes:
        return have
    with torch.cuda.stream(tstream):
        raw = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    ws = raw[off:off + nbytes]
    if not capturing:
        _WORKSPACES[key] = ws
    return ws


def release_workspaces() -> None:
    """Drop the convenience calls' cached workspaces (the caching allocator
    reuses their memory after the work queued on their streams)."""
    _WORKSPACES.clear()


# ------------------------------------------------------------------ C-ABI mirror
def pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale, num_q_heads,
              num_kv_heads, head_dim, page_size, out, stream=None):
    """Same arguments as the C function; tensors are torch tensors on one GPU.
    Uses the library's own split-KV workspace."""
    import torch
    _require_device(q, k_cache, v_cache, block_tables, context_lens, out)
    with torch.cuda.device(q.device):
        rc = LIB.pa_decode(tensor_desc(q), tensor_desc(k_cache), tensor_desc(v_cache),
                           tensor_desc(block_tables), tensor_desc(context_lens), float(scale),
                           num_q_heads, num_kv_heads, head_dim, page_size, tensor_desc(out),
                           _stream_handle(stream, q.device))
    _check(rc, "pa_decode")
    return out


def pa_cache_append(k_new, v_new, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
                    head_dim, page_size, stream=None):
    """C ``pa_cache_append``: write each sequence's newest token (position
    context_lens[b] - 1) into its page slot of the K and V pools."""
    import torch
    _require_device(k_new, v_new, k_cache, v_cache, block_tables, context_lens)
    with torch.cuda.device(k_new.device):
        rc = LIB.pa_cache_append(tensor_desc(k_new), tensor_desc(v_new), tensor_desc(k_cache),
                                 tensor_desc(v_cache), tensor_desc(block_tables),
                                 tensor_desc(context_lens), num_kv_heads, head_dim, page_size,
                                 _stream_handle(stream, k_new.device))
    _check(rc, "pa_cache_append")


def cache_append(k_new, v_new, k_cache, v_cache, block_tables, context_lens, stream=None):
    """KV-cache append on torch tensors; sizes come from the shapes."""
    NP, P, Hkv, D = k_cache.shape
    pa_cache_append(k_new, v_new, k_cache, v_cache, block_tables, context_lens, Hkv, D, P, stream)


def pa_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, num_q_heads,
               num_kv_heads, head_dim, page_size, out, stream=None, opts: PaOpts | None = None,
               workspace=None):
    """C ``pa_prefill``; ``workspace`` is a torch uint8 tensor or None."""
    import torch
    _require_device(q, k_cache, v_cache, block_tables, context_lens, query_start, out)
    with torch.cuda.device(q.device):
        rc = LIB.pa_prefill(tensor_desc(q), tensor_desc(k_cache), tensor_desc(v_cache),
                            tensor_desc(block_tables), tensor_desc(context_lens),
                            tensor_desc(query_start), float(scale), num_q_heads, num_kv_heads,
                            head_dim, page_size, tensor_desc(out), _stream_handle(stream, q.device),
                            ctypes.byref(opts) if opts else None,
                            workspace.data_ptr() if workspace is not None else None,
                            workspace.numel() if workspace is not None else 0)
    _check(rc, "pa_prefill")
    return out


def pa_prefill_workspace_bytes(num_rows, num_seqs, num_q_heads, num_kv_heads, head_dim,
                               max_blocks_per_seq, page_size, opts: PaOpts | None = None) -> int:
    return int(LIB.pa_prefill_workspace_bytes(num_rows, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              max_blocks_per_seq, page_size,
                                              ctypes.byref(opts) if opts else None))


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale=None, out=None, *,
            window: int = 0, partition_tokens: int = 0, schedule="auto", workspace=None, stream=None,
            out_dtype=None):
    """Several queries per sequence on torch tensors: q [R, Hq, D] holds
    sequence b's queries at rows [query_start[b], query_start[b+1]) (its last
    tokens, attending causally).  schedule: "auto", "partitions" or "staged".
    Returns out [R, Hq, D]."""
    import torch
    R, Hq, D = q.shape
    NP, P, Hkv, _ = k_cache.shape
    if scale is None:
        scale = PA_SCALE_DEFAULT
    ts = _torch_stream(stream, q.device)
    if out is None:
        with torch.cuda.stream(ts):
            out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    opts = make_opts("auto", partition_tokens, schedule, 0, window)
    if workspace is None:
        n = pa_prefill_workspace_bytes(R, block_tables.shape[0], Hq, Hkv, D, block_tables.shape[1], P, opts)
        if n:
            workspace = _workspace(n, q.device, ts)
    return pa_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, Hq, Hkv, D, P,
                      out, stream, opts, workspace)


def pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                              max_blocks_per_seq, page_size, opts: PaOpts | None = None) -> int:
    return int(LIB.pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             max_blocks_per_seq, page_size,
                                             ctypes.byref(opts) if opts else None))


def pa_decode_ex(q, k_cache, v_cache, block_tables, context_lens, scale, num_q_heads,
                 num_kv_heads, head_dim, page_size, out, stream=None, opts: PaOpts | None = None,
                 workspace=None):
    """C ``pa_decode_ex``; ``workspace`` is a torch uint8 tensor or None."""
    import torch
    _require_device(q, k_cache, v_cache, block_tables, context_lens, out,
                    *([workspace] if workspace is not None else []))
    ws_ptr = ctypes.c_void_p(workspace.data_ptr() if workspace is not None else None)
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(q.device):
        rc = LIB.pa_decode_ex(tensor_desc(q), tensor_desc(k_cache), tensor_desc(v_cache),
                              tensor_desc(block_tables), tensor_desc(context_lens), float(scale),
                              num_q_heads, num_kv_heads, head_dim, page_size, tensor_desc(out),
                              _stream_handle(stream, q.device),
                              ctypes.byref(opts) if opts else None, ws_ptr, ws_len)
    _check(rc, "pa_decode_ex")
    return out


def pa_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, num_q_heads,
                      num_kv_heads, head_dim, page_size, out, stream=None, opts: PaOpts | None = None):
    """C ``pa_decode_noalloc``: the split-KV partials go to the library's
    static per-device scratch; nothing is allocated."""
    import torch
    _require_device(q, k_cache, v_cache, block_tables, context_lens, out)
    with torch.cuda.device(q.device):
        rc = LIB.pa_decode_noalloc(tensor_desc(q), tensor_desc(k_cache), tensor_desc(v_cache),
                                   tensor_desc(block_tables), tensor_desc(context_lens), float(scale),
                                   num_q_heads, num_kv_heads, head_dim, page_size, tensor_desc(out),
                                   _stream_handle(stream, q.device), ctypes.byref(opts) if opts else None)
    _check(rc, "pa_decode_noalloc")
    return out


def pa_check_args(q, k_cache, v_cache, block_tables, context_lens, scale, num_q_heads,
                  num_kv_heads, head_dim, page_size, out, opts: PaOpts | None = None) -> int:
    """Host-side validation only (no HIP call); returns the error code."""
    return LIB.pa_check_args(tensor_desc(q), tensor_desc(k_cache), tensor_desc(v_cache),
                             tensor_desc(block_tables), tensor_desc(context_lens), float(scale),
                             num_q_heads, num_kv_heads, head_dim, page_size, tensor_desc(out),
                             ctypes.byref(opts) if opts else None)


def pa_get_stats() -> dict:
    s = PaStats()
    _check(LIB.pa_get_stats(ctypes.byref(s)), "pa_get_stats")
    return {name: int(getattr(s, name)) for name, _ in PaStats._fields_}


def pa_reset_stats() -> None:
    LIB.pa_reset_stats()


PA_TRACE_WORDS = 8


def pa_trace_set(buf) -> None:
    """Per-workgroup timeline records of the partitioned MFMA decode into the
    contiguous device tensor ``buf`` (PA_TRACE_WORDS uint64 per workgroup),
    or stop with ``None``.  A measurement aid; see ``pa_trace_set`` in the
    header for the record layout."""
    if buf is None:
        _check(LIB.pa_trace_set(None, 0), "pa_trace_set")
    else:
        _check(LIB.pa_trace_set(buf.data_ptr(), buf.numel() * buf.element_size()), "pa_trace_set")


def pa_trace_clock_khz() -> int:
    """Frequency of the timeline records' clock on the current device (kHz)."""
    v = ctypes.c_int(0)
    _check(LIB.pa_trace_clock_khz(ctypes.byref(v)), "pa_trace_clock_khz")
    return int(v.value)


def pa_release() -> None:
    _check(LIB.pa_release(), "pa_release")


# ------------------------------------------------------------------ convenience
def decode(q, k_cache, v_cache, block_tables, context_lens, scale=None, out=None, *,
           variant="auto", partition_tokens: int = 0, schedule="auto", shares: int = 0,
           window: int = 0, merge="auto", workspace=None, stream=None, out_dtype=None):
    """Decode paged attention on torch tensors.

    q [B, Hq, D]; k_cache/v_cache [NP, P, Hkv, D] (NHD pool) -- each bf16, fp16
    or fp32 (K and V alike); out defaults to q's type (``out_dtype`` overrides);
    block_tables [B, MaxBlk] int32; context_lens [B] int32; scale defaults to
    1/sqrt(D) (chosen by the library); ``window`` > 0 attends to each
    sequence's last ``window`` tokens only.  Returns out [B, Hq, D].  Work
    and any allocation go to ``stream`` (default: the current stream).
    Without a given workspace, the split-KV workspace is one kept per device
    and stream (zeroed when made; a given one must start with
    PA_WORKSPACE_ZERO_BYTES zero bytes; see pa_decode_ex).
    """
    import torch
    B, Hq, D = q.shape
    NP, P, Hkv, _ = k_cache.shape
    if scale is None:
        scale = PA_SCALE_DEFAULT
    ts = _torch_stream(stream, q.device)
    if out is None:
        with torch.cuda.stream(ts):
            out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    opts = make_opts(variant, partition_tokens, schedule, shares, window, merge)
    if workspace is None:
        n = pa_decode_workspace_bytes(B, Hq, Hkv, D, block_tables.shape[1], P, opts)
        if n:
            workspace = _workspace(n, q.device, ts)
    return pa_decode_ex(q, k_cache, v_cache, block_tables, context_lens, scale, Hq, Hkv, D, P,
                        out, stream, opts, workspace)
