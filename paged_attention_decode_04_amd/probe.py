"""ctypes binding of ``libpa_probe.so`` (``include/pa_probe.h``): streaming-read
probes, the bandwidth references the decode kernels are measured against.
Measurement aids of the benchmark; argument marshalling only."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_HERE, "libpa_probe.so")


class PaProbePaged(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_sp", ctypes.c_int64), ("k_ss", ctypes.c_int64), ("k_sh", ctypes.c_int64),
                ("v_sp", ctypes.c_int64), ("v_ss", ctypes.c_int64), ("v_sh", ctypes.c_int64),
                ("row_bytes", ctypes.c_int32), ("block_tables", ctypes.c_void_p), ("bt_sb", ctypes.c_int64),
                ("context_lens", ctypes.c_void_p), ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("max_blocks", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with "
                              "`python -m paged_attention_decode_04_amd.build`")
        lib = ctypes.CDLL(PROBE_LIB_PATH)
        lib.pa_probe_read_contiguous.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                                 ctypes.c_void_p]
        lib.pa_probe_read_contiguous.restype = ctypes.c_int
        lib.pa_probe_read_paged.argtypes = [ctypes.POINTER(PaProbePaged), ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_void_p]
        lib.pa_probe_read_paged.restype = ctypes.c_int
        ip = ctypes.POINTER(ctypes.c_int)
        lib.pa_probe_issue_modes.argtypes = [ctypes.c_int, ip, ip, ip]
        lib.pa_probe_issue_modes.restype = ctypes.c_int
        lib.pa_probe_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.pa_probe_issue.restype = ctypes.c_int
        _lib = lib
    return _lib


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def read_contiguous(buf, n_wg: int, sink, stream=None) -> None:
    """Read every byte of the contiguous device tensor ``buf`` once."""
    rc = _load().pa_probe_read_contiguous(buf.data_ptr(), buf.numel() * buf.element_size(), int(n_wg),
                                          sink.data_ptr(), _stream(stream))
    if rc:
        raise RuntimeError(f"pa_probe_read_contiguous returned {rc}")


def paged_desc(k_cache, v_cache, block_tables, context_lens) -> PaProbePaged:
    """Descriptor of a paged NHD cache [NP, P, Hkv, D] (torch tensors)."""
    es = k_cache.element_size()
    NP, P, Hkv, D = k_cache.shape
    d = PaProbePaged()
    d.k, d.v = k_cache.data_ptr(), v_cache.data_ptr()
    d.k_sp, d.k_ss, d.k_sh = (s * es for s in k_cache.stride()[:3])
    d.v_sp, d.v_ss, d.v_sh = (s * es for s in v_cache.stride()[:3])
    d.row_bytes = D * es
    d.block_tables, d.bt_sb = block_tables.data_ptr(), block_tables.stride(0)
    d.context_lens = context_lens.data_ptr()
    d.batch, d.num_kv_heads, d.page_size = block_tables.shape[0], Hkv, P
    d.num_pages, d.max_blocks = NP, block_tables.shape[1]
    return d


def read_paged(desc: PaProbePaged, n_wg: int, sink, stream=None) -> None:
    """Read the K and V rows of every (sequence, KV head, token) once."""
    rc = _load().pa_probe_read_paged(ctypes.byref(desc), int(n_wg), sink.data_ptr(), _stream(stream))
    if rc:
        raise RuntimeError(f"pa_probe_read_paged returned {rc}")


def issue_modes() -> list:
    """The issue-rate probe's menu: (MFMAs, FMAs, mixed) per round, per mode."""
    lib = _load()
    n = lib.pa_probe_issue_modes(-1, None, None, None)
    out = []
    for i in range(n):
        nm, nv, mixed = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        if lib.pa_probe_issue_modes(i, ctypes.byref(nm), ctypes.byref(nv), ctypes.byref(mixed)) != n:
            raise RuntimeError(f"pa_probe_issue_modes({i}) failed")
        out.append((nm.value, nv.value, bool(mixed.value)))
    return out


def issue(mode: int, n_wg: int, rounds: int, sink, stream=None) -> None:
    """Run mode ``mode`` of the issue-rate probe (n_wg workgroups of 256 threads)."""
    rc = _load().pa_probe_issue(int(mode), int(n_wg), int(rounds), sink.data_ptr(), _stream(stream))
    if rc:
        raise RuntimeError(f"pa_probe_issue returned {rc}")
