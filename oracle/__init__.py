"""CPU oracle for decode paged attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it and
it imports nothing from the product package: the two share no code.

Contents
--------
``attention`` / ``attention_pairs``
    ctypes front end of ``pa_oracle.c``: the plain fp64 definition (gather every
    token through the block table, dense softmax with a max shift, weighted sum
    of V) -- page 1 of the source pages, issue "ROCm gfx1200: PagedAttnOnline is
    8.1x slower per call", section "Where to look"; page 2, PR "head_dim=128
    decode arm", section "Correctness" (a CPU oracle at bf16, GQA 2, d=128).
``brute``
    an independent NumPy dense implementation and a ``decimal`` high-precision
    one for tiny inputs; both pin the C oracle.
``compare``
    the NMSE / max-abs / bitwise comparator and its self-test (page 3, PR
    "head_dim-128 arm for the warp-split-KV decode kernel", comparator
    self-test paragraph).

All arrays use bf16 *bits* (``uint16``) for bf16 data, so nothing here depends
on a bf16 dtype in NumPy.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
LIB_PATH = os.path.join(_HERE, "libpa_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``pa_oracle.c`` with gcc into ``libpa_oracle.so`` (in place)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(LIB_PATH)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int
    common = [p, i64, i64, p, p, i64, i64, i64, i64, p, i64, p,
              i32, i32, i32, i32, i32, ctypes.c_float]
    lib.pa_oracle_f64.argtypes = common + [p, i32]
    lib.pa_oracle_f64.restype = i32
    lib.pa_oracle_f64_pairs.argtypes = common + [p, i64, p, i32]
    lib.pa_oracle_f64_pairs.restype = i32
    lib.pa_oracle_f64_mutant.argtypes = common + [p, i32, i32]
    lib.pa_oracle_f64_mutant.restype = i32
    lib.pa_oracle_f64_window.argtypes = common + [i64, p, i32, i32]
    lib.pa_oracle_f64_window.restype = i32
    lib.pa_oracle_f64_pairs_window.argtypes = common + [i64, p, i64, p, i32]
    lib.pa_oracle_f64_pairs_window.restype = i32
    lib.pa_oracle_f64_typed.argtypes = common + [i32, i32, i64, p, i32, i32]
    lib.pa_oracle_f64_typed.restype = i32
    lib.pa_oracle_f64_queries.argtypes = common + [p, i64, i32, i32, i64, p, i32, i32]
    lib.pa_oracle_f64_queries.restype = i32
    lib.pa_oracle_decode.argtypes = [p, i32, i64, p]
    lib.pa_oracle_decode.restype = i32
    lib.pa_oracle_num_mutants.argtypes = []
    lib.pa_oracle_num_mutants.restype = i32
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count() or 1)


# Storage types: bf16 as uint16 bit patterns, IEEE binary16 as numpy float16,
# binary32 as numpy float32 (codes shared with the C oracle).
DTYPE_CODES = {np.dtype(np.uint16): 1, np.dtype(np.float32): 3, np.dtype(np.float16): 4}


def dtype_code(a) -> int:
    code = DTYPE_CODES.get(np.asarray(a).dtype)
    if code is None:
        raise OracleError(f"unsupported element type {np.asarray(a).dtype} "
                          "(uint16 = bf16 bits, float16, float32)")
    return code


def _prep(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads):
    q = np.asarray(q)
    dtype_code(q)
    if q.ndim != 3 or q.strides[2] != q.itemsize:
        raise OracleError("q must be [B, Hq, D] with contiguous D")
    dtype_code(k_cache)
    for name, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        if c.ndim != 4 or c.strides[3] != c.itemsize:
            raise OracleError(f"{name} must be [NP, P, Hkv, D], D contiguous")
    if k_cache.dtype != v_cache.dtype:
        raise OracleError("k_cache and v_cache must share their element type")
    if k_cache.shape != v_cache.shape or k_cache.strides != v_cache.strides:
        raise OracleError("k_cache and v_cache must share shape and strides")
    B, Hq, D = q.shape
    NP, P, Hkv, D2 = k_cache.shape
    if D2 != D or Hkv != num_kv_heads or Hq % Hkv:
        raise OracleError("inconsistent head geometry")
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    if bt.ndim != 2 or bt.shape[0] != B or ctx.shape != (B,):
        raise OracleError("block_tables must be [B, MaxBlk] and context_lens [B]")
    st = [s // k_cache.itemsize for s in k_cache.strides[:3]]
    qst = [s // q.itemsize for s in q.strides[:2]]
    return q, bt, ctx, (B, Hq, D, NP, P, Hkv), st, qst


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def attention(q, k_cache, v_cache, block_tables, context_lens, scale,
              num_kv_heads, threads: int | None = None, mutant: int = 0, window: int = 0):
    """fp64 output [B, Hq, D] of the plain definition.  ``scale`` is taken as
    the fp32 value a caller would pass to the GPU and widened exactly.
    ``window`` > 0 restricts each query to its sequence's last ``window``
    tokens."""
    lib = _load()
    q, bt, ctx, (B, Hq, D, NP, P, Hkv), st, qst = _prep(
        q, k_cache, v_cache, block_tables, context_lens, num_kv_heads)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    n = threads or default_threads()
    args = [_ptr(q), qst[0], qst[1], _ptr(k_cache), _ptr(v_cache), st[0], st[1], st[2], NP,
            _ptr(bt), bt.shape[1], _ptr(ctx), B, Hq, Hkv, D, P, ctypes.c_float(scale)]
    qt, kt = dtype_code(q), dtype_code(k_cache)
    if qt != 1 or kt != 1:
        rc = lib.pa_oracle_f64_typed(*args, qt, kt, int(window), _ptr(out), n, mutant)
    elif window:
        rc = lib.pa_oracle_f64_window(*args, int(window), _ptr(out), n, mutant)
    elif mutant:
        rc = lib.pa_oracle_f64_mutant(*args, _ptr(out), n, mutant)
    else:
        rc = lib.pa_oracle_f64(*args, _ptr(out), n)
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")
    return out


def attention_pairs(q, k_cache, v_cache, block_tables, context_lens, scale,
                    num_kv_heads, pairs, threads: int | None = None, window: int = 0):
    """fp64 rows [n, D] for the selected (b, h) pairs (an int array [n, 2])."""
    lib = _load()
    q, bt, ctx, (B, Hq, D, NP, P, Hkv), st, qst = _prep(
        q, k_cache, v_cache, block_tables, context_lens, num_kv_heads)
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    out = np.zeros((pairs.shape[0], D), dtype=np.float64)
    n = threads or default_threads()
    rc = lib.pa_oracle_f64_pairs_window(
        _ptr(q), qst[0], qst[1], _ptr(k_cache), _ptr(v_cache), st[0], st[1], st[2], NP,
        _ptr(bt), bt.shape[1], _ptr(ctx), B, Hq, Hkv, D, P, ctypes.c_float(scale),
        int(window), _ptr(pairs), pairs.shape[0], _ptr(out), n)
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")
    return out


def attention_queries(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                      num_kv_heads, threads: int | None = None, mutant: int = 0, window: int = 0):
    """Several queries per sequence (chunked prefill): q [n_rows, Hq, D] holds
    sequence b's queries at rows [query_start[b], query_start[b+1]), which are
    its last tokens; query i attends causally to positions up to its own.
    Returns fp64 [n_rows, Hq, D]."""
    lib = _load()
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    ctx_arr = np.asarray(context_lens)
    B = len(ctx_arr)
    if qs.shape != (B + 1,):
        raise OracleError("query_start must have B + 1 entries")
    q = np.asarray(q)
    # the shape checks of _prep, on a [B, Hq, D] view of the first rows
    # (only the pools, tables and head geometry are taken from it)
    probe = np.broadcast_to(q[:1], (B,) + q.shape[1:]) if q.shape[0] else np.zeros((B,) + q.shape[1:], q.dtype)
    _, bt, ctx, (_, Hq, D, NP, P, Hkv), st, _ = _prep(
        np.ascontiguousarray(probe), k_cache, v_cache, block_tables, context_lens, num_kv_heads)
    if q.ndim != 3 or q.strides[2] != q.itemsize:
        raise OracleError("q must be [n_rows, Hq, D] with contiguous D")
    qst = [s // q.itemsize for s in q.strides[:2]]
    out = np.zeros((q.shape[0], Hq, D), dtype=np.float64)
    n = threads or default_threads()
    rc = lib.pa_oracle_f64_queries(
        _ptr(q), qst[0], qst[1], _ptr(k_cache), _ptr(v_cache), st[0], st[1], st[2], NP,
        _ptr(bt), bt.shape[1], _ptr(ctx), B, Hq, Hkv, D, P, ctypes.c_float(scale),
        _ptr(qs), q.shape[0], dtype_code(q), dtype_code(k_cache), int(window), _ptr(out), n, mutant)
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")
    return out


def decode_elements(a) -> np.ndarray:
    """The oracle's fp64 reading of every element of ``a`` (for its tests)."""
    a = np.ascontiguousarray(a)
    out = np.zeros(a.size, dtype=np.float64)
    rc = _load().pa_oracle_decode(_ptr(a), dtype_code(a), a.size, _ptr(out))
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")
    return out.reshape(a.shape)


def num_mutants() -> int:
    return _load().pa_oracle_num_mutants()


def cache_append(k_cache, v_cache, block_tables, context_lens, k_new, v_new):
    """KV-cache append, the step before decode attention: sequence b's newest
    token, position t = context_lens[b] - 1 (the length already counts it),
    has its K and V rows written to page block_tables[b][t // P], slot t % P.
    Sequences with no tokens write nothing.  Returns new (k_cache, v_cache)
    arrays (uint16 bf16 bits); the inputs are not modified.

    The pages name no cache-write kernel; this is the plainest neighbour of
    the decode step (the cache layout is the same NHD pool the decode reads,
    page 1, issue "ROCm gfx1200: PagedAttnOnline is 8.1x slower per call",
    section "Where to look")."""
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    P = k_cache.shape[1]
    for b, L in enumerate(np.asarray(context_lens)):
        L = int(L)
        if L <= 0:
            continue
        t = L - 1
        page = int(block_tables[b][t // P])
        if not 0 <= page < k_cache.shape[0]:
            raise OracleError(f"sequence {b}: page id {page} out of range")
        k_out[page, t % P] = k_new[b]
        v_out[page, t % P] = v_new[b]
    return k_out, v_out
