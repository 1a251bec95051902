"""Independent brute-force references that pin the C oracle (test infrastructure).

``dense``    NumPy fp64: materialise each sequence's K and V densely by
             indexing the pool with its block-table row, then
             ``softmax(K q * s) . V`` with ``scipy.special.softmax`` -- a
             different gather (fancy indexing of whole pages) and a library
             softmax, no shared code with ``pa_oracle.c``.
``exact``    Python ``decimal`` at 50 significant digits for tiny inputs: every
             bf16 product is exact, the exponentials and the final division are
             correct to far beyond fp64, so this is the mathematically exact
             result up to the last fp64 rounding.
``bf16_bits_to_f64`` widens bf16 bit patterns exactly.

The definition both follow is the one the oracle header states (page 1 of the
source pages, issue "ROCm gfx1200: PagedAttnOnline is 8.1x slower per call",
section "Where to look": online-softmax decode over an NHD cache addressed
through a block table and strides).
"""
from __future__ import annotations

import decimal

import numpy as np
from scipy.special import softmax


def bf16_bits_to_f64(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def widen(a) -> np.ndarray:
    """Exact fp64 values of an array: uint16 holds bf16 bit patterns, numpy
    float16 / float32 widen with numpy's own conversion."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def _dense_kv(pool, bt_row, L, P):
    n = -(-L // P)
    pages = pool[np.asarray(bt_row[:n], dtype=np.int64)]   # [n, P, Hkv, D]
    return pages.reshape(n * P, *pool.shape[2:])[:L]        # [L, Hkv, D]


def dense(q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, window=0):
    """[B, Hq, D] fp64 via dense per-sequence K/V and a library softmax.
    ``window`` > 0 keeps only the last ``window`` rows of each sequence."""
    qf = widen(q)
    kf = widen(k_cache)
    vf = widen(v_cache)
    B, Hq, D = qf.shape
    P = kf.shape[1]
    qg = Hq // num_kv_heads
    s = float(np.float32(scale))
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(context_lens[b])
        if L <= 0:
            continue
        Kb = _dense_kv(kf, block_tables[b], L, P)              # [L, Hkv, D]
        Vb = _dense_kv(vf, block_tables[b], L, P)
        if window > 0:
            Kb, Vb = Kb[-window:], Vb[-window:]
        for h in range(Hq):
            g = h // qg
            logits = (Kb[:, g, :] @ qf[b, h]) * s              # [L]
            out[b, h] = softmax(logits) @ Vb[:, g, :]
    return out


def exact(q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads,
          digits: int = 50):
    """[B, Hq, D] fp64 rounded from a ``digits``-digit decimal evaluation.
    For tiny inputs only (pure Python loops)."""
    ctx = decimal.Context(prec=digits)
    D_ = decimal.Decimal
    qf = bf16_bits_to_f64(q)
    kf = bf16_bits_to_f64(k_cache)
    vf = bf16_bits_to_f64(v_cache)
    B, Hq, D = qf.shape
    P = kf.shape[1]
    qg = Hq // num_kv_heads
    s = D_(float(np.float32(scale)))
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(context_lens[b])
        if L <= 0:
            continue
        rows = [(int(block_tables[b][t // P]), t % P) for t in range(L)]
        for h in range(Hq):
            g = h // qg
            qv = [D_(float(x)) for x in qf[b, h]]
            logits = []
            for pg, sl in rows:
                kr = kf[pg, sl, g]
                acc = D_(0)
                for i in range(D):
                    acc = ctx.add(acc, ctx.multiply(qv[i], D_(float(kr[i]))))
                logits.append(ctx.multiply(acc, s))
            m = max(logits)
            w = [ctx.exp(ctx.subtract(x, m)) for x in logits]
            Z = sum(w, D_(0))
            for i in range(D):
                num = D_(0)
                for (pg, sl), wt in zip(rows, w):
                    num = ctx.add(num, ctx.multiply(wt, D_(float(vf[pg, sl, g, i]))))
                out[b, h, i] = float(ctx.divide(num, Z))
    return out


def dense_queries(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                  num_kv_heads, window=0):
    """[n_rows, Hq, D] fp64 for several queries per sequence: dense K/V per
    sequence, a logits matrix [n, L] with a causal (and window) mask of
    -inf, and a library softmax over each row."""
    qf = widen(q)
    kf = widen(k_cache)
    vf = widen(v_cache)
    n_rows, Hq, D = qf.shape
    P = kf.shape[1]
    qg = Hq // num_kv_heads
    s = float(np.float32(scale))
    out = np.zeros((n_rows, Hq, D))
    for b in range(len(context_lens)):
        L = int(context_lens[b])
        r0, r1 = int(query_start[b]), int(query_start[b + 1])
        n = r1 - r0
        if n == 0 or L <= 0:
            continue
        Kb = _dense_kv(kf, block_tables[b], L, P)              # [L, Hkv, D]
        Vb = _dense_kv(vf, block_tables[b], L, P)
        pos = np.arange(L - n, L)[:, None]                     # [n, 1]
        t = np.arange(L)[None, :]                              # [1, L]
        allowed = t <= pos
        if window > 0:
            allowed &= t > pos - window
        for h in range(Hq):
            g = h // qg
            logits = (qf[r0:r1, h] @ Kb[:, g, :].T) * s       # [n, L]
            logits = np.where(allowed, logits, -np.inf)
            out[r0:r1, h] = softmax(logits, axis=1) @ Vb[:, g, :]
    return out
