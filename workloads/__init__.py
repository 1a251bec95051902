"""Seeded synthetic inputs for decode paged attention.

This module holds random draws, their rounding to a storage type and the
construction of block tables -- nothing of the attention arithmetic.  The
oracle tests, the GPU parity tests and the benchmark all take their inputs
from here, so both sides see the same bytes.

Workloads (the geometry follows the source pages: Qwen3 decode at bf16,
GQA 2, head_dim 128, 28 layers x 32 decoded tokens -- page 1, issue "ROCm
gfx1200: PagedAttnOnline is 8.1x slower per call", Measurement table; page 2,
PR "head_dim=128 decode arm", section "Correctness"; ctx lengths straddling a
32-token page -- page 3, PR "head_dim-128 arm for the warp-split-KV decode
kernel", numerics table):

=================  ===================================================
``tiny``           4 seqs, ctx 1/31/33/100, Hq 16, Hkv 8, d 128, page 32,
                   16-page pool
``single_seq``     1 seq, ctx 1152, Hq 16, Hkv 8, d 128, page 16,
                   2048-page pool; 28 layer caches x 32 query vectors
``batch16``        16 seqs, ctx U[1024, 1152], Hq 16, Hkv 8, d 128, page 16
``hd256_gqa4``     32 seqs, ctx U[512, 4096], Hq 8, Hkv 2, d 256, page 32,
                   K rows x4 on 1% of tokens
``long_ctx_gqa8``  64 seqs, ctx U[8192, 32768], Hq 64, Hkv 8, d 128, page 16
``hd512_gqa4``     16 seqs, ctx U[1024, 4096], Hq 8, Hkv 2, d 512, page 16
                   (head_dim 512; an extra line, not one of the five)
=================  ===================================================

Recipe (NumPy PCG64 ``default_rng(seed)``, draws in this order):

1. context lengths: fixed, or ``rng.integers(lo, hi, B, endpoint=True)``;
2. ``perm = rng.permutation(NP)``; sequence b takes the next ceil(L_b / P)
   entries, in logical order, as its block-table row; unused row entries are
   -1.  NP is the stated pool size, else exactly the pages needed, so the
   sequences' pages interleave at random across the pool;
3. Q ``[n_q, B, Hq, D]`` (n_q = layers x tokens), then for each layer the K
   values and then the V values of the *used* pages, in logical order
   (sequence-major), each ``standard_normal`` fp32 rounded to the storage type
   (bf16 by default, or fp16 / kept fp32; nearest, ties to even).  Unused
   pool pages hold zeros (NaN in poison mode);
4. ``hd256_gqa4`` only: ``rng.random(sum L) < 0.01`` over logical tokens marks
   the tokens whose K rows (every KV head) are multiplied by 4 (exact in bf16).

Poison mode overwrites, after all draws, every unused pool page and every slot
at or past L_b in a sequence's last page with bf16 NaN, so an out-of-range read
or a multiply-by-zero mask shows up as a NaN in the output.

For the 5.4 GB ``long_ctx_gqa8`` pool NumPy would take minutes; ``device_inputs``
draws Q/K/V with torch's generator on the GPU instead (steps 1, 2 and 4 stay
NumPy).  Those values differ from the NumPy draws, so every check compares
against the oracle evaluated on host copies of the very same tensors.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    ctx: tuple = ()              # fixed lengths, or () when drawn
    ctx_range: tuple = ()        # (lo, hi) inclusive
    pool_pages: int = 0          # 0 = exactly the pages needed
    spike_frac: float = 0.0      # fraction of tokens whose K rows are x4
    layers: int = 1
    tokens: int = 1              # distinct query vectors per layer
    desc: str = ""

    @property
    def qg(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def calls(self) -> int:
        return self.layers * self.tokens


WORKLOADS = {
    "tiny": Workload("tiny", 4, 16, 8, 128, 32, ctx=(1, 31, 33, 100), pool_pages=16,
                     desc="4 seqs ctx 1/31/33/100, Hq16/Hkv8, d128, page 32, 16-page pool"),
    "single_seq": Workload("single_seq", 1, 16, 8, 128, 16, ctx=(1152,), pool_pages=2048,
                           layers=28, tokens=32,
                           desc="1 seq ctx 1152, Hq16/Hkv8, d128, page 16, 2048-page pool, "
                                "28 layers x 32 tokens"),
    "batch16": Workload("batch16", 16, 16, 8, 128, 16, ctx_range=(1024, 1152),
                        desc="16 seqs ctx U[1024,1152], Hq16/Hkv8, d128, page 16"),
    "hd256_gqa4": Workload("hd256_gqa4", 32, 8, 2, 256, 32, ctx_range=(512, 4096),
                           spike_frac=0.01,
                           desc="32 seqs ctx U[512,4096], Hq8/Hkv2, d256, page 32, 1% K x4"),
    "long_ctx_gqa8": Workload("long_ctx_gqa8", 64, 64, 8, 128, 16, ctx_range=(8192, 32768),
                              desc="64 seqs ctx U[8192,32768], Hq64/Hkv8, d128, page 16"),
    # head_dim 512 (the pages' EPL=16 case): not one of the five configurations
    "hd512_gqa4": Workload("hd512_gqa4", 16, 8, 2, 512, 16, ctx_range=(1024, 4096),
                           desc="16 seqs ctx U[1024,4096], Hq8/Hkv2, d512, page 16"),
}
ORDER = ["tiny", "single_seq", "batch16", "hd256_gqa4", "long_ctx_gqa8"]


def custom(name="custom", batch=1, num_q_heads=16, num_kv_heads=8, head_dim=128,
           page_size=16, ctx=(), ctx_range=(), pool_pages=0, spike_frac=0.0,
           layers=1, tokens=1) -> Workload:
    return Workload(name, batch, num_q_heads, num_kv_heads, head_dim, page_size,
                    tuple(ctx), tuple(ctx_range), pool_pages, spike_frac, layers, tokens)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


@dataclass
class Layout:
    """Context lengths, block tables and the page bookkeeping of one workload."""
    context_lens: np.ndarray           # [B] int32
    block_tables: np.ndarray           # [B, MaxBlk] int32, -1 past the used pages
    num_pages: int
    used_pages: np.ndarray             # physical ids in logical (sequence-major) order
    spike_tokens: np.ndarray = field(default_factory=lambda: np.zeros(0, bool))

    @property
    def total_tokens(self) -> int:
        return int(self.context_lens.sum())


def make_layout(w: Workload, rng: np.random.Generator) -> Layout:
    B, P = w.batch, w.page_size
    if w.ctx:
        if len(w.ctx) != B:
            raise ValueError("fixed ctx list must have one entry per sequence")
        ctx = np.asarray(w.ctx, dtype=np.int64)
    else:
        lo, hi = w.ctx_range
        ctx = rng.integers(lo, hi, B, endpoint=True).astype(np.int64)
    n_b = (ctx + P - 1) // P
    need = int(n_b.sum())
    NP = w.pool_pages or need
    if NP < need:
        raise ValueError(f"pool of {NP} pages cannot hold {need}")
    perm = rng.permutation(NP)
    max_blk = max(int(n_b.max()) if B else 0, 1)
    bt = np.full((B, max_blk), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        bt[b, :n_b[b]] = perm[pos:pos + n_b[b]]
        pos += n_b[b]
    return Layout(ctx.astype(np.int32), bt, NP, perm[:need].astype(np.int64))


def _spikes(w: Workload, lay: Layout, rng) -> np.ndarray:
    if w.spike_frac <= 0:
        return np.zeros(lay.total_tokens, dtype=bool)
    return rng.random(lay.total_tokens) < w.spike_frac


def _token_slots(w: Workload, lay: Layout):
    """(physical page, slot) of every logical token, sequence-major."""
    pages, slots = [], []
    P = w.page_size
    for b in range(w.batch):
        L = int(lay.context_lens[b])
        t = np.arange(L)
        pages.append(lay.block_tables[b, t // P].astype(np.int64))
        slots.append(t % P)
    if not pages:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return np.concatenate(pages), np.concatenate(slots)


@dataclass
class Inputs:
    """Host inputs.  bf16 tensors are uint16 bit patterns."""
    w: Workload
    q: np.ndarray            # [n_q, B, Hq, D]
    k: np.ndarray            # [layers, NP, P, Hkv, D]
    v: np.ndarray            # [layers, NP, P, Hkv, D]
    layout: Layout

    @property
    def block_tables(self):
        return self.layout.block_tables

    @property
    def context_lens(self):
        return self.layout.context_lens

    def call(self, i: int = 0):
        """Arguments of call i: (q, k_cache, v_cache) of layer i // tokens."""
        layer = i // self.w.tokens
        return self.q[i], self.k[layer], self.v[layer]


def poison(w: Workload, lay: Layout, k: np.ndarray, v: np.ndarray, dtype: str = "bf16") -> None:
    """Overwrite everything a correct kernel must not read with NaN."""
    nan = _NAN[dtype]
    used = np.zeros(lay.num_pages, dtype=bool)
    used[lay.used_pages] = True
    k[:, ~used] = nan
    v[:, ~used] = nan
    P = w.page_size
    for b in range(w.batch):
        L = int(lay.context_lens[b])
        if L % P:
            last = lay.block_tables[b, (L - 1) // P]
            k[:, last, L % P:] = nan
            v[:, last, L % P:] = nan


# Storage types of generated tensors: bf16 as uint16 bit patterns, fp16 and
# fp32 as numpy float16 / float32.
STORAGE = {"bf16": np.uint16, "f16": np.float16, "f32": np.float32}
_NAN = {"bf16": BF16_NAN, "f16": np.float16(np.nan), "f32": np.float32(np.nan)}


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 draws stored as ``dtype`` (round to nearest even)."""
    if dtype == "bf16":
        return round_bf16(x)
    return x.astype(STORAGE[dtype])


def make_inputs(w: Workload | str, seed: int = 0, poison_unused: bool = False,
                dtype: str = "bf16", q_dtype: str | None = None) -> Inputs:
    """Host (NumPy) inputs following the recipe in the module docstring.
    ``dtype`` is the storage type of K and V (and of Q unless ``q_dtype``
    says otherwise); the draws are the same fp32 values whatever the type."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    q_dtype = q_dtype or dtype
    rng = np.random.default_rng(seed)
    lay = make_layout(w, rng)
    B, Hq, Hkv, D, P = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    q = encode(rng.standard_normal((w.calls, B, Hq, D), dtype=np.float32), q_dtype)
    n_used = lay.used_pages.size
    k = np.zeros((w.layers, lay.num_pages, P, Hkv, D), dtype=STORAGE[dtype])
    v = np.zeros_like(k)
    for layer in range(w.layers):
        xk = rng.standard_normal((n_used, P, Hkv, D), dtype=np.float32)
        xv = rng.standard_normal((n_used, P, Hkv, D), dtype=np.float32)
        k[layer, lay.used_pages] = encode(xk, dtype)
        v[layer, lay.used_pages] = encode(xv, dtype)
    spikes = _spikes(w, lay, rng)
    lay.spike_tokens = spikes
    if spikes.any():
        pg, sl = _token_slots(w, lay)
        for layer in range(w.layers):
            rows = k[layer, pg[spikes], sl[spikes]]               # [n, Hkv, D]
            if dtype == "bf16":
                f = (rows.astype(np.uint32) << 16).view(np.float32) * np.float32(4.0)
                k[layer, pg[spikes], sl[spikes]] = round_bf16(f)  # exact (x4)
            else:
                k[layer, pg[spikes], sl[spikes]] = rows * STORAGE[dtype](4.0)   # exact (x4)
    if poison_unused:
        poison(w, lay, k, v, dtype)
    return Inputs(w, q, k, v, lay)


def kv_bytes(w: Workload, context_lens, window: int = 0, elem_bytes: int = 2) -> int:
    """Algorithmic KV bytes of one call: sum_b min(L_b, window) * Hkv * D * 2
    (K and V) * element size (window 0 = the whole sequence)."""
    lens = np.asarray(context_lens, dtype=np.int64)
    if window:
        lens = np.minimum(lens, window)
    return int(lens.sum()) * w.num_kv_heads * w.head_dim * 2 * elem_bytes


# ----------------------------------------------------------------------------
# Device-side inputs (torch) -- used for the large pools.
# ----------------------------------------------------------------------------
@dataclass
class DeviceInputs:
    w: Workload
    q: object                # torch bf16 [n_q, B, Hq, D]
    k: object                # torch bf16 [layers, NP, P, Hkv, D]
    v: object
    block_tables: object     # torch int32 [B, MaxBlk]
    context_lens: object     # torch int32 [B]
    layout: Layout

    def call(self, i: int = 0):
        layer = i // self.w.tokens
        return self.q[i], self.k[layer], self.v[layer]


def to_device(inp: Inputs, device="cuda") -> DeviceInputs:
    import torch
    def bf(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:                    # bf16 bit patterns
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(a).to(device)       # float16 / float32
    return DeviceInputs(inp.w, bf(inp.q), bf(inp.k), bf(inp.v),
                        torch.from_numpy(inp.block_tables).to(device),
                        torch.from_numpy(inp.context_lens).to(device), inp.layout)


def device_inputs(w: Workload | str, seed: int = 0, device="cuda", dtype: str = "bf16") -> DeviceInputs:
    """Same layout recipe (steps 1, 2, 4); Q/K/V drawn on the device with
    ``torch.Generator(device).manual_seed(seed)`` as N(0, 1) fp32 rounded to
    the storage type (bf16 by default; torch rounds to nearest even).  Unused
    pool pages hold zeros."""
    import torch
    if isinstance(w, str):
        w = WORKLOADS[w]
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    rng = np.random.default_rng(seed)
    lay = make_layout(w, rng)
    spikes = _spikes(w, lay, rng)
    lay.spike_tokens = spikes
    B, Hq, Hkv, D, P = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = torch.randn((w.calls, B, Hq, D), generator=gen, device=device).to(tdt)
    used = torch.from_numpy(lay.used_pages).to(device)
    full = lay.used_pages.size == lay.num_pages and np.array_equal(
        np.sort(lay.used_pages), np.arange(lay.num_pages))
    k = torch.zeros((w.layers, lay.num_pages, P, Hkv, D), dtype=tdt, device=device)
    v = torch.zeros_like(k)
    chunk = 4096
    for layer in range(w.layers):
        for dst in (k, v):
            for s in range(0, used.numel(), chunk):
                ids = used[s:s + chunk]
                vals = torch.randn((ids.numel(), P, Hkv, D), generator=gen,
                                   device=device).to(tdt)
                if full:
                    dst[layer].index_copy_(0, ids, vals)
                else:
                    dst[layer][ids] = vals
    if spikes.any():
        pg, sl = _token_slots(w, lay)
        pg_t = torch.from_numpy(pg[spikes]).to(device)
        sl_t = torch.from_numpy(sl[spikes]).to(device)
        for layer in range(w.layers):
            k[layer, pg_t, sl_t] = k[layer, pg_t, sl_t] * 4
    return DeviceInputs(w, q, k, v, torch.from_numpy(lay.block_tables).to(device),
                        torch.from_numpy(lay.context_lens).to(device), lay)


def host_copy(d: DeviceInputs) -> Inputs:
    """Bit-exact host copy of device inputs (for the oracle): bf16 as uint16
    bit patterns, fp16 / fp32 as numpy float16 / float32."""
    import torch
    def bits(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()
    return Inputs(d.w, bits(d.q), bits(d.k), bits(d.v), d.layout)
