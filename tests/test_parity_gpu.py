"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

The bar (stated with the method): NMSE <= 5e-4 and max-abs <= 1e-2 on the bf16
outputs; bit-exact where the result is exact (ctx = 1 returns a V row) or the
reduction order cannot change (physical page relabelling, reruns).  Every
test asserts through the launch counters that the intended kernel variant and
split mode actually ran.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import paged_attention_decode_04_amd as pa
import workloads
from oracle.compare import bf16_bits_to_f64, compare
from workloads import WORKLOADS, custom, make_inputs, to_device

pytestmark = pytest.mark.gpu

# Kernel variant and work schedule: vector-ALU kernel on fixed partitions,
# MFMA kernel on fixed partitions, MFMA kernel on balanced shares, MFMA
# kernel on fitted partitions (size picked on the device; no window).
# "-fused": the same partitions merged inside the decode kernel by the last
# partition of each group to finish (no merge kernel).
VARIANTS = ["valu", "mfma", "mfma-bal", "mfma-fit", "mfma-fused", "mfma-fit-fused"]
VARIANTS_W = ["valu", "mfma", "mfma-bal", "mfma-fused"]   # those that take a window
_MODE = {"valu": ("valu", "partitions"), "mfma": ("mfma", "partitions"),
         "mfma-bal": ("mfma", "balanced"), "mfma-fit": ("mfma", "fitted"),
         "mfma-fused": ("mfma", "partitions"), "mfma-fit-fused": ("mfma", "fitted")}
_MERGE = {"mfma-fused": "fused", "mfma-fit-fused": "fused"}
# Share counts the balanced schedule is exercised with: automatic, a single
# share (every group written directly), and counts whose boundaries fall
# mid-group, mid-sequence and on 16-token tiles of different sequences.
SHARES = (0, 1, 3, 37, 1024)
# Workgroup targets of the fitted schedule: automatic (one per compute unit),
# one (no size fits: the largest is taken), a few, and more than any
# partitioning needs (the smallest size is taken).
FIT_TARGETS = (0, 1, 5, 64, 1024)


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_out(t):
    """An output tensor on the host: bf16 as uint16 bits, fp16 / fp32 as numpy
    float16 / float32 (what the comparator takes)."""
    if t.dtype == torch.bfloat16:
        return bits(t)
    return t.contiguous().cpu().numpy()


def knobs(variant, tokens):
    """Split settings to sweep: partition sizes, or share counts when balanced."""
    if _MODE[variant][1] == "balanced":
        return [dict(shares=n) for n in SHARES]
    if _MODE[variant][1] == "fitted":
        return [dict(shares=n) for n in FIT_TARGETS]
    if variant == "mfma-fused":
        # every split size, and one partition (no split: nothing to merge)
        return [dict(partition_tokens=T) for T in tokens + (64, 1 << 20)]
    return [dict(partition_tokens=T) for T in tokens]


def gpu_run(d, call=0, variant="valu", partition_tokens=0, shares=0, window=0, out_dtype=None, workspace=None,
            scale=None):
    kernel, schedule = _MODE[variant]
    merge = _MERGE.get(variant, "kernel")
    q, k, v = d.call(call)
    out = torch.full(q.shape, float("nan"), dtype=out_dtype or q.dtype, device=q.device)   # every row must be written
    pa.pa_reset_stats()
    pa.decode(q, k, v, d.block_tables, d.context_lens, d.w.scale if scale is None else scale, out=out, variant=kernel,
              partition_tokens=partition_tokens, schedule=schedule, shares=shares, window=window,
              merge=merge if kernel == "mfma" and schedule != "balanced" else "auto", workspace=workspace)
    torch.cuda.synchronize()
    s = pa.pa_get_stats()
    assert s["calls"] == 1
    assert s[f"{kernel}_launches"] == 1, s
    if merge == "fused":
        assert s["merge_launches"] == 0 and s["fused_calls"] == s["split_calls"], s
    elif s["split_calls"]:
        assert s["merge_launches"] == 1 and s["fused_calls"] == 0, s
    expect = {"balanced": pa.PA_SCHEDULE_BALANCED, "partitions": pa.PA_SCHEDULE_PARTITIONS,
              # a call that does not split runs one partition per sequence
              "fitted": pa.PA_SCHEDULE_FITTED if s["split_calls"] else pa.PA_SCHEDULE_PARTITIONS}
    assert s["last_schedule"] == expect[schedule], s
    if schedule == "balanced":
        assert s["balanced_calls"] == 1 and s["merge_launches"] == 1, s
        if shares:
            assert s["last_num_partitions"] == shares, s
    return host_out(out), s


def oracle_run(inp, call=0, window=0, scale=None):
    q, k, v = inp.call(call)
    return oracle.attention(q, k, v, inp.block_tables, inp.context_lens, inp.w.scale if scale is None else scale,
                            inp.w.num_kv_heads, window=window)


def assert_parity(y, ref, what=""):
    r = compare(y, ref)
    print(f"[parity] {what}: {r}", flush=True)
    assert r.ok(), f"{what}: {r}"
    return r


@pytest.fixture(autouse=True)
def _dev(gpu):
    yield


# ------------------------------------------------------------------ configs
@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("name", ["tiny", "batch16", "hd256_gqa4"])
def test_config_parity(name, variant):
    inp = make_inputs(name, seed=0)
    y, s = gpu_run(to_device(inp), variant=variant)
    assert_parity(y, oracle_run(inp), f"{name}/{variant} T={s['last_partition_tokens']}")


@pytest.mark.parametrize("variant", ["valu", "mfma", "mfma-fit"])
def test_hd512_full_size(variant):
    """The head_dim-512 workload timed by the benchmark (16 seqs, ctx
    U[1024,4096], Hq8/Hkv2), all rows against the oracle, on both kernels
    (the automatic choice is the MFMA one)."""
    inp = make_inputs("hd512_gqa4", seed=0)
    y, s = gpu_run(to_device(inp), variant=variant)
    assert_parity(y, oracle_run(inp), f"hd512_gqa4/{variant} T={s['last_partition_tokens']}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_single_seq_layers_and_tokens(variant):
    """The 28-layer x 32-token workload: several calls spread over layers."""
    inp = make_inputs("single_seq", seed=0)
    d = to_device(inp)
    for call in (0, 31, 32, 500, 895):
        y, s = gpu_run(d, call=call, variant=variant)
        assert s["split_calls"] == 1
        assert_parity(y, oracle_run(inp, call), f"single_seq call {call}")


class LongContext:
    """The full-size long-context workload (64 sequences of 8192-32768
    tokens, Hq 64 / Hkv 8, d 128, page 16; 5.4 GB of K/V, pools > 2 GiB each,
    so 64-bit offsets are exercised) on the device, a host copy of the same
    tensors, and the oracle over every (sequence, head) row, per window
    (computed once: about 43 GFLOP of fp64 without a window)."""

    def __init__(self):
        self.w = WORKLOADS["long_ctx_gqa8"]
        self.d = workloads.device_inputs(self.w, seed=0)
        self.host = workloads.host_copy(self.d)
        self._refs = {}

    def ref(self, window=0):
        if window not in self._refs:
            h = self.host
            self._refs[window] = oracle.attention(h.q[0], h.k[0], h.v[0], h.block_tables, h.context_lens,
                                                  self.w.scale, self.w.num_kv_heads, window=window)
        return self._refs[window]


@pytest.fixture(scope="module")
def long_ctx(gpu):
    lc = LongContext()
    yield lc
    del lc.d, lc.host
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant", VARIANTS)
def test_long_context_all_rows(variant, long_ctx):
    """The headline workload in the benchmark's launch configuration (and on
    every other kernel and schedule): all 4096 (sequence, head) rows, every
    element, against the oracle."""
    y, s = gpu_run(long_ctx.d, variant=variant)
    assert s["split_calls"] == 1
    assert_parity(y, long_ctx.ref(), f"long_ctx all rows {variant}")


class SingleLong:
    """One sequence of 200,003 tokens (Hq 64 / Hkv 8, d 128, page 16; 820 MB
    of K/V): every schedule cuts each of its 8 query blocks into many
    partitions or pieces (up to 3126 per row at 64-token partitions), so the
    merges run far past the partials they read in their first round trip."""

    def __init__(self):
        w = custom("single_long", batch=1, num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=16,
                   ctx=(200003,))
        self.inp = make_inputs(w, seed=21)
        self.d = to_device(self.inp)
        self._ref = None

    def ref(self):
        if self._ref is None:
            self._ref = oracle_run(self.inp)
        return self._ref


@pytest.fixture(scope="module")
def single_long(gpu):
    sl = SingleLong()
    yield sl
    del sl.d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant", VARIANTS)
def test_single_long_sequence(variant, single_long):
    for kn in knobs(variant, (0, 64, 4096)):
        y, s = gpu_run(single_long.d, variant=variant, **kn)
        # a partition holds at most 8192 pages' tokens (131072 here), so even
        # the largest size asked for splits this sequence
        assert s["split_calls"] == 1, s
        assert_parity(y, single_long.ref(),
                      f"200003 tokens {variant} {kn} (x{s['last_num_partitions']}, T={s['last_partition_tokens']})")


# ------------------------------------------------------------------ geometry
@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 4), (8, 2), (16, 2), (32, 2), (6, 6), (12, 3), (40, 5)])
def test_head_geometries(D, Hq, Hkv, variant):
    w = custom(batch=3, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=16,
               ctx=(1, 257, 700))
    inp = make_inputs(w, seed=D + Hq)
    d = to_device(inp)
    ref = oracle_run(inp)
    for kn in knobs(variant, (0, 64, 4096)):
        y, _ = gpu_run(d, variant=variant, **kn)
        assert_parity(y, ref, f"D={D} Hq={Hq} Hkv={Hkv} {kn}")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("P,lens", [(32, (1, 31, 32, 33, 64, 100, 685, 1000)),
                                    (16, (15, 16, 17)), (1, (1, 2, 77)), (7, (6, 7, 8, 50))])
def test_page_boundary_sweep_poisoned(P, lens, variant):
    """ctx lengths straddling the page boundary, with every unread slot and
    page set to NaN: any out-of-range read or multiply-by-zero mask shows."""
    w = custom(batch=len(lens), num_q_heads=16, num_kv_heads=8, head_dim=128, page_size=P,
               ctx=lens, pool_pages=sum(-(-L // P) for L in lens) + 5)
    inp = make_inputs(w, seed=P, poison_unused=True)
    d = to_device(inp)
    ref = oracle_run(inp)
    for kn in knobs(variant, (0, 64, 128)):
        y, _ = gpu_run(d, variant=variant, **kn)
        assert np.all(np.isfinite(workloads_f32(y)))
        assert_parity(y, ref, f"P={P} {kn}")


def workloads_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("D,Hq,Hkv,P", [(128, 16, 8, 48), (128, 16, 8, 64), (128, 16, 8, 256),
                                        (256, 8, 2, 128)])
def test_large_pages_poisoned(D, Hq, Hkv, P, variant):
    """Pages of several tiles, as long as a partition or longer (48 to 256
    tokens): lengths on and off page and partition boundaries, with every
    unread slot and page set to NaN."""
    lens = (1, P - 1, P, P + 1, 1000, 4097, 9000)
    w = custom(batch=len(lens), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
               ctx=lens, pool_pages=sum(-(-L // P) for L in lens) + 3)
    inp = make_inputs(w, seed=P + D, poison_unused=True)
    d = to_device(inp)
    ref = oracle_run(inp)
    for kn in knobs(variant, (0, 64, 320)):
        y, _ = gpu_run(d, variant=variant, **kn)
        assert np.all(np.isfinite(workloads_f32(y)))
        assert_parity(y, ref, f"D={D} P={P} {kn}")


# ------------------------------------------------------------------ exactness
@pytest.mark.parametrize("variant", VARIANTS)
def test_scale_sweep(variant):
    """Logit scales from a nearly flat to a nearly one-hot softmax, and a
    negative one, over keys with 2% of rows x4: the lazy rescale, the
    weights' hi + lo split at weights far above 1, and merges of partitions
    whose maxima lie far apart all stay within the bar."""
    w = custom(batch=5, num_q_heads=16, num_kv_heads=8, head_dim=128, page_size=16,
               ctx=(1, 100, 700, 2000, 5000), spike_frac=0.02)
    inp = make_inputs(w, seed=33)
    d = to_device(inp)
    for f in (1e-3, 0.25, 4.0, 16.0, 64.0, -2.0):
        sc = float(np.float32(w.scale * f))
        ref = oracle_run(inp, scale=sc)
        for kn in knobs(variant, (0, 64)):
            y, _ = gpu_run(d, variant=variant, scale=sc, **kn)
            assert_parity(y, ref, f"scale x{f} {kn}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_ctx1_returns_v_row_bitwise(variant):
    w = custom(batch=5, num_q_heads=16, num_kv_heads=8, head_dim=128, page_size=32,
               ctx=(1, 1, 1, 1, 1), pool_pages=9)
    inp = make_inputs(w, seed=3)
    y, _ = gpu_run(to_device(inp), variant=variant)
    y = y.reshape(5, 16, 128)
    for b in range(5):
        for h in range(16):
            assert np.array_equal(y[b, h], inp.v[0][inp.block_tables[b, 0], 0, h // 2])


@pytest.mark.parametrize("variant", VARIANTS)
def test_page_relabelling_is_bitwise_invariant(variant):
    inp = make_inputs("tiny", seed=4)
    y0, _ = gpu_run(to_device(inp), variant=variant)
    NP = inp.layout.num_pages
    pi = np.random.default_rng(9).permutation(NP)
    k2 = np.empty_like(inp.k); k2[:, pi] = inp.k
    v2 = np.empty_like(inp.v); v2[:, pi] = inp.v
    bt = inp.block_tables
    bt2 = np.where(bt >= 0, pi[np.maximum(bt, 0)], -1).astype(np.int32)
    lay2 = workloads.Layout(inp.context_lens, bt2, NP, pi[inp.layout.used_pages])
    inp2 = workloads.Inputs(inp.w, inp.q, k2, v2, lay2)
    y1, _ = gpu_run(to_device(inp2), variant=variant)
    assert np.array_equal(y0, y1)


@pytest.mark.parametrize("variant", VARIANTS)
def test_reruns_are_bitwise_identical(variant):
    inp = make_inputs("batch16", seed=0)
    d = to_device(inp)
    y0, _ = gpu_run(d, variant=variant)
    for _ in range(3):
        y1, _ = gpu_run(d, variant=variant)
        assert np.array_equal(y0, y1)


@pytest.mark.parametrize("variant", VARIANTS)
def test_split_sizes_agree(variant):
    inp = make_inputs("batch16", seed=1)
    d = to_device(inp)
    ref = oracle_run(inp)
    seen = set()
    for kn in knobs(variant, (64, 128, 320, 1024, 1 << 20)):
        y, s = gpu_run(d, variant=variant, **kn)
        seen.add(s["split_calls"])
        assert_parity(y, ref, f"{kn}")
    assert seen == ({1} if variant in ("mfma-bal", "mfma-fit", "mfma-fit-fused") else {0, 1})


# ------------------------------------------------------------------ layouts
@pytest.mark.parametrize("variant", VARIANTS)
def test_strided_views(variant):
    """K and V as views into one interleaved buffer, q with a padded head
    stride and out with a padded batch stride."""
    inp = make_inputs("tiny", seed=6)
    d = to_device(inp)
    q0, k0, v0 = d.call(0)
    NP, P, Hkv, D = k0.shape
    kv = torch.empty((NP, P, Hkv, 2 * D), dtype=torch.bfloat16, device=k0.device)
    kv[..., :D] = k0
    kv[..., D:] = v0
    qpad = torch.zeros((q0.shape[0], q0.shape[1], D + 64), dtype=torch.bfloat16, device=q0.device)
    qpad[..., :D] = q0
    obuf = torch.zeros((q0.shape[0] + 1, q0.shape[1], D), dtype=torch.bfloat16, device=q0.device)
    out = obuf[1:]
    kernel, schedule = _MODE[variant]
    pa.pa_reset_stats()
    pa.decode(qpad[..., :D], kv[..., :D], kv[..., D:], d.block_tables, d.context_lens,
              inp.w.scale, out=out, variant=kernel, schedule=schedule)
    torch.cuda.synchronize()
    assert pa.pa_get_stats()[f"{kernel}_launches"] == 1
    assert_parity(bits(out), oracle_run(inp), "strided views")
    assert torch.all(obuf[0] == 0)


@pytest.mark.parametrize("variant", VARIANTS)
def test_empty_sequences_and_batch(variant):
    w = custom(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
               ctx=(0, 40, 0), pool_pages=4)
    inp = make_inputs(w, seed=8)
    d = to_device(inp)
    for kn in knobs(variant, (0, 64)):
        y, _ = gpu_run(d, variant=variant, **kn)
        y = y.reshape(3, 8, 128)
        assert np.all(y[0] == 0) and np.all(y[2] == 0)
        assert_parity(y, oracle_run(inp), f"empty {kn}")
    # every sequence empty: all rows zero, and no partial is ever read
    w0 = custom(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                ctx=(0, 0), pool_pages=1)
    d0 = to_device(make_inputs(w0, seed=8))
    for kn in knobs(variant, (0,)):
        y, _ = gpu_run(d0, variant=variant, **kn)
        assert np.all(y == 0)
    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = pa.decode(q, d.k[0], d.v[0], d.block_tables[:0], d.context_lens[:0], 0.1)
    assert out.shape == (0, 8, 128)


def test_library_workspace_entry_point():
    """pa_decode (library-owned workspace) equals pa_decode_ex (caller's)."""
    inp = make_inputs("single_seq", seed=0)
    d = to_device(inp)
    q, k, v = d.call(7)
    out1 = torch.empty_like(q)
    pa.pa_decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale, 16, 8, 128, 16, out1)
    out2 = pa.decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    pa.pa_release()


def test_device_errors_do_not_stick():
    """An invalid call raises and leaves the library usable."""
    inp = make_inputs("tiny", seed=0)
    d = to_device(inp)
    q, k, v = d.call(0)
    with pytest.raises(pa.PaError):
        pa.pa_decode(q, k, v, d.block_tables, d.context_lens, float("inf"), 16, 8, 128, 32,
                     torch.empty_like(q))
    y, _ = gpu_run(d)
    assert_parity(y, oracle_run(inp), "after error")


def test_default_scale_is_the_fp32_reciprocal_root():
    """PA_SCALE_DEFAULT (what decode() and prefill() pass when no scale is
    given) gives the same bits as the fp32 value nearest 1/sqrt(D) passed
    explicitly, at every head size."""
    for D, Hq, Hkv, P in ((128, 16, 8, 16), (256, 8, 2, 32), (512, 8, 2, 16)):
        w = custom(batch=3, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P, ctx=(5, 300, 900))
        inp = make_inputs(w, seed=D)
        d = to_device(inp)
        q, k, v = d.call(0)
        y0 = pa.decode(q, k, v, d.block_tables, d.context_lens)
        y1 = pa.decode(q, k, v, d.block_tables, d.context_lens, float(np.float32(1.0 / np.sqrt(D))))
        qs = torch.arange(0, 4, dtype=torch.int32, device="cuda")
        if D != 512:
            z0 = pa.prefill(q, k, v, d.block_tables, d.context_lens, qs)
            z1 = pa.prefill(q, k, v, d.block_tables, d.context_lens, qs, float(np.float32(1.0 / np.sqrt(D))))
            torch.cuda.synchronize()
            assert torch.equal(z0, z1), D
        torch.cuda.synchronize()
        assert torch.equal(y0, y1), D
        assert_parity(bits(y0), oracle_run(inp), f"default scale D={D}")


def test_side_stream_calls():
    """decode() and prefill() given another stream: the workspace and output
    are made on that stream and the work runs there (the results match the
    oracle after the caller waits for that stream)."""
    inp = make_inputs("hd256_gqa4", seed=5)
    d = to_device(inp)
    q, k, v = d.call(0)
    ref = oracle_run(inp)
    for sched in ("auto", "balanced", "partitions"):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        out = pa.decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale, schedule=sched, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        assert_parity(bits(out), ref, f"side stream {sched}")
    B = q.shape[0]
    qs = torch.arange(0, B + 1, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out = pa.prefill(q, k, v, d.block_tables, d.context_lens, qs, inp.w.scale, schedule="partitions",
                     partition_tokens=256, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert_parity(bits(out), ref, "side stream prefill")


def test_library_workspace_refused_under_capture():
    """pa_decode (the library's own workspace) on a stream under graph
    capture returns PA_EINVAL before enqueuing anything; the same call with
    a caller workspace captures and replays."""
    inp = make_inputs("single_seq", seed=1)
    d = to_device(inp)
    q, k, v = d.call(0)
    out = torch.empty_like(q)
    eager = pa.decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    code = None
    with torch.cuda.graph(g):
        out.zero_()
        try:
            pa.pa_decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale, 16, 8, 128, 16, out)
        except pa.PaError as e:
            code = e.code
    assert code == pa.PA_EINVAL, code
    assert "captured" in pa.last_error()
    g.replay()
    torch.cuda.synchronize()
    assert bool(torch.all(out == 0))
    y = pa.decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale)
    torch.cuda.synchronize()
    assert torch.equal(y, eager)


@pytest.mark.parametrize("schedule,B", [("fitted", 256), ("fitted", 257), ("balanced", 4096), ("balanced", 4097)])
def test_schedule_batch_caps(schedule, B):
    """At the batch caps of the fitted (256 sequences) and balanced (4096)
    schedules: at the cap the forced schedule runs and matches the oracle;
    one sequence past it, forcing the schedule is PA_ENOTSUP and the
    automatic choice falls back to fixed partitions, also at parity."""
    rng = np.random.default_rng(B)
    hi = 700 if schedule == "fitted" else 70
    lens = tuple(int(x) for x in rng.integers(0, hi + 1, B))
    w = custom(batch=B, num_q_heads=8, num_kv_heads=8 if schedule == "balanced" else 2, head_dim=128,
               page_size=16, ctx=lens)
    inp = make_inputs(w, seed=B, poison_unused=True)
    d = to_device(inp)
    ref = oracle_run(inp)
    cap = 256 if schedule == "fitted" else 4096
    variant = "mfma-fit" if schedule == "fitted" else "mfma-bal"
    if B <= cap:
        y, s = gpu_run(d, variant=variant, shares=64 if schedule == "fitted" else 0)
        assert_parity(y, ref, f"{schedule} at its cap B={B}")
        return
    q, k, v = d.call(0)
    with pytest.raises(pa.PaError) as e:
        pa.decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale, variant="mfma", schedule=schedule)
    assert e.value.code == pa.PA_ENOTSUP
    out = torch.full_like(q, float("nan"))
    pa.pa_reset_stats()
    pa.decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale, out=out, partition_tokens=0,
              schedule="auto")
    torch.cuda.synchronize()
    st = pa.pa_get_stats()
    assert st["last_schedule"] == pa.PA_SCHEDULE_PARTITIONS, st
    assert_parity(bits(out), ref, f"automatic past the {schedule} cap B={B}")


@pytest.mark.parametrize("schedule,merge", [("partitions", "kernel"), ("balanced", "auto"), ("fitted", "kernel"),
                                            ("partitions", "fused"), ("fitted", "fused")])
def test_graph_capture_replays_match_eager(schedule, merge):
    """Calls captured in a HIP graph: every replay, with eager work and
    synchronisations in between, equals the eager result bit for bit (the
    balanced schedule's work counters and the in-kernel merge's arrival
    counters return to zero after every replay)."""
    inp = make_inputs("single_seq", seed=2)
    d = to_device(inp)
    q, k, v = d.call(3)
    kw = dict(variant="mfma", schedule=schedule, merge=merge)
    eager = pa.decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale, **kw)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    ws = torch.zeros(pa.pa_decode_workspace_bytes(1, 16, 8, 128, d.block_tables.shape[1], 16,
                                                  pa.make_opts(**kw)) + 256,
                     dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    ws = ws[off:]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pa.decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale, out=out, workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale, out=out, workspace=ws, **kw)
    for i in range(4):
        out.zero_()
        junk = pa.decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale * 0.5, **kw)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        assert not torch.equal(junk, eager)
        assert torch.all(ws[:pa.PA_WORKSPACE_ZERO_BYTES] == 0), f"counters after replay {i}"


# ------------------------------------------------------------------ balanced schedule
def test_balanced_max_batch_ragged():
    """4096 sequences (the balanced schedule's limit) of 0..70 tokens: the
    tile prefix sums span 16 chunks of the in-LDS scan, and shares cut through
    many short sequences and empty ones."""
    rng = np.random.default_rng(11)
    lens = tuple(int(x) for x in rng.integers(0, 71, 4096))
    w = custom(batch=4096, num_q_heads=8, num_kv_heads=8, head_dim=128, page_size=16, ctx=lens)
    inp = make_inputs(w, seed=11)
    d = to_device(inp)
    ref = oracle_run(inp)
    for n in (0, 1, 255, 1024):
        y, _ = gpu_run(d, variant="mfma-bal", shares=n)
        assert_parity(y, ref, f"B=4096 shares={n}")


# ------------------------------------------------------------------ fitted partitions
@pytest.mark.parametrize("B,Hq,Hkv,D", [(65, 4, 1, 128), (200, 4, 1, 128), (100, 8, 2, 256)])
def test_fitted_many_sequences_ragged(B, Hq, Hkv, D):
    """Batches past one wave's 64 lanes (each lane holds sequences i, i + 64,
    ...): the size search and the triple numbering run over several chunks
    of lengths, with empty sequences and lengths on and off page boundaries,
    for workgroup targets from one (largest size) to more than any partitioning
    needs (smallest size)."""
    rng = np.random.default_rng(B + D)
    lens = rng.integers(0, 2001, B)
    lens[rng.choice(B, 5, replace=False)] = 0
    lens[rng.choice(B, 5, replace=False)] = 2000
    lens[rng.choice(B, 5, replace=False)] = 1
    w = custom(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=16,
               ctx=tuple(int(x) for x in lens))
    inp = make_inputs(w, seed=B, poison_unused=True)
    d = to_device(inp)
    ref = oracle_run(inp)
    for n in FIT_TARGETS + (256, 300):
        y, s = gpu_run(d, variant="mfma-fit", shares=n)
        assert s["split_calls"] == 1, s
        assert_parity(y, ref, f"B={B} D={D} target={n}")


@pytest.mark.parametrize("variant", ["mfma-fit", "mfma-fit-fused", "mfma"])
def test_trace_records(variant):
    """The timeline records (pa_trace_set) of the partitioned MFMA decode on
    the head_dim-256 workload: the output is unchanged, every workgroup that
    ran a partition stamps its phases in order, and the (sequence, query
    block, partition) triples of the records cover each group's tokens once;
    with the merge in the kernel, one workgroup per split group merges it."""
    inp = make_inputs("hd256_gqa4", seed=0)
    d = to_device(inp)
    ref = oracle_run(inp)
    buf = torch.zeros(4096 * pa.PA_TRACE_WORDS, dtype=torch.int64, device="cuda")
    pa.pa_trace_set(buf)
    try:
        y, s = gpu_run(d, variant=variant)
    finally:
        pa.pa_trace_set(None)
    assert_parity(y, ref, f"hd256_gqa4/{variant} traced")
    rec = buf.view(-1, pa.PA_TRACE_WORDS).cpu().numpy().astype(np.uint64)
    rec = rec[rec[:, 4] != 0]                            # workgroups that wrote a record
    assert len(rec) > 0
    flags = (rec[:, 7] >> np.uint64(32)).astype(np.int64)
    T = (rec[:, 7] & np.uint64(0xFFFFFFFF)).astype(np.int64)
    ran = rec[flags != 1]
    t = ran[:, :5].astype(np.int64)
    assert (t > 0).all() and (np.diff(t, axis=1) >= 0).all(), "phase stamps out of order"
    lens = inp.context_lens
    b = (ran[:, 6] & np.uint64(0xFFFF)).astype(np.int64)
    qb = ((ran[:, 6] >> np.uint64(16)) & np.uint64(0xFFFF)).astype(np.int64)
    part = (ran[:, 6] >> np.uint64(32)).astype(np.int64)
    Tr = T[flags != 1]
    assert len(set(Tr.tolist())) == 1, "one partition size per call"
    Tc = int(Tr[0])
    groups = {}
    for bi, qi, pi in zip(b.tolist(), qb.tolist(), part.tolist()):
        groups.setdefault((bi, qi), []).append(pi)
    n_qb = max(qb.tolist()) + 1
    for bi in range(len(lens)):
        need = max(1, -(-int(lens[bi]) // Tc))
        for qi in range(n_qb):
            assert sorted(groups.get((bi, qi), [])) == list(range(need)), (bi, qi, groups.get((bi, qi)))
    merged = int((flags == 2).sum())
    split_groups = sum(1 for bi in range(len(lens)) if -(-int(lens[bi]) // Tc) > 1) * n_qb
    if _MERGE.get(variant) == "fused":
        assert merged == split_groups, (merged, split_groups)
    else:
        assert merged == 0


def test_fitted_workspace_garbage_and_foreign_hints():
    """Fitted partitions keep each workgroup's last partition in the workspace
    as the next call's guess.  Any content there must give the same result:
    a workspace of random bytes, hints left by a batch of another shape, and
    reruns (hints that hit) -- all against the oracle, reruns bitwise."""
    ws_n = 0
    cases = []
    for B, lens_hi, seed in ((32, 4096, 21), (9, 3000, 22)):
        rng = np.random.default_rng(seed)
        lens = tuple(int(x) for x in rng.integers(1, lens_hi + 1, B))
        w = custom(batch=B, num_q_heads=8, num_kv_heads=2, head_dim=256, page_size=32, ctx=lens)
        inp = make_inputs(w, seed=seed)
        d = to_device(inp)
        q, k, v = d.call(0)
        opts = pa.make_opts("mfma", 0, "fitted")
        ws_n = max(ws_n, pa.pa_decode_workspace_bytes(B, 8, 2, 256, d.block_tables.shape[1], 32, opts))
        cases.append((inp, d, q, k, v))
    raw = torch.randint(0, 256, (ws_n + 256,), dtype=torch.uint8, device="cuda")
    off = (-raw.data_ptr()) % 256
    ws = raw[off:off + ws_n]
    ws[:pa.PA_WORKSPACE_ZERO_BYTES] = 0         # the counters must start at zero; the rest is garbage
    first = {}
    for rnd in range(3):
        for i, (inp, d, q, k, v) in enumerate(cases):
            out = torch.full_like(q, float("nan"))
            pa.pa_reset_stats()
            pa.decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale, out=out, variant="mfma",
                      schedule="fitted", workspace=ws)
            torch.cuda.synchronize()
            st = pa.pa_get_stats()
            assert st["last_schedule"] == pa.PA_SCHEDULE_FITTED and st["split_calls"] == 1, st
            y = bits(out)
            if rnd == 0:
                assert_parity(y, oracle_run(inp), f"fitted case {i}, workspace of random bytes")
                first[i] = y
            else:
                assert np.array_equal(y, first[i]), f"fitted case {i} round {rnd}: result depends on the hints"


def test_fitted_stale_hints():
    """Each call's hints (the previous call's size and triples) are checked
    against the current lengths and target before use.  A run of calls on one
    workspace whose lengths shrink, empty out and come back, and whose
    triple target changes, must match bit for bit a run on a fresh workspace
    (no usable hint, full search) and, for two of them, the oracle."""
    B, P = 32, 32
    rng = np.random.default_rng(31)
    base = rng.integers(1, 4097, B)
    w = custom(batch=B, num_q_heads=8, num_kv_heads=2, head_dim=256, page_size=P, ctx=tuple(int(x) for x in base))
    inp = make_inputs(w, seed=31)
    d = to_device(inp)
    q, k, v = d.call(0)
    cut = base.copy()
    cut[::3] = np.maximum(cut[::3] // 2, 1)
    empty = base.copy()
    empty[1::5] = 0
    series = [(base, 0), (base - 1, 0), (cut, 0), (empty, 0), (base, 0), (base, 64), (base, 300), (cut, 1000),
              (base, 0), (base, 0)]
    opts_n = max(pa.pa_decode_workspace_bytes(B, 8, 2, 256, d.block_tables.shape[1], P,
                                              pa.make_opts("mfma", 0, "fitted", shares=sh)) for _, sh in series)

    def workspace():
        raw = torch.zeros(opts_n + 256, dtype=torch.uint8, device="cuda")
        off = (-raw.data_ptr()) % 256
        return raw[off:off + opts_n]

    def run(lens, shares, ws):
        ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
        out = torch.full_like(q, float("nan"))
        pa.pa_reset_stats()
        pa.decode(q, k, v, d.block_tables, ctx, inp.w.scale, out=out, variant="mfma", schedule="fitted",
                  shares=shares, workspace=ws)
        torch.cuda.synchronize()
        st = pa.pa_get_stats()
        assert st["last_schedule"] == pa.PA_SCHEDULE_FITTED, st
        return bits(out)

    kept = workspace()
    for i, (lens, shares) in enumerate(series):
        y = run(lens, shares, kept)
        fresh = run(lens, shares, workspace())
        assert np.array_equal(y, fresh), f"call {i} (shares {shares}): result depends on the hints"
        if i in (1, 3):
            qh, kh, vh = inp.call(0)
            ref = oracle.attention(qh, kh, vh, inp.block_tables, np.asarray(lens, dtype=np.int32), inp.w.scale,
                                   inp.w.num_kv_heads)
            assert_parity(y, ref, f"fitted stale hints, call {i}")


@pytest.mark.parametrize("P,ctx", [(1, (9000, 5000, 100, 0)), (2, (20000, 1, 16385, 700))])
def test_balanced_multi_fill(P, ctx):
    """The balanced schedule fetches a segment's page ids 4096 tokens at a
    time: with pages of 1 and 2 tokens a fill holds 4098 and 2050 page ids,
    and segments of up to 20000 tokens cross several fills, inside a share
    and at its edges."""
    w = custom(batch=len(ctx), num_q_heads=16, num_kv_heads=8, head_dim=128, page_size=P, ctx=ctx)
    inp = make_inputs(w, seed=P + 40)
    d = to_device(inp)
    ref = oracle_run(inp)
    for n in (1, 7, 64):
        y, _ = gpu_run(d, variant="mfma-bal", shares=n)
        assert_parity(y, ref, f"balanced, page {P}, shares {n}")


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 16, 8), (256, 32, 4), (128, 64, 4)])
def test_balanced_share_sweep(D, Hq, Hkv):
    """Many share counts over a length mix with one long sequence: share
    boundaries land in every position of the (sequence, query block, tile)
    order, including the 4096-token page-id refills of a long piece."""
    w = custom(batch=5, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=16,
               ctx=(9000, 1, 300, 0, 4100))
    inp = make_inputs(w, seed=D + Hq)
    d = to_device(inp)
    ref = oracle_run(inp)
    for n in (1, 2, 5, 16, 100, 333, 1000):
        y, _ = gpu_run(d, variant="mfma-bal", shares=n)
        assert_parity(y, ref, f"D={D} Hq={Hq} Hkv={Hkv} shares={n}")


def test_balanced_workspace_reuse_and_counters():
    """One caller workspace serves many calls of every schedule and variant
    (partition counts varying between calls): the balanced schedule's work
    counters are zero after every call and balanced reruns are bitwise
    identical (units have fixed bounds, whichever workgroup takes them)."""
    inp = make_inputs("hd256_gqa4", seed=3)
    d = to_device(inp)
    q, k, v = d.call(0)
    B, Hq, D = q.shape
    NP, P, Hkv, _ = k.shape
    n = max(pa.pa_decode_workspace_bytes(B, Hq, Hkv, D, d.block_tables.shape[1], P, pa.make_opts(var, T, sch))
            for var, sch, T in (("mfma", "partitions", 0), ("mfma", "balanced", 0), ("mfma", "partitions", 256),
                                ("valu", "partitions", 256), ("mfma", "fitted", 0)))
    raw = torch.zeros(n + 256, dtype=torch.uint8, device="cuda")
    off = (-raw.data_ptr()) % 256
    ws = raw[off:off + n]
    ref = oracle_run(inp)
    first = None
    for i, (var, sch, shares, T) in enumerate([
            ("mfma", "balanced", 0, 0), ("mfma", "partitions", 0, 0), ("mfma", "balanced", 256, 0),
            ("mfma", "partitions", 0, 256), ("mfma", "balanced", 7, 0), ("valu", "partitions", 0, 256),
            ("mfma", "balanced", 256, 0), ("mfma", "partitions", 0, 0), ("mfma", "partitions", 0, 1024),
            ("mfma", "balanced", 1024, 0), ("mfma", "partitions", 0, 256), ("mfma", "balanced", 256, 0),
            ("mfma", "fitted", 0, 0), ("mfma", "fitted", 3, 0), ("mfma", "balanced", 256, 0),
            ("mfma", "fitted", 1024, 0), ("mfma", "partitions", 0, 0)]):
        out = torch.full_like(q, float("nan"))
        pa.decode(q, k, v, d.block_tables, d.context_lens, inp.w.scale, out=out, variant=var,
                  schedule=sch, shares=shares, partition_tokens=T, workspace=ws)
        torch.cuda.synchronize()
        assert torch.all(ws[:pa.PA_WORKSPACE_ZERO_BYTES] == 0), f"call {i}: counters not reset"
        y = bits(out)
        assert_parity(y, ref, f"reuse call {i} {var} {sch} {shares} T={T}")
        if sch == "balanced" and shares == 256:
            if first is None:
                first = y
            assert np.array_equal(y, first), f"call {i}: rerun differs"


# ------------------------------------------------------------------ sliding window
def poison_before_window(inp, W):
    """Copy of the inputs whose K/V rows before each sequence's window hold
    bf16 NaN: a kernel that reads them into the softmax shows it."""
    k, v = inp.k.copy(), inp.v.copy()
    P = inp.w.page_size
    for b, L in enumerate(inp.context_lens):
        for t in range(max(0, int(L) - W)):
            pg, sl = inp.block_tables[b, t // P], t % P
            k[:, pg, sl] = 0x7FC0
            v[:, pg, sl] = 0x7FC0
    return workloads.Inputs(inp.w, inp.q, k, v, inp.layout)


@pytest.mark.parametrize("variant", VARIANTS_W)
@pytest.mark.parametrize("D,Hq,Hkv,P", [(128, 16, 8, 16), (256, 8, 2, 32), (128, 64, 8, 16),
                                        (128, 16, 4, 7), (128, 16, 8, 64), (256, 8, 2, 256)])
def test_window_parity_poisoned(variant, D, Hq, Hkv, P):
    """Windows of 1 token to beyond the longest sequence, every row before a
    window set to NaN, lengths on and off tile and page boundaries."""
    w = custom(batch=7, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
               ctx=(1, 15, 16, 17, 300, 1000, 2500))
    inp0 = make_inputs(w, seed=D + Hq + P)
    for W in (1, 7, 16, 100, 1000, 4096):
        inp = poison_before_window(inp0, W)
        d = to_device(inp)
        ref = oracle_run(inp, window=W)
        for kn in knobs(variant, (0, 64)):
            y, _ = gpu_run(d, variant=variant, window=W, **kn)
            assert np.all(np.isfinite(workloads_f32(y))), f"W={W} {kn}: NaN leaked from before the window"
            assert_parity(y, ref, f"W={W} {kn}")


@pytest.mark.parametrize("variant", VARIANTS_W)
def test_window_covering_every_sequence_is_bitwise_unwindowed(variant):
    inp = make_inputs("hd256_gqa4", seed=5)
    d = to_device(inp)
    y0, _ = gpu_run(d, variant=variant)
    Lmax = int(inp.context_lens.max())
    for W in (Lmax, Lmax + 1, 1 << 30):
        y1, _ = gpu_run(d, variant=variant, window=W)
        assert np.array_equal(y0, y1), f"W={W}"


@pytest.mark.parametrize("variant", ["mfma", "mfma-bal"])
def test_window_long_context_all_rows(variant, long_ctx):
    """Full-size long-context workload with a 4096-token window: every
    (sequence, head) row against the oracle with the same window."""
    W = 4096
    y, s = gpu_run(long_ctx.d, variant=variant, window=W)
    assert_parity(y, long_ctx.ref(W), f"long ctx W={W} all rows {variant}")


# ------------------------------------------------------------------ KV-cache append
@pytest.mark.parametrize("D,Hkv,P", [(128, 8, 16), (256, 2, 32), (128, 4, 7), (64, 8, 1), (128, 8, 256)])
def test_append_matches_oracle_bitwise(D, Hkv, P):
    """The whole K and V pools after the append equal the oracle's, bit for
    bit: the newest token's rows land in their slots and nothing else moves.
    k_new is a strided view (padded head stride)."""
    lens = (0, 1, P, P + 1, 3 * P + 2, 100)
    w = custom(batch=len(lens), num_q_heads=2 * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=P,
               ctx=lens)
    inp = make_inputs(w, seed=D + P)
    rng = np.random.default_rng(D * P)
    B = len(lens)
    k_new = workloads.round_bf16(rng.standard_normal((B, Hkv, D)).astype(np.float32))
    v_new = workloads.round_bf16(rng.standard_normal((B, Hkv, D)).astype(np.float32))
    k_ref, v_ref = oracle.cache_append(inp.k[0], inp.v[0], inp.block_tables, inp.context_lens,
                                       k_new, v_new)
    d = to_device(inp)
    k, v = d.k[0].clone(), d.v[0].clone()
    dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    kn_pad = torch.zeros((B, Hkv, D + 64), dtype=torch.bfloat16, device="cuda")
    kn_pad[..., :D] = dev(k_new)
    pa.pa_reset_stats()
    pa.cache_append(kn_pad[..., :D], dev(v_new), k, v, d.block_tables, d.context_lens)
    torch.cuda.synchronize()
    assert pa.pa_get_stats()["append_launches"] == 1
    assert np.array_equal(bits(k).reshape(k_ref.shape), k_ref)
    assert np.array_equal(bits(v).reshape(v_ref.shape), v_ref)


@pytest.mark.parametrize("variant", VARIANTS)
def test_append_then_decode(variant):
    """A decode step: append the newest token, then attend; equals the
    oracle's append followed by the oracle's attention."""
    w = custom(batch=5, num_q_heads=16, num_kv_heads=8, head_dim=128, page_size=16,
               ctx=(1, 16, 17, 300, 1000))
    inp = make_inputs(w, seed=71)
    rng = np.random.default_rng(71)
    k_new = workloads.round_bf16(rng.standard_normal((5, 8, 128)).astype(np.float32))
    v_new = workloads.round_bf16(rng.standard_normal((5, 8, 128)).astype(np.float32))
    k_ref, v_ref = oracle.cache_append(inp.k[0], inp.v[0], inp.block_tables, inp.context_lens,
                                       k_new, v_new)
    ref = oracle.attention(inp.q[0], k_ref, v_ref, inp.block_tables, inp.context_lens,
                           inp.w.scale, inp.w.num_kv_heads)
    d = to_device(inp)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    pa.cache_append(dev(k_new), dev(v_new), d.k[0], d.v[0], d.block_tables, d.context_lens)
    y, _ = gpu_run(d, variant=variant)
    assert_parity(y, ref, f"append + decode {variant}")


def test_append_skips_sequences_it_cannot_place():
    """A newest token whose block-table entry is out of the pool, or whose
    length exceeds the table, writes nothing; the other sequences are written."""
    w = custom(batch=3, num_q_heads=8, num_kv_heads=4, head_dim=128, page_size=16, ctx=(5, 20, 9))
    inp = make_inputs(w, seed=72)
    d = to_device(inp)
    bt = d.block_tables.clone()
    bt[1, 1] = -1                                  # sequence 1's newest page: not a page
    ctx = d.context_lens.clone()
    ctx[2] = 16 * bt.shape[1] + 1                  # sequence 2: past its table
    k, v = d.k[0].clone(), d.v[0].clone()
    k0, v0 = bits(k), bits(v)
    kn = torch.ones((3, 4, 128), dtype=torch.bfloat16, device="cuda")
    pa.cache_append(kn, kn, k, v, bt, ctx)
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.cache_append(inp.k[0], inp.v[0], inp.block_tables[:1], inp.context_lens[:1],
                                       bits(kn)[:1].reshape(1, 4, 128), bits(kn)[:1].reshape(1, 4, 128))
    assert np.array_equal(bits(k).reshape(k_ref.shape), k_ref)
    assert np.array_equal(bits(v).reshape(v_ref.shape), v_ref)
    assert not np.array_equal(bits(k), k0)


# ------------------------------------------------------------------ element types, head_dim 512
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
# (Q, K/V, out): the same type throughout, and fp32 activations over a 16-bit cache
DTYPE_COMBOS = [("f16", "f16", "f16"), ("f32", "f32", "f32"), ("f32", "bf16", "f32"),
                ("f32", "f16", "f32"), ("bf16", "f16", "bf16"), ("f16", "bf16", "f32")]


# fp32 caches run on the vector-ALU kernel only: the MFMA variants answer
# ENOTSUP for them (test_fp32_cache_on_mfma_is_enotsup), so those
# combinations are not parametrized here.
DTYPE_CASES = [(v, qt, kt, ot) for v in VARIANTS for (qt, kt, ot) in DTYPE_COMBOS if kt != "f32" or v == "valu"]


@pytest.mark.parametrize("variant,qt,kt,ot", DTYPE_CASES)
@pytest.mark.parametrize("D", [128, 256])
def test_dtype_parity_poisoned(variant, qt, kt, ot, D):
    w = custom(batch=5, num_q_heads=16, num_kv_heads=4, head_dim=D, page_size=16,
               ctx=(1, 17, 300, 1000, 2500), pool_pages=300)
    inp = make_inputs(w, seed=D + len(qt + kt), poison_unused=True, dtype=kt, q_dtype=qt)
    d = to_device(inp)
    ref = oracle_run(inp)
    for kn in knobs(variant, (0, 64)):
        y, _ = gpu_run(d, variant=variant, out_dtype=TORCH_DT[ot], **kn)
        assert np.all(np.isfinite(y.astype(np.float64) if ot != "bf16" else workloads_f32(y)))
        assert_parity(y, ref, f"q {qt} kv {kt} out {ot} D={D} {kn}")
    for W in ((7, 500) if variant in VARIANTS_W else ()):
        y, _ = gpu_run(d, variant=variant, out_dtype=TORCH_DT[ot], window=W)
        assert_parity(y, oracle_run(inp, window=W), f"q {qt} kv {kt} out {ot} D={D} W={W}")


@pytest.mark.parametrize("variant", ["mfma", "mfma-bal", "mfma-fit"])
@pytest.mark.parametrize("D", [128, 256])
def test_fp32_cache_on_mfma_is_enotsup(variant, D):
    """The fp32-cache combinations the MFMA variants do not take are refused
    with PA_ENOTSUP before any launch, and leave the output untouched."""
    w = custom(batch=5, num_q_heads=16, num_kv_heads=4, head_dim=D, page_size=16,
               ctx=(1, 17, 300, 1000, 2500), pool_pages=300)
    d = to_device(make_inputs(w, seed=1, dtype="f32"))
    q, k, v = d.call(0)
    kernel, schedule = _MODE[variant]
    out = torch.full(q.shape, 7.0, dtype=q.dtype, device=q.device)
    pa.pa_reset_stats()
    with pytest.raises(pa.PaError) as e:
        pa.decode(q, k, v, d.block_tables, d.context_lens, out=out, variant=kernel, schedule=schedule)
    assert e.value.code == pa.PA_ENOTSUP
    torch.cuda.synchronize()
    assert pa.pa_get_stats()["calls"] == 0
    assert bool(torch.all(out == 7.0))


@pytest.mark.parametrize("kt", ["bf16", "f16"])
@pytest.mark.parametrize("P", [8, 24])
def test_head_dim_512_wide_groups_small_pages(kt, P):
    """head_dim 512 with 16 query heads per KV head (the row = token layout)
    on pages that are not a power of two of at least 16 tokens (per-row page
    lookup): the MFMA kernel instantiation whose registers run out (it keeps
    some in scratch), split and unsplit, against the oracle."""
    w = custom(batch=3, num_q_heads=16, num_kv_heads=1, head_dim=512, page_size=P, ctx=(1, 77, 900))
    inp = make_inputs(w, seed=P + 512, poison_unused=True, dtype=kt)
    d = to_device(inp)
    ref = oracle_run(inp)
    for T in (0, 64, 256):
        y, _ = gpu_run(d, variant="mfma", partition_tokens=T)
        assert_parity(y, ref, f"D=512 qg=16 P={P} kv {kt} T={T}")


@pytest.mark.parametrize("kt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (16, 4), (16, 2)])
def test_head_dim_512(kt, Hq, Hkv):
    """head_dim 512: the vector-ALU kernel (two query heads per workgroup at
    most) and, for 16-bit caches, the MFMA kernel (all query heads of a KV
    head; 32 KB tiles): split and unsplit, with and without a window."""
    w = custom(batch=4, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=512, page_size=16,
               ctx=(1, 33, 700, 1500))
    inp = make_inputs(w, seed=Hq * Hkv, poison_unused=True, dtype=kt)
    d = to_device(inp)
    ref = oracle_run(inp)
    ref_w = oracle_run(inp, window=100)
    variants = ["valu"] + (["mfma"] if kt != "f32" else [])
    for var in variants:
        for T in (0, 64, 4096):
            y, s = gpu_run(d, variant=var, partition_tokens=T)
            assert_parity(y, ref, f"D=512 {var} kv {kt} Hq={Hq} Hkv={Hkv} T={T}")
        y, _ = gpu_run(d, variant=var, window=100)
        assert_parity(y, ref_w, f"D=512 {var} kv {kt} W=100")
    if kt != "f32":
        for n in FIT_TARGETS:
            y, _ = gpu_run(d, variant="mfma-fit", shares=n)
            assert_parity(y, ref, f"D=512 fitted kv {kt} Hq={Hq} Hkv={Hkv} target={n}")
    # the automatic choice: MFMA for 16-bit caches, vector ALU for fp32
    pa.pa_reset_stats()
    q, k, v = d.call(0)
    pa.decode(q, k, v, d.block_tables, d.context_lens)
    torch.cuda.synchronize()
    st = pa.pa_get_stats()
    assert st["valu_launches" if kt == "f32" else "mfma_launches"] == 1, st


@pytest.mark.parametrize("kt", ["f16", "f32"])
def test_append_typed_caches_bitwise(kt):
    w = custom(batch=4, num_q_heads=8, num_kv_heads=4, head_dim=128, page_size=16, ctx=(1, 16, 17, 90))
    inp = make_inputs(w, seed=9, dtype=kt)
    rng = np.random.default_rng(9)
    dt = workloads.STORAGE[kt]
    k_new = rng.standard_normal((4, 4, 128)).astype(dt)
    v_new = rng.standard_normal((4, 4, 128)).astype(dt)
    k_ref, v_ref = oracle.cache_append(inp.k[0], inp.v[0], inp.block_tables, inp.context_lens, k_new, v_new)
    d = to_device(inp)
    k, v = d.k[0].clone(), d.v[0].clone()
    pa.cache_append(torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda(), k, v,
                    d.block_tables, d.context_lens)
    torch.cuda.synchronize()
    assert np.array_equal(k.cpu().numpy().view(np.uint8), k_ref.view(np.uint8))
    assert np.array_equal(v.cpu().numpy().view(np.uint8), v_ref.view(np.uint8))


# ------------------------------------------------------------------ several queries per sequence
def queries_case(lens, chunks, Hq, Hkv, D, P, dtype="bf16", q_dtype=None, seed=0):
    w = custom(batch=len(lens), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P, ctx=lens)
    inp = make_inputs(w, seed=seed, poison_unused=True, dtype=dtype)
    rng = np.random.default_rng(seed + 1)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = workloads.encode(rng.standard_normal((int(qs[-1]), Hq, D)).astype(np.float32), q_dtype or dtype)
    return inp, q, qs


def to_torch(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def prefill_run(d, q, qs, out_dtype=None, scale=None, **kw):
    qd = to_torch(q)
    out = torch.full(qd.shape, float("nan"), dtype=out_dtype or qd.dtype, device="cuda")
    pa.pa_reset_stats()
    pa.prefill(qd, d.k[0], d.v[0], d.block_tables, d.context_lens, torch.from_numpy(qs).cuda(),
               d.w.scale if scale is None else scale, out=out, **kw)
    torch.cuda.synchronize()
    s = pa.pa_get_stats()
    assert s["prefill_launches"] == 1, s
    if kw.get("schedule") == "staged":
        assert s["last_schedule"] == pa.PA_SCHEDULE_STAGED and s["merge_launches"] == 0, s
    elif kw.get("schedule") == "partitions":
        assert s["last_schedule"] == pa.PA_SCHEDULE_PARTITIONS, s
    return host_out(out), s


# (schedule, partition_tokens): the per-block kernel unsplit / split / one
# partition, and eight query blocks per workgroup sharing K/V stages in LDS
PREFILL_SCHEDULES = [("partitions", 0), ("partitions", 64), ("partitions", 1 << 20), ("staged", 0)]


def oracle_queries(inp, q, qs, window=0, scale=None):
    return oracle.attention_queries(q, inp.k[0], inp.v[0], inp.block_tables, inp.context_lens, qs,
                                    inp.w.scale if scale is None else scale, inp.w.num_kv_heads, window=window)


@pytest.mark.parametrize("D,Hq,Hkv,P", [(128, 16, 8, 16), (128, 32, 2, 16), (256, 8, 2, 32),
                                        (128, 16, 16, 16), (128, 16, 1, 7), (256, 16, 4, 1),
                                        (128, 16, 8, 64), (128, 16, 8, 256), (256, 8, 2, 128),
                                        (128, 12, 3, 16), (256, 40, 5, 32)])
def test_prefill_parity(D, Hq, Hkv, P):
    """A batch mixing whole-prompt prefill, chunked prefill and decode steps:
    every query row against the causal oracle, split and unsplit, with and
    without a window; unused pool slots are NaN."""
    lens = (1, 17, 40, 300, 1000, 2500)
    chunks = (1, 17, 1, 100, 64, 33)
    inp, q, qs = queries_case(lens, chunks, Hq, Hkv, D, P, seed=D + Hq + P)
    d = to_device(inp)
    for W in (0, 7, 200):
        ref = oracle_queries(inp, q, qs, window=W)
        for sched, T in PREFILL_SCHEDULES:
            y, s = prefill_run(d, q, qs, window=W, partition_tokens=T, schedule=sched)
            assert_parity(y, ref, f"prefill D={D} Hq={Hq} Hkv={Hkv} P={P} W={W} {sched} T={T} "
                                  f"(x{s['last_num_partitions']})")


@pytest.mark.parametrize("D", [128, 256])
def test_prefill_scale_sweep(D):
    """Several queries per sequence over logit scales from nearly flat to
    nearly one-hot, and a negative one: the staged kernel's lazy rescale and
    weight split, and the per-block kernel's, split and unsplit."""
    Hq, Hkv = (16, 8) if D == 128 else (8, 2)
    inp, q, qs = queries_case((1, 17, 300, 1000, 2500), (1, 17, 64, 100, 200), Hq, Hkv, D, 16, seed=D + 5)
    d = to_device(inp)
    for f in (1e-3, 4.0, 16.0, 64.0, -2.0):
        sc = float(np.float32(inp.w.scale * f))
        ref = oracle_queries(inp, q, qs, scale=sc)
        for sched, T in PREFILL_SCHEDULES:
            y, _ = prefill_run(d, q, qs, scale=sc, partition_tokens=T, schedule=sched)
            assert_parity(y, ref, f"prefill D={D} scale x{f} {sched} T={T}")


@pytest.mark.parametrize("Hq,Hkv,P,kt", [(8, 2, 16, "bf16"), (16, 16, 32, "bf16"), (16, 1, 7, "bf16"),
                                         (8, 2, 16, "f16")])
def test_prefill_head_dim_512(Hq, Hkv, P, kt):
    """Several queries per sequence at head_dim 512 (per-block kernel, split
    and unsplit, with and without a window; unused slots NaN) against the
    causal oracle; the staged schedule answers ENOTSUP there."""
    lens = (1, 17, 40, 300, 1000)
    chunks = (1, 17, 1, 100, 64)
    inp, q, qs = queries_case(lens, chunks, Hq, Hkv, 512, P, dtype=kt, seed=512 + Hq + P)
    d = to_device(inp)
    for W in (0, 7, 200):
        ref = oracle_queries(inp, q, qs, window=W)
        for sched, T in (("partitions", 0), ("partitions", 64), ("auto", 0)):
            y, s = prefill_run(d, q, qs, window=W, partition_tokens=T, schedule=sched)
            assert s["last_schedule"] == pa.PA_SCHEDULE_PARTITIONS, s
            assert_parity(y, ref, f"prefill d512 Hq={Hq} Hkv={Hkv} P={P} {kt} W={W} {sched} T={T} "
                                  f"(x{s['last_num_partitions']})")
    with pytest.raises(pa.PaError) as e:
        prefill_run(d, q, qs, schedule="staged")
    assert e.value.code == pa.PA_ENOTSUP


@pytest.mark.parametrize("kt,qt,ot", [("f16", "f16", "f16"), ("bf16", "f32", "f32"), ("f16", "bf16", "f32")])
def test_prefill_element_types(kt, qt, ot):
    inp, q, qs = queries_case((64, 900, 33), (64, 40, 1), 16, 4, 128, 16, dtype=kt, q_dtype=qt, seed=5)
    d = to_device(inp)
    ref = oracle_queries(inp, q, qs)
    for sched in ("partitions", "staged"):
        y, _ = prefill_run(d, q, qs, out_dtype=TORCH_DT[ot], schedule=sched)
        assert_parity(y, ref, f"prefill {sched} q {qt} kv {kt} out {ot}")


def test_prefill_one_query_per_sequence_matches_decode():
    """n_b = 1 everywhere is decode: the several-query kernel and the decode
    kernels agree with the oracle and with each other."""
    inp = make_inputs("batch16", seed=3)
    q = inp.q[0]
    qs = np.arange(inp.w.batch + 1, dtype=np.int32)
    d = to_device(inp)
    y, _ = prefill_run(d, q, qs)
    ref = oracle_run(inp)
    assert_parity(y, ref, "prefill as decode")
    yd, _ = gpu_run(d, variant="mfma")
    r = compare(y, yd)
    assert r.nmse < 1e-4, r


def test_prefill_long_chunk_spare_slots_and_empty_sequences():
    """A long chunk (many query blocks), empty sequences (no rows), and a
    sequence with no tokens at all."""
    lens = (0, 700, 5, 2048)
    chunks = (0, 700, 0, 512)
    inp, q, qs = queries_case(lens, chunks, 8, 2, 128, 16, seed=11)
    d = to_device(inp)
    ref = oracle_queries(inp, q, qs)
    for sched in ("auto", "partitions", "staged"):
        y, _ = prefill_run(d, q, qs, schedule=sched)
        assert_parity(y, ref, f"long chunks {sched}")


def test_prefill_full_size_all_rows():
    """The chunked-prefill workload the benchmark times (8 sequences of 4096
    tokens whose last 512 are queried, Hq 32 / Hkv 8, d 128, page 16) in its
    launch configuration (automatic: staged) and on the per-block kernel:
    every query row and head against the causal oracle (about 260 GFLOP of
    fp64, some 20 s on the host cores)."""
    B, ctx, chunk, Hq, Hkv, D, P = 8, 4096, 512, 32, 8, 128, 16
    w = custom(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P, ctx=(ctx,) * B)
    inp = make_inputs(w, seed=0)
    rng = np.random.default_rng(7)
    qs = np.arange(0, B * chunk + 1, chunk, dtype=np.int32)
    q = workloads.encode(rng.standard_normal((B * chunk, Hq, D)).astype(np.float32), "bf16")
    d = to_device(inp)
    y, s = prefill_run(d, q, qs)
    assert s["last_schedule"] == pa.PA_SCHEDULE_STAGED, s
    y2, _ = prefill_run(d, q, qs, schedule="partitions")
    ref = oracle_queries(inp, q, qs)
    assert_parity(y, ref, "full-size prefill, all rows, staged")
    assert_parity(y2, ref, "full-size prefill, all rows, per-block kernel")


@pytest.mark.parametrize("schedule", ["partitions", "staged"])
def test_prefill_more_queries_than_tokens(schedule):
    """A broken precondition (n_b > L_b) is handled safely: rows at negative
    positions give zeros, the others attend to their [0, pos] as a decode
    query over pos + 1 tokens would (the oracle refuses such inputs, so
    those rows are checked through that identity)."""
    lens, chunks = (40, 3), (4, 8)
    inp, q, qs = queries_case(lens, chunks, 16, 4, 128, 16, seed=23)
    d = to_device(inp)
    y, _ = prefill_run(d, q, qs, schedule=schedule)
    yf = bf16_bits_to_f64(y) if y.dtype == np.uint16 else y.astype(np.float64)
    assert np.all(yf[4:9] == 0), "rows at negative positions must be zero"
    rows = np.array([0, 1, 2, 3, 9, 10, 11])
    b_of = np.array([0, 0, 0, 0, 1, 1, 1])
    pos = np.array([36, 37, 38, 39, 0, 1, 2])
    ref = oracle.attention(np.ascontiguousarray(q[rows]), inp.k[0], inp.v[0],
                           np.ascontiguousarray(inp.block_tables[b_of]), (pos + 1).astype(np.int32),
                           inp.w.scale, inp.w.num_kv_heads)
    assert_parity(y[rows], ref, f"n_b > L_b, {schedule}")


@pytest.mark.parametrize("schedule", ["partitions", "staged"])
def test_prefill_graph_replays_match_eager(schedule):
    """Several-query calls captured in a HIP graph: every replay, with eager
    work and synchronisations in between, equals the eager result bit for
    bit (split partitions included: the workspace holds partials only)."""
    inp, q, qs = queries_case((300, 1000, 2500), (100, 64, 33), 16, 4, 128, 16, seed=21)
    d = to_device(inp)
    qd, qsd = to_torch(q), torch.from_numpy(qs).cuda()
    kw = dict(schedule=schedule, partition_tokens=64 if schedule == "partitions" else 0)
    eager = pa.prefill(qd, d.k[0], d.v[0], d.block_tables, d.context_lens, qsd, d.w.scale, **kw)
    torch.cuda.synchronize()
    R, Hq, D = qd.shape
    n = pa.pa_prefill_workspace_bytes(R, 3, Hq, 4, D, d.block_tables.shape[1], 16, pa.make_opts(**kw))
    ws = torch.zeros(n + 256, dtype=torch.uint8, device="cuda")
    ws = ws[(-ws.data_ptr()) % 256:][:max(n, 1)]
    out = torch.empty_like(qd)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pa.prefill(qd, d.k[0], d.v[0], d.block_tables, d.context_lens, qsd, d.w.scale, out=out, workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.prefill(qd, d.k[0], d.v[0], d.block_tables, d.context_lens, qsd, d.w.scale, out=out, workspace=ws, **kw)
    for i in range(4):
        out.zero_()
        junk = pa.prefill(qd, d.k[0], d.v[0], d.block_tables, d.context_lens, qsd, d.w.scale * 0.5, **kw)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        del junk
    assert_parity(host_out(out), oracle_queries(inp, q, qs), f"graph {schedule}")


def test_prefill_speculative_decode_full_size_all_rows():
    """The speculative-decode workload the benchmark times (64 sequences of
    8192 cached tokens, the last 4 queried, Hq 64 / Hkv 8, d 128, page 16;
    2.1 GB of K/V, so 64-bit offsets) in its launch configuration
    (automatic: staged, 6 of 8 waves per workgroup without a query) and on
    the per-block kernel: every query row and head against the causal
    oracle."""
    B, ctx, nq, Hq, Hkv, D, P = 64, 8192, 4, 64, 8, 128, 16
    w = custom(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P, ctx=(ctx,) * B)
    d = workloads.device_inputs(w, seed=2)
    rng = np.random.default_rng(9)
    qs = np.arange(0, B * nq + 1, nq, dtype=np.int32)
    q = workloads.encode(rng.standard_normal((B * nq, Hq, D)).astype(np.float32), "bf16")
    y, s = prefill_run(d, q, qs)
    assert s["last_schedule"] == pa.PA_SCHEDULE_STAGED, s
    y2, _ = prefill_run(d, q, qs, schedule="partitions")
    host = workloads.host_copy(d)
    ref = oracle_queries(host, q, qs)
    assert_parity(y, ref, "speculative decode, all rows, staged")
    assert_parity(y2, ref, "speculative decode, all rows, per-block kernel")
    del d, host
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ in-kernel merge
@pytest.mark.parametrize("name", ["tiny", "single_seq", "batch16", "hd256_gqa4", "hd512_gqa4"])
def test_fused_merge_bitwise_equals_merge_kernel(name):
    """Partitions merged inside the decode kernel (last arriver per group)
    and by the separate merge kernel add the same partials in the same order:
    bit-identical outputs, on fixed and fitted partitions, over one
    workspace whose counters are zero after every call."""
    inp = make_inputs(name, seed=7)
    d = to_device(inp)
    q, k, v = d.call(0)
    B, Hq, D = q.shape
    NP, P, Hkv, _ = k.shape
    n = max(pa.pa_decode_workspace_bytes(B, Hq, Hkv, D, d.block_tables.shape[1], P, pa.make_opts("mfma", T, sch))
            for sch, T in (("partitions", 64), ("partitions", 0), ("fitted", 0)))
    raw = torch.zeros(n + 256, dtype=torch.uint8, device="cuda")
    ws = raw[(-raw.data_ptr()) % 256:][:n]
    ref = oracle_run(inp)
    for kn in (dict(partition_tokens=64), dict(partition_tokens=128), dict(), dict(shares=7), dict(shares=0),
               dict(shares=300)):
        fit = "shares" in kn
        y_k, s_k = gpu_run(d, variant="mfma-fit" if fit else "mfma", workspace=ws, **kn)
        y_f, s_f = gpu_run(d, variant="mfma-fit-fused" if fit else "mfma-fused", workspace=ws, **kn)
        assert torch.all(ws[:pa.PA_WORKSPACE_ZERO_BYTES] == 0), f"{name} {kn}: counters not reset"
        assert np.array_equal(y_f, y_k), f"{name} {kn}: in-kernel merge differs from the merge kernel"
        assert_parity(y_f, ref, f"{name} fused {kn} (split {s_f['split_calls']})")


def test_fused_merge_empty_sequences_fitted():
    """Fitted partitions merged in the kernel: sequences with no tokens have
    no partition, so their zero rows come from the first workgroup."""
    lens = (0, 700, 0, 5, 2048, 0, 1)
    w = custom(batch=len(lens), num_q_heads=8, num_kv_heads=2, head_dim=256, page_size=32, ctx=lens)
    inp = make_inputs(w, seed=41, poison_unused=True)
    d = to_device(inp)
    ref = oracle_run(inp)
    for n in (0, 1, 5, 64):
        y, s = gpu_run(d, variant="mfma-fit-fused", shares=n)
        assert s["split_calls"] == 1, s
        assert_parity(y, ref, f"fitted fused, empty sequences, target {n}")


# ------------------------------------------------------------------ numerics table
# The pages' kernel-numerics table (page 3, PR "head_dim-128 arm for the
# warp-split-KV decode kernel", EVIDENCE): context lengths straddling the
# 32-token page, 2048 elements each (one sequence, 16 query heads x 128
# dims); here against the correctly rounded oracle rather than another
# kernel, for every kernel and schedule, plus the five workloads.
NUMERICS_CTX = (1, 31, 32, 33, 64, 100, 685, 1000)
NUMERICS_VARIANTS = ("auto",) + tuple(VARIANTS)


def run_any(d, variant, call=0):
    """gpu_run for a named variant, or the automatic choice ("auto"), which
    is what the benchmark times; returns (output, schedule name)."""
    if variant != "auto":
        y, s = gpu_run(d, call=call, variant=variant)
    else:
        q, k, v = d.call(call)
        out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=q.device)
        pa.pa_reset_stats()
        pa.decode(q, k, v, d.block_tables, d.context_lens, d.w.scale, out=out)
        torch.cuda.synchronize()
        s = pa.pa_get_stats()
        y = host_out(out)
    kern = {1: "valu", 2: "mfma"}[s["last_variant"]]
    sched = {1: "partitions", 2: "balanced", 4: "fitted"}[s["last_schedule"]]
    return y, f"{kern}/{sched}" + (f" T={s['last_partition_tokens']}" if s["last_partition_tokens"] else "")


def test_numerics_table(long_ctx):
    rows = []

    def add(case, variant, y, how, ref):
        r = compare(y, ref)
        rows.append((case, variant, how, r))
        print(f"[numerics] {case} {variant} ({how}): {r}", flush=True)
        assert r.ok(), f"{case} {variant}: {r}"

    for L in NUMERICS_CTX:
        w = custom(batch=1, num_q_heads=16, num_kv_heads=8, head_dim=128, page_size=32, ctx=(L,))
        inp = make_inputs(w, seed=L)
        d = to_device(inp)
        ref = oracle_run(inp)
        for variant in NUMERICS_VARIANTS:
            y, how = run_any(d, variant)
            add(f"ctx {L}", variant, y, how, ref)
    for name in ("tiny", "single_seq", "batch16", "hd256_gqa4"):
        inp = make_inputs(name, seed=0)
        d = to_device(inp)
        ref = oracle_run(inp)
        for variant in NUMERICS_VARIANTS:
            y, how = run_any(d, variant)
            add(name, variant, y, how, ref)
    for variant in NUMERICS_VARIANTS:
        y, how = run_any(long_ctx.d, variant)
        add("long_ctx_gqa8", variant, y, how, long_ctx.ref())
    text = ["| case | variant | kernel / schedule | max_abs | max_rel | max ULPs | bitwise % | NMSE |",
            "|---|---|---|---|---|---|---|---|"]
    for case, variant, how, r in rows:
        text.append(f"| {case} | {variant} | {how} | {r.max_abs:.3e} | {r.max_rel:.3e} | {r.max_ulps:.3f} | "
                    f"{r.bitwise:.4f} | {r.nmse:.2e} |")
    out = os.environ.get("PA_NUMERICS_OUT")
    if out:
        with open(out, "w") as f:
            f.write("\n".join(text) + "\n")
    print("\n".join(text), flush=True)
