"""pa_decode_noalloc: the decode entry point that allocates nothing (its
split-KV partials go to a static per-device scratch array), checked through
the C ABI against pa_decode_ex with a caller workspace and against the
oracle: calls in a row that shrink (the scratch keeps the previous call's
contents), every schedule that uses the scratch, graph replays, and the
size limit."""
import numpy as np
import pytest
import torch

import oracle
import paged_attention_decode_04_amd as pa
from oracle.compare import compare
from workloads import custom, make_inputs, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _dev(gpu):
    yield


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_both(d, **kn):
    """The same call through pa_decode_ex (own zeroed workspace) and
    pa_decode_noalloc; returns both outputs (bf16 bits) and the schedule."""
    q, k, v = d.call(0)
    B, Hq, D = q.shape
    NP, P, Hkv, _ = k.shape
    opts = pa.make_opts(**kn)
    n = pa.pa_decode_workspace_bytes(B, Hq, Hkv, D, d.block_tables.shape[1], P, opts)
    raw = torch.zeros(n + 256, dtype=torch.uint8, device="cuda")
    ws = raw[(-raw.data_ptr()) % 256:][:max(n, 1)]
    out_ex = torch.full_like(q, float("nan"))
    out_na = torch.full_like(q, float("nan"))
    pa.pa_decode_ex(q, k, v, d.block_tables, d.context_lens, d.w.scale, Hq, Hkv, D, P, out_ex, None, opts,
                    ws if n else None)
    pa.pa_reset_stats()
    pa.pa_decode_noalloc(q, k, v, d.block_tables, d.context_lens, d.w.scale, Hq, Hkv, D, P, out_na, None, opts)
    torch.cuda.synchronize()
    st = pa.pa_get_stats()
    assert st["calls"] == 1, st
    return bits(out_ex), bits(out_na), st


def oracle_run(inp):
    q, k, v = inp.call(0)
    return oracle.attention(q, k, v, inp.block_tables, inp.context_lens, inp.w.scale, inp.w.num_kv_heads)


CASES = [
    # (workload, knobs, schedule expected) -- each call smaller than the one before
    ("hd256_gqa4", dict(), pa.PA_SCHEDULE_FITTED),
    ("hd256_gqa4", dict(merge="fused"), pa.PA_SCHEDULE_FITTED),
    ("batch16", dict(schedule="balanced"), pa.PA_SCHEDULE_BALANCED),
    ("batch16", dict(merge="fused"), pa.PA_SCHEDULE_PARTITIONS),
    ("batch16", dict(), pa.PA_SCHEDULE_PARTITIONS),
    ("tiny", dict(partition_tokens=64), pa.PA_SCHEDULE_PARTITIONS),
]


def test_noalloc_matches_decode_ex_calls_in_a_row():
    for name, kn, sched in CASES:
        inp = make_inputs(name, seed=0)
        d = to_device(inp)
        y_ex, y_na, st = run_both(d, **kn)
        assert st["last_schedule"] == sched and st["split_calls"] == 1, (name, kn, st)
        r = compare(y_na, oracle_run(inp))
        print(f"[noalloc] {name} {kn}: {r}", flush=True)
        assert r.ok(), f"{name} {kn}: {r}"
        assert np.array_equal(y_na, y_ex), f"{name} {kn}: pa_decode_noalloc differs from pa_decode_ex"


def test_noalloc_graph_replays_match_eager():
    """Captured after a first eager call: every replay equals the eager
    result bit for bit, with other eager calls on the scratch in between
    (the balanced schedule's counters return to zero each time)."""
    inp = make_inputs("batch16", seed=4)
    d = to_device(inp)
    q, k, v = d.call(0)
    B, Hq, D = q.shape
    NP, P, Hkv, _ = k.shape
    opts = pa.make_opts(schedule="balanced")
    eager = torch.empty_like(q)
    pa.pa_decode_noalloc(q, k, v, d.block_tables, d.context_lens, d.w.scale, Hq, Hkv, D, P, eager, None, opts)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.pa_decode_noalloc(q, k, v, d.block_tables, d.context_lens, d.w.scale, Hq, Hkv, D, P, out, None, opts)
    other = make_inputs("tiny", seed=1)
    od = to_device(other)
    oq, ok_, ov = od.call(0)
    for i in range(4):
        out.zero_()
        junk = torch.empty_like(oq)
        pa.pa_decode_noalloc(oq, ok_, ov, od.block_tables, od.context_lens, od.w.scale, 16, 8, 128, 32, junk,
                             None, pa.make_opts(partition_tokens=64))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
    r = compare(bits(out), oracle_run(inp))
    assert r.ok(), r


def test_noalloc_rejects_calls_beyond_its_scratch():
    """A plan needing more than the static scratch is refused with
    PA_ENOMEM before any launch; the output is untouched."""
    B, Hq, Hkv, D, P, maxblk = 64, 64, 8, 128, 16, 2048
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(4, P, Hkv, D, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(B, maxblk, dtype=torch.int32, device="cuda")
    ctx = torch.ones(B, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 3.0)
    opts = pa.make_opts("valu", 64)
    need = pa.pa_decode_workspace_bytes(B, Hq, Hkv, D, maxblk, P, opts)
    assert need > pa.PA_NOALLOC_SCRATCH_BYTES
    pa.pa_reset_stats()
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode_noalloc(q, k, k, bt, ctx, 0.1, Hq, Hkv, D, P, out, None, opts)
    assert e.value.code == pa.PA_ENOMEM
    assert "scratch" in pa.last_error()
    torch.cuda.synchronize()
    assert pa.pa_get_stats()["calls"] == 0
    assert bool(torch.all(out == 3.0))
