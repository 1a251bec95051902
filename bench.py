#!/usr/bin/env python3
"""Benchmark of decode paged attention on one MI355X.

Metric: paged-attention decode microseconds per call and the achieved KV-read
bandwidth, i.e. algorithmic KV bytes (sum_b L_b * Hkv * D * 2 tensors * 2 B)
divided by the time per call, also as a fraction of the MI355X HBM3E peak
(8 TB/s).  A step is one decode call over the whole batch (decode kernel plus,
when the context is split, the log-sum-exp merge kernel), with every input
already resident in HBM.

Default workload: the long-context, high-GQA batch (64 sequences, ctx
U[8192, 32768], Hq 64 / Hkv 8, head_dim 128, page 16; about 5.4 GB of KV per
call).  The same JSON line also carries every other workload's time per call
(``per_config``), the bandwidth roofline of the dominant kernel and the CPU
oracle timed on the host cores as a reported baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix-core peak
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "paged-attn decode µs/call + achieved KV-read GB/s (% of MI355X HBM peak)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# The sources compiled into the matrix-core decode kernels (the kernels whose
# HBM traffic the profiles record); their launch geometry is compared apart.
DECODE_KERNEL_SOURCES = ["pa_mfma.hip", "pa_mfma_core.h", "pa_device.h", "pa_launch.h"]


def kernel_source_hash() -> str:
    """sha256 over the decode kernels' sources and the build script; a
    profile's HBM traffic is only reported while the kernels still hash to
    it."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "paged_attention_decode_04_amd")
    for f in DECODE_KERNEL_SOURCES:
        h.update(f.encode())
        h.update(open(os.path.join(pkg, "csrc", f), "rb").read())
    h.update(open(os.path.join(pkg, "build.py"), "rb").read())
    return h.hexdigest()


def profiled_traffic(kernel: str, workload: str, launch: dict):
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this kernel and workload, or None if absent, taken
    on other kernel sources or in another launch configuration."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    doc = json.load(open(path))
    if doc.get("source_sha256") != kernel_source_hash() or doc.get("launch") != launch:
        return None
    return int(round(doc["traffic_bytes_per_launch"]))


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_ctx_gqa8")
    ap.add_argument("--variant", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--schedule", default="auto", choices=["auto", "partitions", "balanced", "fitted"])
    ap.add_argument("--shares", type=int, default=0, help="balanced schedule: shares; fitted: workgroups to fill (0 = automatic)")
    ap.add_argument("--merge", default="auto", choices=["auto", "kernel", "fused"],
                    help="split partitions merged by a second kernel or inside the decode kernel")
    ap.add_argument("--window", type=int, default=0,
                    help="attend to each sequence's last WINDOW tokens only (the timed step; 0 = all)")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "f16", "f32"],
                    help="storage type of the K/V cache and Q of the timed step")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--no-probes", action="store_true", help="skip the streaming-read probes")
    ap.add_argument("--profile", action="store_true",
                    help="timed steps only (no per-config sweep, no CPU baseline): for rocprofv3 runs")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a HIP graph (as the per-config lines are timed) instead of "
                         "launching it eagerly: for kernel traces of the small, launch-bound workloads")
    ap.add_argument("--profile-prefill", action="store_true",
                    help="only the several-query (chunked-prefill) line, printed as the JSON line: "
                         "for rocprofv3 runs over its kernel")
    ap.add_argument("--timeline", metavar="WORKLOAD", default=None,
                    help="per-workgroup phase timeline (pa_trace_set) of one call of WORKLOAD on the "
                         "partitioned MFMA decode, warm and MALL-cold, summarised per phase as one JSON line")
    ap.add_argument("--issue-probe", action="store_true",
                    help="only the MFMA/VALU issue-rate probe, printed as one JSON line")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also time a plain device copy of this many MiB (HBM reference and the "
                         "calibration kernel for rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="a headline oracle run longer than this is not repeated (else: median of 3)")
    return ap.parse_args()


# ----------------------------------------------------------------------------
def make_workspace(pa, d, knobs):
    """A zeroed, 256-byte-aligned workspace for calls of d's shape (None when
    they do not split)."""
    import torch
    q, k, v = d.call(0)
    B, Hq, D = q.shape
    NP, P, Hkv, _ = k.shape
    n = pa.pa_decode_workspace_bytes(B, Hq, Hkv, D, d.block_tables.shape[1], P, pa.make_opts(**knobs))
    if not n:
        return None
    raw = torch.zeros(n + 256, dtype=torch.uint8, device=q.device)
    off = (-raw.data_ptr()) % 256
    return raw[off:off + n]


def make_call(pa, d, call, knobs, ws=None):
    """A closure issuing one decode call on the current stream; knobs are
    make_opts' keyword arguments (variant, partition_tokens, schedule, shares,
    window, merge).  The calls of one workload share ws, as the layers of a
    decode step share one workspace (a new one is made when none is given)."""
    import torch
    q, k, v = d.call(call)
    out = torch.empty_like(q)
    B, Hq, D = q.shape
    NP, P, Hkv, _ = k.shape
    opts = pa.make_opts(**knobs)
    if ws is None:
        ws = make_workspace(pa, d, knobs)
    scale = d.w.scale

    def run():
        pa.pa_decode_ex(q, k, v, d.block_tables, d.context_lens, scale, Hq, Hkv, D, P, out,
                        None, opts, ws)
    return run, out


def event_time_ms(fn, n, torch):
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e)


def graph_time_us(calls, reps, torch):
    """Capture the list of calls into one HIP graph, replay it, and return
    the event-timed microseconds per call."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for c in calls:          # warm outside the graph
            c()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    ms = event_time_ms(g.replay, reps, torch)
    return 1e3 * ms / (reps * len(calls))


# ----------------------------------------------------------------------------
def launch_info(st):
    """Kernel names and launch configuration of the last call, from the counters."""
    variant = {1: "valu", 2: "mfma"}.get(int(st["last_variant"]), "?")
    schedule = {2: "balanced", 4: "fitted"}.get(int(st["last_schedule"]), "partitions")
    balanced = schedule == "balanced"
    if variant == "valu":
        kernel, merge = "pa_decode_valu_kernel", "pa_lse_merge_kernel"
    elif balanced:
        kernel, merge = "pa_decode_mfma_lean_kernel", "pa_lean_merge_kernel"
    else:
        kernel, merge = "pa_decode_mfma_kernel", "pa_lse_merge_kernel"
    # fitted: partition_tokens is the largest size the device may pick and
    # partitions the partial slots per sequence (the smallest size)
    launch = {"variant": variant, "schedule": schedule,
              "partition_tokens": int(st["last_partition_tokens"]),
              ("shares" if balanced else "partitions"): int(st["last_num_partitions"])}
    if st["split_calls"] and not balanced:
        launch["merge"] = "fused" if st["fused_calls"] else "kernel"
    return kernel, (merge if st["merge_launches"] else None), launch


# Extra per-config lines: (workload, window, K/V element type).  The window
# on two workloads, an fp16 cache, an fp32 cache and head_dim 512.
EXTRA = (("long_ctx_gqa8", 4096, "bf16"), ("hd256_gqa4", 1024, "bf16"),
         ("long_ctx_gqa8", 0, "f16"), ("batch16", 0, "f32"), ("hd512_gqa4", 0, "bf16"))
ELEM_BYTES = {"bf16": 2, "f16": 2, "f32": 4}


def probe_sink(torch):
    return torch.zeros(4096, dtype=torch.int32, device="cuda")


def stream_probes(torch, d):
    """Streaming-read references (libpa_probe.so): a 4 GiB contiguous read,
    and the headline workload's own paged NHD pattern (256-byte K and V rows
    of one KV head at the 2 KB slot stride, pages in block-table order), at
    several workgroup counts.  GB/s = bytes read / event time per read."""
    from paged_attention_decode_04_amd import probe
    sink = probe_sink(torch)
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    res = {"contiguous_GBps": {}, "nhd_GBps": {}}
    for n_wg in (256, 512, 1024, 2048):
        fn = lambda: probe.read_contiguous(buf, n_wg, sink)
        event_time_ms(fn, 2, torch)
        ms = event_time_ms(fn, 10, torch) / 10
        res["contiguous_GBps"][n_wg] = round(buf.numel() / (ms * 1e-3) / 1e9, 1)
    del buf
    torch.cuda.empty_cache()
    desc = probe.paged_desc(d.k[0], d.v[0], d.block_tables, d.context_lens)
    import workloads as wl
    nbytes = wl.kv_bytes(d.w, d.layout.context_lens)
    for n_wg in (256, 512):
        fn = lambda: probe.read_paged(desc, n_wg, sink)
        event_time_ms(fn, 2, torch)
        ms = event_time_ms(fn, 10, torch) / 10
        res["nhd_GBps"][n_wg] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    res["stream_peak_GBps"] = max(res["contiguous_GBps"].values())
    res["nhd_peak_GBps"] = max(res["nhd_GBps"].values())
    res["note"] = ("contiguous: 4 GiB read once per launch, n_wg workgroups of 256 threads; nhd: the K and V "
                   "rows of the headline workload read through its block tables in equal shares (probe kernels "
                   "of libpa_probe.so, event-timed)")
    log(f"[probe] {res}")
    return res


def per_config(pa, knobs, torch, workloads_mod, probes=None):
    """Time every workload: warm (inputs reused, MALL may hold them) and, for
    footprints that fit the 256 MB MALL, cold (calls rotate over replicas of
    the KV pools totalling >= 1 GB).  Windowed lines count the KV bytes of
    the attended tokens only.  Unwindowed 16-bit lines also time the paged
    streaming-read probe over the same pools (warm and cold), the reference
    for what the memory system gives that access pattern."""
    import numpy as np
    from paged_attention_decode_04_amd import probe
    sink = probe_sink(torch)
    stream_peak = probes["stream_peak_GBps"] if probes else None
    res = {}
    runs = [(name, 0, "bf16") for name in workloads_mod.ORDER] + list(EXTRA)
    for name, window, dt in runs:
        w = workloads_mod.WORKLOADS[name]
        if name == "long_ctx_gqa8":
            d = workloads_mod.device_inputs(w, seed=0, dtype=dt)
        else:
            d = workloads_mod.to_device(workloads_mod.make_inputs(w, seed=0, dtype=dt))
        lens = d.layout.context_lens
        kn = dict(knobs, window=window)
        kvb = workloads_mod.kv_bytes(w, lens, window, ELEM_BYTES[dt])
        n_calls = w.calls if w.calls > 1 else 1
        pa.pa_reset_stats()
        ws = make_workspace(pa, d, kn)
        calls = [make_call(pa, d, i, kn, ws)[0] for i in range(n_calls)]
        entry = {"kv_bytes_per_call": kvb, "calls": n_calls}
        if window:
            entry["window"] = window
        entry["kv_dtype"] = dt
        if name == "long_ctx_gqa8":
            ms = event_time_ms(calls[0], 3, torch)
            ms = event_time_ms(calls[0], 10, torch) / 10
            entry["us_per_call"] = round(1e3 * ms, 2)
            if probes and not window and dt == "bf16":
                # the paged probe of this very pattern (stream_probes), its best workgroup count
                entry["probe_us"] = round(kvb / (probes["nhd_peak_GBps"] * 1e3), 2)
        else:
            # one graph of at least 64 calls, so graph-launch cost is amortised
            warm = calls * max(1, -(-64 // n_calls))
            reps = max(3, min(200, int(20000 // len(warm))))
            entry["us_per_call"] = round(graph_time_us(warm, reps, torch), 3)
            footprint = kvb * (w.layers if w.layers > 1 else 1)
            R = min(int(np.ceil(1.0e9 / max(footprint, 1))), 64)
            if R > 1:
                reps_k = []
                for r in range(R):
                    k2 = d.k.clone()
                    v2 = d.v.clone()
                    d2 = workloads_mod.DeviceInputs(w, d.q, k2, v2, d.block_tables, d.context_lens,
                                                    d.layout)
                    reps_k.append(d2)
                # call k on replica k mod R: each replica's bytes were last
                # read R - 1 calls (>= 1 GB) before; at least 64 calls per
                # graph, so the graph's own launch is amortised as in the
                # warm line
                n_cold = max(64, min(n_calls * R, 2048))
                cold_calls = [make_call(pa, reps_k[k % R], k % n_calls, kn, ws)[0] for k in range(n_cold)]
                entry["us_per_call_cold"] = round(graph_time_us(cold_calls, 5, torch), 3)
                entry["cold_replicas"] = R
                if not window and dt != "f32" and w.head_dim <= 256:
                    # the same bytes, read with no arithmetic, over the same replicas
                    descs = [probe.paged_desc(d2.k[0], d2.v[0], d2.block_tables, d2.context_lens) for d2 in reps_k]
                    pcalls = [(lambda dd=dd: probe.read_paged(dd, 256, sink)) for dd in descs]
                    entry["probe_us_cold"] = round(graph_time_us(pcalls * max(1, 64 // len(pcalls)), 5, torch), 3)
                del reps_k
                if not window and dt != "f32" and kvb >= (64 << 20):
                    # as many bytes read contiguously (no block table, no page
                    # scatter), best of 256 / 512 workgroups, same rotation
                    bufs = [torch.empty(kvb // 16 * 16, dtype=torch.uint8, device="cuda") for _ in range(R)]
                    best = None
                    for n_wg in (256, 512):
                        cc = [(lambda bb=bufs[k % R]: probe.read_contiguous(bb, n_wg, sink)) for k in range(64)]
                        t = graph_time_us(cc, 5, torch)
                        best = t if best is None else min(best, t)
                    entry["contig_probe_us_cold"] = round(best, 3)
                    del bufs
            if not window and dt != "f32" and w.head_dim <= 256:
                desc = probe.paged_desc(d.k[0], d.v[0], d.block_tables, d.context_lens)
                entry["probe_us"] = round(graph_time_us([lambda: probe.read_paged(desc, 256, sink)] * 64, 20,
                                                        torch), 3)
        kernel, _, launch = launch_info(pa.pa_get_stats())
        entry["kernel"] = kernel
        entry.update(launch)
        for key in ("us_per_call", "us_per_call_cold"):
            if key in entry:
                gbs = kvb / (entry[key] * 1e-6) / 1e9
                entry[key.replace("us_per_call", "kv_GBps")] = round(gbs, 1)
                entry[key.replace("us_per_call", "hbm_frac")] = round(gbs / HBM_PEAK_GBS, 4)
                if stream_peak:
                    entry[key.replace("us_per_call", "stream_frac")] = round(gbs / stream_peak, 4)
        for key in ("probe_us", "probe_us_cold", "contig_probe_us_cold"):
            if key in entry:
                # the probe's time as a fraction of the decode call's: 1.0 = as fast as streaming the bytes
                call_key = "us_per_call_cold" if key.endswith("_cold") else "us_per_call"
                entry[key.replace("_us", "").replace("probe", "frac_of_probe")] = round(entry[key] / entry[call_key], 4)
                entry[key.replace("_us", "_hbm_frac")] = round(kvb / (entry[key] * 1e3) / HBM_PEAK_GBS, 4)
        key = name + (f"_w{window}" if window else "") + (f"_{dt}" if dt != "bf16" else "")
        res[key] = entry
        log(f"[per_config] {key}: {entry}")
        del d, calls
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return res


def append_line(pa, torch, workloads_mod, name="long_ctx_gqa8"):
    """KV-cache append at one workload's geometry (one new token per
    sequence): graph-timed microseconds per call.  Algorithmic bytes: the new
    K and V rows read and written once."""
    w = workloads_mod.WORKLOADS[name]
    d = workloads_mod.device_inputs(w, seed=0) if name == "long_ctx_gqa8" else \
        workloads_mod.to_device(workloads_mod.make_inputs(w, seed=0))
    B, Hkv, D = w.batch, w.num_kv_heads, w.head_dim
    kn = torch.randn((B, Hkv, D), device="cuda").to(torch.bfloat16)
    vn = torch.randn((B, Hkv, D), device="cuda").to(torch.bfloat16)
    k, v = d.k[0], d.v[0]
    calls = [lambda: pa.cache_append(kn, vn, k, v, d.block_tables, d.context_lens)] * 64
    us = graph_time_us(calls, 50, torch)
    nbytes = 2 * 2 * B * Hkv * D * 2
    entry = {"workload": name, "us_per_call": round(us, 3), "bytes_per_call": nbytes,
             "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "kernel": "pa_cache_append_kernel"}
    log(f"[append] {entry}")
    del d
    torch.cuda.empty_cache()
    return entry


def prefill_line(pa, torch, workloads_mod, B=8, ctx=4096, chunk=512, Hq=32, Hkv=8, D=128, P=16):
    """Several queries per sequence: B sequences of ctx tokens whose last
    chunk tokens are queried (chunked prefill).  Graph-timed microseconds
    per call, attention FLOPs (4 D Hq per query per attended token) as
    TFLOP/s against the dense bf16 MFMA peak."""
    import numpy as np
    w = workloads_mod.custom("prefill_chunks", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                             page_size=P, ctx=(ctx,) * B)
    inp = workloads_mod.make_inputs(w, seed=0)
    d = workloads_mod.to_device(inp)
    rows = B * chunk
    q = torch.randn((rows, Hq, D), device="cuda").to(torch.bfloat16)
    qs = torch.arange(0, rows + 1, chunk, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    k, v = d.k[0], d.v[0]
    calls = [lambda: pa.prefill(q, k, v, d.block_tables, d.context_lens, qs, w.scale, out=out)] * 16
    us = graph_time_us(calls, 20, torch)
    st = pa.pa_get_stats()
    staged = st["last_schedule"] == pa.PA_SCHEDULE_STAGED
    ws = torch.zeros(pa.pa_prefill_workspace_bytes(rows, B, Hq, Hkv, D, d.block_tables.shape[1], P,
                                                   pa.make_opts(schedule="partitions")) + 256,
                     dtype=torch.uint8, device="cuda")
    calls = [lambda: pa.prefill(q, k, v, d.block_tables, d.context_lens, qs, w.scale, out=out,
                                schedule="partitions", workspace=ws[:ws.numel() - 256])] * 16
    us_blocks = graph_time_us(calls, 20, torch)
    st_blocks = pa.pa_get_stats()
    attended = B * (chunk * (ctx - chunk) + chunk * (chunk + 1) // 2)
    flops = 4 * D * Hq * attended
    tflops = flops / (us * 1e-6) / 1e12
    kvb = B * ctx * Hkv * D * 4
    entry = {"workload": f"{B} seqs x ctx {ctx}, last {chunk} tokens queried, Hq{Hq}/Hkv{Hkv}, d{D}, page {P}",
             "us_per_call": round(us, 2), "flops_per_call": flops, "TFLOPs": round(tflops, 1),
             "kv_bytes_per_call": kvb, "kv_GBps": round(kvb / (us * 1e-6) / 1e9, 1),
             "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
             "kernel": "pa_prefill_staged_kernel" if staged else "pa_prefill_mfma_kernel",
             "schedule": "staged" if staged else "partitions",
             "per_block_kernel": {"kernel": "pa_prefill_mfma_kernel", "us_per_call": round(us_blocks, 2),
                                  "TFLOPs": round(flops / (us_blocks * 1e-6) / 1e12, 1),
                                  "partitions": int(st_blocks["last_num_partitions"])}}
    log(f"[prefill] {entry}")
    del d
    torch.cuda.empty_cache()
    return entry


def _pct(a, q):
    import numpy as np
    return float(np.percentile(a, q)) if len(a) else float("nan")


def timeline_summary(rec, khz, lens, D, elem):
    """Phase statistics of one call's timeline records (PA_TRACE_WORDS uint64
    per workgroup) in microseconds from the first workgroup's entry."""
    import numpy as np
    rec = rec[rec[:, 4] != 0]
    flags = (rec[:, 7] >> np.uint64(32)).astype(np.int64)
    T = (rec[:, 7] & np.uint64(0xFFFFFFFF)).astype(np.int64)
    t = rec[:, :5].astype(np.int64)
    us = 1e3 / khz                                        # microseconds per tick
    t0 = t[:, 0].min()
    run = flags != 1
    tr = (t[run] - t0) * us
    b = (rec[run, 6] & np.uint64(0xFFFF)).astype(np.int64)
    part = (rec[run, 6] >> np.uint64(32)).astype(np.int64)
    Tr = T[run]
    L = np.asarray(lens, dtype=np.int64)[b]
    tokens = np.clip(L - part * Tr, 0, Tr)
    stream_us = tr[:, 2] - tr[:, 1]
    gbs = tokens * D * elem * 2 / np.maximum(stream_us, 1e-3) / 1e3    # K and V rows of one KV head
    where = rec[:, 5]
    xcc = (where >> np.uint64(32)).astype(np.int64)
    cu = ((where >> np.uint64(8)) & np.uint64(0xFF)).astype(np.int64)
    per_cu = {}
    for x, c in zip(xcc.tolist(), cu.tolist()):
        per_cu[(x, c)] = per_cu.get((x, c), 0) + 1
    out = {
        "workgroups": int(len(rec)), "ran_partition": int(run.sum()),
        "partition_tokens": int(Tr[0]) if len(Tr) else 0,
        "merged_in_kernel": int((flags == 2).sum()),
        "cus_used": len(per_cu), "max_wgs_per_cu": max(per_cu.values()) if per_cu else 0,
        "decode_span_us": round(float((t[:, 4].max() - t0) * us), 3),
    }
    def stat(name, v):
        out[name] = {"min": round(float(v.min()), 3), "p50": round(_pct(v, 50), 3), "p90": round(_pct(v, 90), 3),
                     "max": round(float(v.max()), 3)}
    stat("entry_us", (t[:, 0] - t0) * us)
    stat("prologue_us", tr[:, 1] - tr[:, 0])
    stat("streaming_us", stream_us)
    stat("stream_end_us", tr[:, 2])
    stat("wave_merge_us", tr[:, 3] - tr[:, 2])
    stat("exit_us", tr[:, 4])
    stat("stream_GBps_per_wg", gbs)
    if (flags == 2).any():
        stat("kernel_merge_us", (t[flags == 2, 4] - t[flags == 2, 3]) * us)
    # Workgroups whose partition is full (T tokens) stream the same bytes:
    # their streaming time split by query block (which KV head they read)
    # and by XCD.
    qb = ((rec[run, 6] >> np.uint64(16)) & np.uint64(0xFFFF)).astype(np.int64)
    xr = (rec[run, 5] >> np.uint64(32)).astype(np.int64)
    full = tokens == Tr
    out["full_partitions"] = int(full.sum())
    def groups(keys):
        res = {}
        for k in sorted(set(keys[full].tolist())):
            v = stream_us[full & (keys == k)]
            res[str(k)] = {"n": int(len(v)), "p50": round(_pct(v, 50), 3), "max": round(float(v.max()), 3)}
        return res
    if full.any():
        out["stream_full_by_query_block_us"] = groups(qb)
        out["stream_full_by_xcd_us"] = groups(xr)
    last = {}
    for x, e in zip(xcc.tolist(), ((t[:, 4] - t0) * us).tolist()):
        last[x] = max(last.get(x, 0.0), e)
    out["exit_by_xcd_us"] = {str(k): round(v, 3) for k, v in sorted(last.items())}
    return out


def timeline_line(pa, torch, workloads_mod, name, knobs):
    """One traced call of `name` (warm and on the MALL-cold replica rotation)
    with the per-phase statistics of its workgroups, and the untraced call
    time of the same graphs for comparison."""
    import numpy as np
    w = workloads_mod.WORKLOADS[name]
    d = workloads_mod.to_device(workloads_mod.make_inputs(w, seed=0))
    lens = d.layout.context_lens
    kvb = workloads_mod.kv_bytes(w, lens)
    khz = pa.pa_trace_clock_khz()
    ws = make_workspace(pa, d, knobs)
    call = make_call(pa, d, 0, knobs, ws)[0]
    R = min(int(np.ceil(1.0e9 / max(kvb, 1))), 64)
    reps_k = [workloads_mod.DeviceInputs(w, d.q, d.k.clone(), d.v.clone(), d.block_tables, d.context_lens, d.layout)
              for _ in range(R)]
    cold = [make_call(pa, reps_k[k % R], 0, knobs, ws)[0] for k in range(max(64, R))]
    res = {"workload": name, "kv_bytes_per_call": kvb, "clock_khz": khz, "cold_replicas": R}
    res["warm_us_untraced"] = round(graph_time_us([call] * 64, 20, torch), 3)
    res["cold_us_untraced"] = round(graph_time_us(cold, 5, torch), 3)
    buf = torch.zeros(16384 * pa.PA_TRACE_WORDS, dtype=torch.int64, device="cuda")
    pa.pa_trace_set(buf)
    try:
        res["warm_us_traced"] = round(graph_time_us([call] * 64, 20, torch), 3)
        torch.cuda.synchronize()
        rec_w = buf.view(-1, pa.PA_TRACE_WORDS).cpu().numpy().astype(np.uint64)
        buf.zero_()
        res["cold_us_traced"] = round(graph_time_us(cold, 5, torch), 3)
        torch.cuda.synchronize()
        rec_c = buf.view(-1, pa.PA_TRACE_WORDS).cpu().numpy().astype(np.uint64)
    finally:
        pa.pa_trace_set(None)
    kernel, _, launch = launch_info(pa.pa_get_stats())
    res["kernel"] = kernel
    res["launch"] = launch
    res["warm"] = timeline_summary(rec_w, khz, lens, w.head_dim, 2)
    res["cold"] = timeline_summary(rec_c, khz, lens, w.head_dim, 2)
    return res


def issue_probe_line(torch, rounds=4096):
    """How MFMA and vector-ALU work share a SIMD (libpa_probe.so's issue-rate
    probe): per mode, rounds of NM 16x16x32 bf16 MFMAs and NV independent fp32
    FMAs, in every wave (mixed) or in separate MFMA-only and FMA-only waves,
    at one and four waves per SIMD.  Times are turned into cycles per
    wave-round with one clock calibration: the MFMA-only mode at four waves
    per SIMD keeps the matrix pipe saturated at 16 cycles per MFMA.
    References: serial = 16 NM + 4 NV cycles (the two pipes one after the
    other), overlapped = max(16 NM, 4 NV); for split modes, per wave-round
    over both kinds of wave, half of each."""
    from paged_attention_decode_04_amd import probe
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(4 * cus, dtype=torch.int32, device="cuda")
    modes = probe.issue_modes()
    times = {}
    for wps in (1, 4):
        n_wg = cus * wps                      # 4 waves per workgroup, 4 SIMDs per CU
        for i in range(len(modes)):
            f = (lambda i=i, n_wg=n_wg: probe.issue(i, n_wg, rounds, sink))
            event_time_ms(f, 2, torch)
            times[(wps, i)] = min(event_time_ms(f, 5, torch) / 5 for _ in range(3))
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
    ref = next(i for i, m in enumerate(modes) if m == (1, 0, True))
    hz = rounds * 4 * 16 / (times[(4, ref)] * 1e-3)      # cycles per second of the saturated MFMA run
    rows = []
    for (wps, i), ms in sorted(times.items()):
        nm, nv, mixed = modes[i]
        cyc = ms * 1e-3 * hz / (rounds * wps)
        serial = 16 * nm + 4 * nv
        over = max(16 * nm, 4 * nv)
        if not mixed:
            serial, over = serial / 2, over / 2
        rows.append({"waves_per_simd": wps, "mfma_per_round": nm, "fma_per_round": nv,
                     "waves": "mixed" if mixed else "split", "us_per_launch": round(ms * 1e3, 2),
                     "cycles_per_wave_round": round(cyc, 1), "serial_cycles": serial, "overlapped_cycles": over})
    return {"probe": "issue-rate (pa_probe_issue)", "cus": cus, "rounds": rounds,
            "clock_GHz_from_mfma_rate": round(hz / 1e9, 3), "modes": rows}


def _median_time(fn, runs):
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2], len(ts)


def cpu_baseline(d, w, target_s, workloads_mod):
    """The oracle as it stands (fp64, the plain definition) on the host cores:
    the headline workload's whole call on all threads, and one call of each
    other workload on all threads and, for the three small ones, on one
    thread.  Median of 3 runs (one where a run takes longer than target_s);
    input generation and host copies are not timed.  Unit: KV-read GB/s."""
    import oracle
    threads = oracle.default_threads()
    host = workloads_mod.host_copy(d)
    lens = host.context_lens
    kvb = workloads_mod.kv_bytes(w, lens)

    def head():
        oracle.attention(host.q[0], host.k[0], host.v[0], host.block_tables, lens, w.scale, w.num_kv_heads,
                         threads=threads)
    t0 = time.perf_counter()
    head()
    first = time.perf_counter() - t0
    t_med, runs = (first, 1) if first > target_s else _median_time(head, 3)
    per = {}
    for name in ("tiny", "single_seq", "batch16", "hd256_gqa4"):
        wk = workloads_mod.WORKLOADS[name]
        inp = workloads_mod.make_inputs(wk, seed=0)
        q, k, v = inp.call(0)
        nbytes = workloads_mod.kv_bytes(wk, inp.context_lens)
        entry = {"kv_bytes_per_call": nbytes}
        for label, nt in (("all", threads), ("1thread", 1)):
            if label == "1thread" and name == "hd256_gqa4":
                continue
            tm, n = _median_time(lambda: oracle.attention(q, k, v, inp.block_tables, inp.context_lens, wk.scale,
                                                          wk.num_kv_heads, threads=nt), 3)
            sfx = "" if label == "all" else "_1thread"
            entry["us_per_call" + sfx] = round(tm * 1e6, 1)
            entry["GBps" + sfx] = round(nbytes / tm / 1e9, 4)
        per[name] = entry
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:
        pass
    per[w.name] = {"kv_bytes_per_call": kvb, "us_per_call": round(t_med * 1e6, 1),
                   "GBps": round(kvb / t_med / 1e9, 4)}
    return {"value": round(kvb / t_med / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle", "cpu": cpu,
            "seconds": round(t_med, 2), "runs": runs, "us_per_call_equiv": round(1e6 * t_med, 1),
            "sample": f"the whole {w.name} call ({w.batch} sequences, {int(lens.sum())} tokens, all "
                      f"{w.num_q_heads} query heads), fp64, {threads} threads, median of {runs}; per_config: "
                      f"one call of each other workload, all threads and (tiny, single_seq, batch16) one thread, "
                      f"median of 3",
            "per_config": per}


def advancing_line(pa, torch, workloads_mod, knobs, name="hd256_gqa4", n_calls=64, R=8):
    """A decode loop: n_calls calls whose lengths advance by one token per
    call (sequence b at L_b - n_calls + 1 + i in call i, inside the pages the
    workload already holds), all on one workspace, so the fitted schedule's
    per-workgroup hint is taken from the previous call as in a real decode.
    Warm (one pool) and MALL-cold (call i on replica i mod R, R * footprint
    >= 1 GB); microseconds per call averaged over the loop."""
    import numpy as np
    w = workloads_mod.WORKLOADS[name]
    d = workloads_mod.to_device(workloads_mod.make_inputs(w, seed=0))
    base = d.layout.context_lens.astype(np.int64)
    lens = [np.maximum(base - (n_calls - 1) + i, 1).astype(np.int32) for i in range(n_calls)]
    ctx = [torch.from_numpy(x).cuda() for x in lens]
    kvb = float(np.mean([workloads_mod.kv_bytes(w, x) for x in lens]))
    q, k, v = d.call(0)
    B, Hq, D = q.shape
    NP, P, Hkv, _ = k.shape
    opts = pa.make_opts(**knobs)
    n = pa.pa_decode_workspace_bytes(B, Hq, Hkv, D, d.block_tables.shape[1], P, opts)
    raw = torch.zeros(n + 256, dtype=torch.uint8, device="cuda")
    ws = raw[(-raw.data_ptr()) % 256:][:max(n, 1)]
    out = torch.empty_like(q)
    pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(R - 1)]

    def call(i, pool):
        kk, vv = pool
        return lambda: pa.pa_decode_ex(q, kk, vv, d.block_tables, ctx[i], w.scale, Hq, Hkv, D, P, out, None, opts,
                                       ws if n else None)
    warm = graph_time_us([call(i, pools[0]) for i in range(n_calls)], 20, torch)
    cold = graph_time_us([call(i, pools[i % R]) for i in range(n_calls)], 20, torch)
    _, _, launch = launch_info(pa.pa_get_stats())
    entry = {"workload": f"{name}, lengths advancing one token per call over {n_calls} calls",
             "kv_bytes_per_call": round(kvb), "us_per_call": round(warm, 3), "us_per_call_cold": round(cold, 3),
             "cold_replicas": R, **launch}
    for key in ("us_per_call", "us_per_call_cold"):
        gbs = kvb / (entry[key] * 1e-6) / 1e9
        entry[key.replace("us_per_call", "kv_GBps")] = round(gbs, 1)
        entry[key.replace("us_per_call", "hbm_frac")] = round(gbs / HBM_PEAK_GBS, 4)
    log(f"[advancing] {entry}")
    del d, pools
    torch.cuda.empty_cache()
    return entry


def copy_probe(mib, torch):
    """A plain elementwise kernel that reads and writes mib MiB once each
    (torch.neg on fp32): the HBM reference and the kernel whose rocprofv3
    FETCH_SIZE / WRITE_SIZE calibrate the counters."""
    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    reps = 20
    ms = event_time_ms(lambda: torch.neg(src, out=dst), reps, torch) / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read": n, "bytes_written": n, "us": round(ms * 1e3, 2),
            "GBps_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}


# ----------------------------------------------------------------------------
def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "decode paged attention here is a single-GPU kernel; no multi-GPU path exists.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_attention_decode_04_amd as pa
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.profile_prefill:
        print(json.dumps(prefill_line(pa, torch, wl)), flush=True)
        return
    if args.issue_probe:
        print(json.dumps(issue_probe_line(torch)), flush=True)
        return
    if args.timeline:
        knobs = dict(variant=args.variant, partition_tokens=args.partition_tokens,
                     schedule=args.schedule, shares=args.shares, merge=args.merge)
        print(json.dumps(timeline_line(pa, torch, wl, args.timeline, knobs)), flush=True)
        return
    w = wl.WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    dt = args.kv_dtype
    if w.name == "long_ctx_gqa8":
        d = wl.device_inputs(w, seed=args.seed, dtype=dt)
    else:
        d = wl.to_device(wl.make_inputs(w, seed=args.seed, dtype=dt))
    torch.cuda.synchronize()
    log(f"[bench] inputs for {w.name} ({dt}) ready in {time.perf_counter() - t_gen:.1f}s")
    kvb_per_call = wl.kv_bytes(w, d.layout.context_lens, args.window, ELEM_BYTES[dt])
    n_calls = w.calls
    knobs = dict(variant=args.variant, partition_tokens=args.partition_tokens,
                 schedule=args.schedule, shares=args.shares, merge=args.merge)
    if args.window:
        knobs["window"] = args.window
    ws = make_workspace(pa, d, knobs)
    calls = [make_call(pa, d, i, knobs, ws)[0] for i in range(n_calls)]

    def step():                       # one pass of the whole path over the batch
        for c in calls:
            c()

    pa.pa_reset_stats()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = pa.pa_get_stats()
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        step = graph.replay
    ev_s, ev_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_s.record()
    for _ in range(args.steps):
        step()
    ev_e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev_s.elapsed_time(ev_e)
    ms_per_step = 1e3 * wall / args.steps
    us_per_call_ev = 1e3 * gpu_ms / (args.steps * n_calls)
    kv_per_step = kvb_per_call * n_calls
    value = kv_per_step / (ms_per_step * 1e-3) / 1e9
    achieved = kvb_per_call / (us_per_call_ev * 1e-6) / 1e9
    kernel, merge, launch = launch_info(st)
    variant = launch["variant"]
    log(f"[bench] {w.name}: {ms_per_step:.3f} ms/step wall, {us_per_call_ev:.2f} us/call (events), "
        f"{achieved:.0f} GB/s KV, {kernel} {launch}")

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt if variant == "mfma" else "f32",   # MFMA products in the cache's 16-bit type
        "storage_dtype": dt,
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, shuffled block tables)",
        "config": {
            "workload": w.name, "desc": w.desc, "batch": w.batch,
            "sum_ctx": int(d.layout.context_lens.sum()), "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "page_size": w.page_size,
            "calls_per_step": n_calls, "kv_bytes_per_call": kvb_per_call, **launch,
            **({"window": args.window} if args.window else {}),
        },
        "launch_mode": "graph replay" if args.graph else "eager",
        "us_per_call": round(us_per_call_ev, 3),
        "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            # the committed counter runs are of the bf16, unwindowed workloads
            "traffic": profiled_traffic(kernel, w.name, launch) if dt == "bf16" and not args.window else None,
            "kernel": kernel + (f" + {merge}" if merge else ""),
            "duration_us": round(us_per_call_ev, 3),
            "note": "achieved = algorithmic KV bytes per call / HIP-event time per call over the "
                    "timed region (decode kernel plus merge kernel, on the launch stream)",
        },
    }
    if args.copy_probe_mib:
        result["copy_probe"] = copy_probe(args.copy_probe_mib, torch)
        log(f"[bench] copy probe: {result['copy_probe']}")
    probes = None
    if not args.profile and not args.no_probes:
        probes = stream_probes(torch, d) if w.head_dim * 2 in (256, 512) else None
        if probes:
            result["stream_probe"] = probes
            result["stream_peak_GBps"] = probes["stream_peak_GBps"]
            result["stream_frac"] = round(achieved / probes["stream_peak_GBps"], 4)
            result["nhd_stream_frac"] = round(achieved / probes["nhd_peak_GBps"], 4)
    if not args.profile and not args.no_per_config:
        result["per_config"] = per_config(pa, knobs, torch, wl, probes)
        result["advancing"] = advancing_line(pa, torch, wl, knobs)
        result["append"] = append_line(pa, torch, wl)
        result["prefill"] = prefill_line(pa, torch, wl)
        # several queries per sequence in a decode step (speculative decoding)
        result["prefill_spec4"] = prefill_line(pa, torch, wl, B=64, ctx=8192, chunk=4, Hq=64, Hkv=8)
    if not args.profile and not args.no_cpu_baseline:
        t = time.perf_counter()
        result["cpu_baseline"] = cpu_baseline(d, w, args.cpu_seconds, wl)
        log(f"[bench] cpu baseline in {time.perf_counter() - t:.1f}s: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
