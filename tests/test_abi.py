"""The C ABI without a GPU: the library loads, exports every function the
header declares, and validates arguments on the host (no HIP call)."""
import ctypes
import os
import re

import pytest
import torch

import paged_attention_decode_04_amd as pa
from paged_attention_decode_04_amd import _binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "pa_decode.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(pa_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("pa_decode", "pa_decode_ex", "pa_decode_workspace_bytes", "pa_check_args",
                 "pa_get_stats", "pa_reset_stats", "pa_strerror", "pa_last_error",
                 "pa_release", "pa_version"):
        assert must in names


def test_trace_set_arguments():
    lib = _binding.LIB
    assert lib.pa_trace_set(None, 0) == pa.PA_OK                  # stop (also when never started)
    assert lib.pa_trace_set(ctypes.c_void_p(0x1008), 4096) == pa.PA_EINVAL   # not 16-byte aligned
    assert "aligned" in pa.last_error()
    assert lib.pa_trace_set(None, 4096) == pa.PA_OK
    assert pa.PA_TRACE_WORDS == 8
    assert lib.pa_trace_clock_khz(None) == pa.PA_EINVAL
    if not torch.cuda.is_available():
        v = ctypes.c_int(0)
        assert lib.pa_trace_clock_khz(ctypes.byref(v)) in (pa.PA_ENODEV, pa.PA_EHIP)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pa.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


PROBE_HEADER = os.path.join(os.path.dirname(HEADER), "pa_probe.h")


def test_probe_library_exports_and_validates():
    """libpa_probe.so (the benchmark's streaming-read and issue-rate probes)
    exports every function pa_probe.h declares and refuses bad arguments
    before any HIP call."""
    from paged_attention_decode_04_amd import probe
    lib = ctypes.CDLL(probe.PROBE_LIB_PATH)
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"^\s*int\s+(pa_probe_[a-z_]+)\s*\(", text, flags=re.M)))
    assert names == ["pa_probe_issue", "pa_probe_issue_modes", "pa_probe_read_contiguous", "pa_probe_read_paged"]
    assert all(hasattr(lib, n) for n in names)
    plib = probe._load()
    assert plib.pa_probe_read_contiguous(None, 16, 1, None, None) == 1
    assert plib.pa_probe_read_contiguous(0x1008, 16, 1, 0x2000, None) == 1      # misaligned base
    assert plib.pa_probe_read_contiguous(0x1000, 17, 1, 0x2000, None) == 1      # not whole 16-byte chunks
    d = probe.PaProbePaged()
    assert plib.pa_probe_read_paged(ctypes.byref(d), 256, 0x2000, None) == 1   # null pools
    d.k = d.v = 0x1000
    d.block_tables = d.context_lens = 0x3000
    d.row_bytes, d.batch, d.num_kv_heads, d.num_pages, d.max_blocks, d.bt_sb = 256, 4, 2, 8, 4, 4
    d.k_sp = d.v_sp = 16 * 2 * 256
    d.k_ss = d.v_ss = 2 * 256
    d.k_sh = d.v_sh = 256
    d.page_size = 24                                                            # not a power of two
    assert plib.pa_probe_read_paged(ctypes.byref(d), 256, 0x2000, None) == 1
    d.page_size = 16
    d.row_bytes = 128
    assert plib.pa_probe_read_paged(ctypes.byref(d), 256, 0x2000, None) == 1
    d.row_bytes = 256
    assert plib.pa_probe_read_paged(ctypes.byref(d), 0, 0x2000, None) == 1     # no workgroups
    # the issue-rate probe: its menu, and arguments refused before any launch
    assert probe.issue_modes()[0] == (1, 0, True)
    n = len(probe.issue_modes())
    assert plib.pa_probe_issue_modes(n, None, None, None) == -1
    assert plib.pa_probe_issue(0, 256, 16, None, None) == 1                     # no sink
    assert plib.pa_probe_issue(n, 256, 16, 0x2000, None) == 1                   # mode past the menu
    assert plib.pa_probe_issue(-1, 256, 16, 0x2000, None) == 1
    assert plib.pa_probe_issue(0, 0, 16, 0x2000, None) == 1                     # no workgroups
    assert plib.pa_probe_issue(0, 256, 0, 0x2000, None) == 1                    # no rounds
    assert plib.pa_probe_issue(0, 256, (1 << 20) + 1, 0x2000, None) == 1


def test_version_and_strerror():
    assert pa.version() == "0.1.0"
    for code in range(7):
        assert pa.strerror(code) and pa.strerror(code) != "unknown error code"
    assert pa.strerror(99) == "unknown error code"


# ------------------------------------------------------------- validation
def args(B=2, Hq=16, Hkv=8, D=128, P=16, NP=8, maxblk=4, dtype=torch.bfloat16):
    q = torch.zeros(B, Hq, D, dtype=dtype)
    k = torch.zeros(NP, P, Hkv, D, dtype=torch.bfloat16)
    v = torch.zeros(NP, P, Hkv, D, dtype=torch.bfloat16)
    bt = torch.zeros(B, maxblk, dtype=torch.int32)
    ctx = torch.ones(B, dtype=torch.int32)
    out = torch.zeros(B, Hq, D, dtype=torch.bfloat16)
    return dict(q=q, k_cache=k, v_cache=v, block_tables=bt, context_lens=ctx, scale=0.1,
                num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P, out=out)


def check(a, opts=None):
    return pa.pa_check_args(a["q"], a["k_cache"], a["v_cache"], a["block_tables"],
                            a["context_lens"], a["scale"], a["num_q_heads"], a["num_kv_heads"],
                            a["head_dim"], a["page_size"], a["out"], opts)


def test_valid_arguments_pass():
    assert check(args()) == pa.PA_OK
    assert check(args(Hq=8, Hkv=2, D=256, P=32)) == pa.PA_OK
    assert check(args(Hq=64, Hkv=8)) == pa.PA_OK
    assert check(args(Hq=16, Hkv=1)) == pa.PA_OK
    assert check(args(B=0)) == pa.PA_OK


@pytest.mark.parametrize("mutate,code", [
    (lambda a: a.update(q=a["q"].double()), pa.PA_EINVAL),
    (lambda a: a.update(v_cache=a["v_cache"].half()), pa.PA_EINVAL),   # K and V types differ
    (lambda a: a.update(out=a["out"].to(torch.int32)), pa.PA_EINVAL),
    (lambda a: a.update(num_q_heads=15), pa.PA_EINVAL),
    (lambda a: a.update(scale=float("-inf")), pa.PA_EINVAL),
    (lambda a: a.update(scale=float("inf")), pa.PA_EINVAL),
    (lambda a: a.update(page_size=0), pa.PA_EINVAL),
    (lambda a: a.update(page_size=32), pa.PA_EINVAL),
    (lambda a: a.update(block_tables=torch.zeros(3, 4, dtype=torch.int32)), pa.PA_EINVAL),
    (lambda a: a.update(block_tables=torch.zeros(2, 4, dtype=torch.int64)), pa.PA_EINVAL),
    (lambda a: a.update(context_lens=torch.ones(3, dtype=torch.int32)), pa.PA_EINVAL),
    (lambda a: a.update(out=torch.zeros(2, 16, 64, dtype=torch.bfloat16)), pa.PA_EINVAL),
    (lambda a: a.update(v_cache=torch.zeros(8, 16, 8, 64, dtype=torch.bfloat16)), pa.PA_EINVAL),
    (lambda a: a.update(q=a["q"].transpose(1, 2).contiguous().transpose(1, 2)), pa.PA_EINVAL),
])
def test_bad_arguments_are_rejected(mutate, code):
    a = args()
    mutate(a)
    assert check(a) == code
    assert pa.last_error() != ""


def test_default_scale_sentinel_is_accepted():
    """PA_SCALE_DEFAULT (a NaN) asks the library for 1/sqrt(head_dim)."""
    a = args()
    a.update(scale=pa.PA_SCALE_DEFAULT)
    assert check(a) == pa.PA_OK


def test_element_types_and_head_sizes():
    """bf16 / fp16 / fp32 for Q, K/V and out.  fp32 K/V runs on the
    vector-ALU kernel only (the MFMA variant is ENOTSUP there); head_dim 512
    runs on both, but not on the balanced schedule."""
    for qt in (torch.bfloat16, torch.float16, torch.float32):
        for kt in (torch.bfloat16, torch.float16, torch.float32):
            a = args()
            a.update(q=a["q"].to(qt), k_cache=a["k_cache"].to(kt), v_cache=a["v_cache"].to(kt),
                     out=a["out"].to(qt))
            assert check(a) == pa.PA_OK, (qt, kt)
    a = args()
    a.update(k_cache=a["k_cache"].float(), v_cache=a["v_cache"].float())
    assert check(a, pa.make_opts("mfma")) == pa.PA_ENOTSUP
    assert check(a, pa.make_opts("valu")) == pa.PA_OK
    assert check(args(D=512, Hq=16, Hkv=8)) == pa.PA_OK
    assert check(args(D=512, Hq=16, Hkv=8), pa.make_opts("mfma")) == pa.PA_OK
    assert check(args(D=512, Hq=16, Hkv=8), pa.make_opts("mfma", 0, "balanced")) == pa.PA_ENOTSUP
    a = args()
    big = torch.zeros(8, 16, 8, 130, dtype=torch.float32)[..., :128]   # fp32 rows 520 B apart
    a.update(k_cache=big, v_cache=torch.zeros(8, 16, 8, 128))
    assert check(a) == pa.PA_EALIGN


def test_unsupported_geometry():
    assert check(args(D=64)) == pa.PA_ENOTSUP
    assert check(args(Hq=6, Hkv=2)) == pa.PA_ENOTSUP     # qg = 3
    assert check(args(Hq=32, Hkv=1)) == pa.PA_ENOTSUP    # qg = 32


def test_misalignment():
    a = args()
    big = torch.zeros(2 * 16 * 128 + 1, dtype=torch.bfloat16)
    a["q"] = big[1:].view(2, 16, 128)                      # 2-byte offset
    assert check(a) == pa.PA_EALIGN
    a = args()
    k = torch.zeros(8, 16, 8, 132, dtype=torch.bfloat16)[..., :128]   # row stride 132
    a["k_cache"] = k
    assert check(a) == pa.PA_EALIGN


def test_strided_nhd_views_are_accepted():
    a = args()
    big = torch.zeros(8, 16, 8, 256, dtype=torch.bfloat16)
    a["k_cache"] = big[..., :128]                          # row stride 256
    a["v_cache"] = big[..., 128:]
    assert check(a) == pa.PA_OK


def test_opts_are_validated():
    o = pa.make_opts("valu", 0)
    assert check(args(), o) == pa.PA_OK
    o.reserved[1] = 1
    assert check(args(), o) == pa.PA_EINVAL
    assert check(args(), pa.make_opts(merge=3)) == pa.PA_EINVAL
    # the in-kernel merge: MFMA partition schedules only
    assert check(args(), pa.make_opts("mfma", 64, merge="fused")) == pa.PA_OK
    assert check(args(), pa.make_opts("mfma", 0, "fitted", merge="fused")) == pa.PA_OK
    assert check(args(), pa.make_opts("valu", 64, merge="fused")) == pa.PA_ENOTSUP
    assert check(args(), pa.make_opts("mfma", 0, "balanced", merge="fused")) == pa.PA_ENOTSUP
    assert check(args(), pa.make_opts("mfma", 64, merge="kernel")) == pa.PA_OK
    o = pa.make_opts(7, 0)
    assert check(args(), o) == pa.PA_EINVAL
    o = pa.make_opts("valu", -5)
    assert check(args(), o) == pa.PA_EINVAL
    o = pa.make_opts("mfma", 0, 5)
    assert check(args(), o) == pa.PA_EINVAL
    o = pa.make_opts("mfma", 0, "staged")                 # several queries only
    assert check(args(), o) == pa.PA_ENOTSUP
    assert check(args(), pa.make_opts(window=-1)) == pa.PA_EINVAL
    assert check(args(), pa.make_opts(window=7)) == pa.PA_OK
    for sched in ("auto", "partitions", "balanced", "fitted"):
        assert check(args(), pa.make_opts("mfma", 0, sched)) == pa.PA_OK


def test_fitted_schedule_preconditions():
    """Fitted partitions: MFMA only, no window, no partition size given, at
    most 256 sequences (every workgroup reads all lengths)."""
    fit = lambda **kw: pa.make_opts(schedule="fitted", **kw)
    assert check(args(), fit(variant="mfma")) == pa.PA_OK
    assert check(args(), fit(variant="valu")) == pa.PA_ENOTSUP
    assert "fitted" in pa.last_error()
    assert check(args(), fit(window=64)) == pa.PA_ENOTSUP
    assert check(args(), fit(partition_tokens=256)) == pa.PA_ENOTSUP
    assert check(args(B=256), fit()) == pa.PA_OK
    assert check(args(B=257), fit()) == pa.PA_ENOTSUP
    assert check(args(), fit(shares=1024)) == pa.PA_OK
    # block tables of 2^24 tokens or more keep fixed partitions
    assert check(args(P=16, maxblk=(1 << 20) - 1), fit()) == pa.PA_OK
    assert check(args(P=16, maxblk=1 << 20), fit()) == pa.PA_ENOTSUP
    assert check(args(), fit(shares=1025)) == pa.PA_EINVAL


def test_balanced_schedule_needs_mfma_and_bounded_batch():
    assert check(args(), pa.make_opts("valu", 0, "balanced")) == pa.PA_ENOTSUP
    assert "balanced" in pa.last_error()
    assert check(args(B=4096), pa.make_opts("mfma", 0, "balanced")) == pa.PA_OK
    assert check(args(B=4097), pa.make_opts("mfma", 0, "balanced")) == pa.PA_ENOTSUP
    # automatic choice falls back to partitions past 4096 sequences
    assert check(args(B=4097), pa.make_opts("mfma", 0, "auto")) == pa.PA_OK


def test_null_descriptor_is_einval_not_a_crash():
    a = args()
    T = _binding.tensor_desc
    rc = _binding.LIB.pa_check_args(None, T(a["k_cache"]), T(a["v_cache"]), T(a["block_tables"]),
                                    T(a["context_lens"]), 0.1, 16, 8, 128, 16, T(a["out"]), None)
    assert rc == pa.PA_EINVAL
    rc = _binding.LIB.pa_decode(T(a["q"]), None, T(a["v_cache"]), T(a["block_tables"]),
                                T(a["context_lens"]), 0.1, 16, 8, 128, 16, T(a["out"]), None)
    assert rc == pa.PA_EINVAL


def test_decode_rejects_bad_arguments_before_any_hip_call():
    a = args(D=64)
    T = _binding.tensor_desc
    rc = _binding.LIB.pa_decode(T(a["q"]), T(a["k_cache"]), T(a["v_cache"]), T(a["block_tables"]),
                                T(a["context_lens"]), 0.1, 16, 8, 64, 16, T(a["out"]), None)
    assert rc == pa.PA_ENOTSUP
    with pytest.raises(ValueError):
        pa.pa_decode(**args(), stream=0)        # host tensors never reach the library
    # a later valid check is not affected by the earlier error (no sticky state)
    assert check(args()) == pa.PA_OK and pa.last_error() == ""


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a host without a GPU")
def test_valid_call_without_a_device_is_enodev():
    a = args()
    T = _binding.tensor_desc
    rc = _binding.LIB.pa_decode(T(a["q"]), T(a["k_cache"]), T(a["v_cache"]), T(a["block_tables"]),
                                T(a["context_lens"]), 0.1, 16, 8, 128, 16, T(a["out"]), None)
    assert rc == pa.PA_ENODEV


def test_workspace_bytes():
    # no split: a single partition covers MaxBlk * P tokens
    assert pa.pa_decode_workspace_bytes(4, 16, 8, 128, 4, 32, pa.make_opts("valu", 4096)) == 0
    # forced split of a 1152-token table into 64-token partitions: 18 partitions
    n = pa.pa_decode_workspace_bytes(1, 16, 8, 128, 72, 16, pa.make_opts("valu", 64))
    parts = 18
    o_bytes = 1 * 16 * parts * 128 * 4
    lse_bytes = 1 * 16 * parts * 4
    rnd = lambda x: (x + 255) // 256 * 256
    HDR = pa.PA_WORKSPACE_ZERO_BYTES   # the counters (balanced schedule, in-kernel merge), in every layout
    assert n == HDR + rnd(o_bytes) + rnd(lse_bytes)
    assert pa.pa_decode_workspace_bytes(-1, 16, 8, 128, 4, 32, None) == 0
    # balanced schedule: one partial slot per (group, unit) piece it can
    # produce (groups + 1024 * 7 units at most) of qw = qg query rows, plus the
    # B + 4 ints of tile prefix sums and unit sizes
    B, Hq, Hkv, D = 3, 32, 4, 256
    n = pa.pa_decode_workspace_bytes(B, Hq, Hkv, D, 100, 16, pa.make_opts("mfma", 0, "balanced"))
    slots = (B * (Hq // 8) + 1024 * 7) * 8
    assert n == HDR + rnd(slots * D * 4) + rnd(slots * 4) + rnd((B + 4) * 4)
    # the automatic choice: balanced for a large call (64 sequences of up to
    # 32768 tokens, 8 query blocks), partitions for a small one
    big = pa.pa_decode_workspace_bytes(64, 64, 8, 128, 2048, 16, pa.make_opts("mfma"))
    slots = (64 * 8 + 1024 * 7) * 8
    assert big == HDR + rnd(slots * 128 * 4) + rnd(slots * 4) + rnd(68 * 4)
    assert big == pa.pa_decode_workspace_bytes(64, 64, 8, 128, 2048, 16,
                                               pa.make_opts("mfma", 0, "balanced"))
    # the automatic variant covers both kernels (an fp32 cache takes the
    # vector-ALU one): 8 query heads per workgroup, 1024-token partitions
    auto = pa.pa_decode_workspace_bytes(64, 64, 8, 128, 2048, 16, None)
    valu = HDR + rnd(64 * 64 * 32 * 128 * 4) + rnd(64 * 64 * 32 * 4)
    assert auto == max(big, valu)
    # fitted partitions when asked for: 16 sequences x 8 query blocks of up
    # to 1152 tokens give a largest size of 576, a smallest of 256 (max(256,
    # 576 / 4)), so 5 partial slots, plus the slot of the size picked
    # and one 16-byte hint per workgroup the grid can have (at least 1024)
    fit = pa.pa_decode_workspace_bytes(16, 16, 8, 128, 72, 16, pa.make_opts("mfma", 0, "fitted"))
    assert fit == HDR + rnd(16 * 16 * 5 * 128 * 4) + rnd(16 * 16 * 5 * 4) + 256 + 1024 * 16
    # the automatic choice keeps the 2 fixed partitions there (fewer than 4)
    small = pa.pa_decode_workspace_bytes(16, 16, 8, 128, 72, 16, pa.make_opts("mfma"))
    assert small == pa.pa_decode_workspace_bytes(16, 16, 8, 128, 72, 16,
                                                 pa.make_opts("mfma", 0, "partitions"))
    assert small == HDR + rnd(16 * 16 * 2 * 128 * 4) + rnd(16 * 16 * 2 * 4)
    # one 1152-token sequence: the fixed size is the floor (64 tokens), so
    # the automatic choice keeps fixed partitions (18 of them)
    one = pa.pa_decode_workspace_bytes(1, 16, 8, 128, 72, 16, pa.make_opts("mfma"))
    assert one == HDR + rnd(16 * 18 * 128 * 4) + rnd(16 * 18 * 4)
    # a 128-token table would split in two at 64 tokens: it stays whole
    assert pa.pa_decode_workspace_bytes(4, 16, 8, 128, 4, 32, pa.make_opts("mfma")) == 0
    # 32 sequences x 2 query blocks in a 4096-token table (head_dim 256):
    # 4 fixed partitions of 1024 and 268 MB of KV capacity, so the automatic
    # choice fits them; in 2048-token tables (134 MB) it keeps them fixed
    hd = pa.pa_decode_workspace_bytes(32, 8, 2, 256, 128, 32, pa.make_opts("mfma"))
    assert hd == pa.pa_decode_workspace_bytes(32, 8, 2, 256, 128, 32, pa.make_opts("mfma", 0, "fitted"))
    half = pa.pa_decode_workspace_bytes(32, 8, 2, 256, 64, 32, pa.make_opts("mfma"))
    assert half == pa.pa_decode_workspace_bytes(32, 8, 2, 256, 64, 32, pa.make_opts("mfma", 0, "partitions"))
    assert half != pa.pa_decode_workspace_bytes(32, 8, 2, 256, 64, 32, pa.make_opts("mfma", 0, "fitted"))
    # a window bounds the span a sequence's work covers (W + 15 tokens): the
    # same large call with a 4096-token window falls below the balanced
    # threshold and splits into ceil(4111 / 4096) = 2 partitions of 4096
    n = pa.pa_decode_workspace_bytes(64, 64, 8, 128, 2048, 16, pa.make_opts("mfma", window=4096))
    assert n == HDR + rnd(64 * 64 * 2 * 128 * 4) + rnd(64 * 64 * 2 * 4)
    # setting partition_tokens alone selects the partition schedule
    n = pa.pa_decode_workspace_bytes(1, 16, 8, 128, 72, 16, pa.make_opts("mfma", 64))
    assert n == HDR + rnd(1 * 16 * 18 * 128 * 4) + rnd(1 * 16 * 18 * 4)
    assert pa.pa_decode_workspace_bytes(1, 15, 8, 128, 4, 32, None) == 0
    # fitted partitions: the fixed schedule's size T (here 4096 * 64 groups /
    # 256 = 1024 tokens) is the largest the device may pick, max(256, T / 4)
    # = 256 the smallest, so the partial slots cover 4096 / 256 = 16
    # partitions; one more 256-byte slot holds the size picked, then the
    # workgroups' hints
    n = pa.pa_decode_workspace_bytes(32, 8, 2, 256, 128, 32, pa.make_opts("mfma", 0, "fitted"))
    assert n == HDR + rnd(32 * 8 * 16 * 256 * 4) + rnd(32 * 8 * 16 * 4) + 256 + 1024 * 16


def test_stats_roundtrip():
    pa.pa_reset_stats()
    s = pa.pa_get_stats()
    assert s["calls"] == 0 and s["valu_launches"] == 0
    assert set(s) == {"calls", "valu_launches", "mfma_launches", "split_calls", "merge_launches",
                      "last_partition_tokens", "last_num_partitions", "last_variant",
                      "balanced_calls", "last_schedule", "append_launches", "prefill_launches",
                      "fused_calls"}


# ------------------------------------------------------------------ KV-cache append
def append_args(B=3, Hkv=4, D=128, P=16, NP=8, maxblk=4):
    kn = torch.zeros(B, Hkv, D, dtype=torch.bfloat16)
    vn = torch.zeros(B, Hkv, D, dtype=torch.bfloat16)
    k = torch.zeros(NP, P, Hkv, D, dtype=torch.bfloat16)
    v = torch.zeros(NP, P, Hkv, D, dtype=torch.bfloat16)
    bt = torch.zeros(B, maxblk, dtype=torch.int32)
    ctx = torch.ones(B, dtype=torch.int32)
    return [kn, vn, k, v, bt, ctx], (Hkv, D, P)


def call_append(ts, dims):
    T = _binding.tensor_desc
    return _binding.LIB.pa_cache_append(*[T(t) if t is not None else None for t in ts], *dims, None)


@pytest.mark.parametrize("mutate,code", [
    (lambda ts, d: (ts.__setitem__(0, ts[0].float()), d), pa.PA_EINVAL),
    (lambda ts, d: (ts.__setitem__(1, torch.zeros(3, 4, 64, dtype=torch.bfloat16)), d), pa.PA_EINVAL),
    (lambda ts, d: (ts.__setitem__(3, torch.zeros(8, 16, 4, 64, dtype=torch.bfloat16)), d), pa.PA_EINVAL),
    (lambda ts, d: (ts.__setitem__(4, torch.zeros(2, 4, dtype=torch.int32)), d), pa.PA_EINVAL),
    (lambda ts, d: (ts.__setitem__(5, torch.ones(2, dtype=torch.int32)), d), pa.PA_EINVAL),
    (lambda ts, d: (ts.__setitem__(2, None), d), pa.PA_EINVAL),
])
def test_append_rejects_bad_arguments(mutate, code):
    ts, dims = append_args()
    mutate(ts, dims)
    assert call_append(ts, dims) == code
    assert pa.last_error() != ""


def test_append_geometry_and_alignment():
    ts, dims = append_args(D=12)
    assert call_append(ts, dims) == pa.PA_ENOTSUP        # rows must be whole 16-byte chunks
    ts, dims = append_args()
    big = torch.zeros(3 * 4 * 128 + 1, dtype=torch.bfloat16)
    ts[0] = big[1:].view(3, 4, 128)
    assert call_append(ts, dims) == pa.PA_EALIGN
    ts, dims = append_args()
    assert call_append(ts, (4, 128, 32)) == pa.PA_EINVAL  # page_size does not match the pool


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a host without a GPU")
def test_valid_append_without_a_device_is_enodev():
    ts, dims = append_args()
    assert call_append(ts, dims) == pa.PA_ENODEV
    ts, dims = append_args(B=0)
    assert call_append(ts, dims) == pa.PA_OK             # nothing to write


def test_missing_library_fails_loudly_at_first_use(monkeypatch, tmp_path):
    """Importing the package never needs the library (so it can be built);
    the first call through the binding raises ImportError when it is absent."""
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "libpa_decode.so"))
    monkeypatch.setattr(_binding._Library, "_lib", None)
    with pytest.raises(ImportError):
        pa.version()


# ------------------------------------------------------------------ several queries per sequence
def prefill_args(R=6, B=2, Hq=16, Hkv=8, D=128, P=16, NP=8, maxblk=4, kv=torch.bfloat16):
    q = torch.zeros(R, Hq, D, dtype=torch.bfloat16)
    k = torch.zeros(NP, P, Hkv, D, dtype=kv)
    v = torch.zeros(NP, P, Hkv, D, dtype=kv)
    bt = torch.zeros(B, maxblk, dtype=torch.int32)
    ctx = torch.full((B,), 10, dtype=torch.int32)
    qs = torch.tensor([0, 4, R][:B + 1] if B == 2 else list(range(B)) + [R], dtype=torch.int32)
    out = torch.zeros(R, Hq, D, dtype=torch.bfloat16)
    return [q, k, v, bt, ctx, qs], out, (Hq, Hkv, D, P)


def call_prefill(ts, out, dims, opts=None, scale=0.1):
    T = _binding.tensor_desc
    return _binding.LIB.pa_prefill(*[T(t) if t is not None else None for t in ts], scale, *dims, T(out),
                                   None, opts, None, 0)


def test_prefill_validation():
    ts, out, dims = prefill_args()
    if not torch.cuda.is_available():
        assert call_prefill(ts, out, dims) == pa.PA_ENODEV        # valid, no device here
    bad = list(ts); bad[5] = torch.tensor([0, 6], dtype=torch.int32)   # needs B + 1 entries
    assert call_prefill(bad, out, dims) == pa.PA_EINVAL
    assert call_prefill(ts, torch.zeros(5, 16, 128, dtype=torch.bfloat16), dims) == pa.PA_EINVAL
    ts2, out2, dims2 = prefill_args(kv=torch.float32)
    assert call_prefill(ts2, out2, dims2) == pa.PA_ENOTSUP      # fp32 cache: no MFMA path
    ts3, out3, dims3 = prefill_args(Hq=16, Hkv=16, D=512)
    if not torch.cuda.is_available():
        assert call_prefill(ts3, out3, dims3) == pa.PA_ENODEV   # head_dim 512: per-block kernel
    assert call_prefill(ts3, out3, dims3, pa.make_opts("auto", 0, "staged")) == pa.PA_ENOTSUP
    ts5, out5, dims5 = prefill_args(D=64)
    assert call_prefill(ts5, out5, dims5) == pa.PA_ENOTSUP
    assert call_prefill(ts, out, dims, pa.make_opts("valu")) == pa.PA_ENOTSUP
    assert call_prefill(ts, out, dims, pa.make_opts("auto", 0, "balanced")) == pa.PA_ENOTSUP
    assert call_prefill(ts, out, dims, pa.make_opts(window=-2)) == pa.PA_EINVAL
    assert call_prefill(ts, out, dims, pa.make_opts("auto", 64, "staged")) == pa.PA_EINVAL   # no partitions
    assert call_prefill(ts, out, dims, pa.make_opts("auto", 0, "fitted")) == pa.PA_ENOTSUP
    assert call_prefill(ts, out, dims, pa.make_opts("auto", 0, 5)) == pa.PA_EINVAL
    ts4, out4, dims4 = prefill_args(R=0, B=2)
    ts4[5] = torch.zeros(3, dtype=torch.int32)
    assert call_prefill(ts4, out4, dims4) == pa.PA_OK           # no rows: nothing to do


def test_prefill_workspace_bytes():
    rnd = lambda x: (x + 255) // 256 * 256
    # 4 sequences x 1 query (decode-like): 4 + 4 slots x 8 KV heads = 64 blocks
    # -> split: T = clamp(1024 * 64 / 256 = 256) = 256 -> 4 partitions
    n = pa.pa_prefill_workspace_bytes(4, 4, 16, 8, 128, 64, 16, None)
    parts = 4
    assert n == pa.PA_WORKSPACE_ZERO_BYTES + rnd(4 * 16 * parts * 128 * 4) + rnd(4 * 16 * parts * 4)
    # many query rows: enough blocks, no split
    assert pa.pa_prefill_workspace_bytes(4096, 4, 16, 8, 128, 64, 16, None) == 0
    assert pa.pa_prefill_workspace_bytes(4, 4, 12, 8, 128, 64, 16, None) == 0   # Hq % Hkv
    # the staged schedule never splits; the same call on partitions does
    staged = pa.make_opts("auto", 0, "staged")
    parts = pa.make_opts("auto", 0, "partitions")
    assert pa.pa_prefill_workspace_bytes(64, 4, 16, 8, 128, 64, 16, staged) == 0
    assert pa.pa_prefill_workspace_bytes(64, 4, 16, 8, 128, 64, 16, parts) > 0
    # automatic: 64 rows over 4 sequences (qt = 8: two blocks each) but only
    # (64 / 32 + 4) x 8 = 48 staged workgroups -> partitions
    assert pa.pa_prefill_workspace_bytes(64, 4, 16, 8, 128, 64, 16, None) == \
        pa.pa_prefill_workspace_bytes(64, 4, 16, 8, 128, 64, 16, parts)
