"""Seeded input generator: determinism, block-table structure, stated sizes."""
import numpy as np
import pytest

import workloads
from workloads import WORKLOADS, kv_bytes, make_inputs, make_layout


def test_same_seed_same_bytes():
    a = make_inputs("tiny", seed=0)
    b = make_inputs("tiny", seed=0)
    c = make_inputs("tiny", seed=1)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert not np.array_equal(a.q, c.q)


def test_tiny_layout_is_a_page_permutation():
    inp = make_inputs("tiny")
    lay = inp.layout
    assert list(lay.context_lens) == [1, 31, 33, 100]
    assert lay.num_pages == 16
    used = inp.block_tables[inp.block_tables >= 0]
    assert used.size == 1 + 1 + 2 + 4 and len(set(used.tolist())) == used.size
    assert used.min() >= 0 and used.max() < 16
    assert inp.block_tables.shape == (4, 4)
    # stated algorithmic KV bytes: 165 tokens * 8 heads * 128 * 4 B
    assert kv_bytes(inp.w, lay.context_lens) == 675_840


@pytest.mark.parametrize("name,sum_l", [("batch16", 17_416), ("hd256_gqa4", 76_827),
                                        ("long_ctx_gqa8", 1_326_175)])
def test_seed0_lengths(name, sum_l):
    w = WORKLOADS[name]
    lay = make_layout(w, np.random.default_rng(0))
    assert lay.total_tokens == sum_l
    lo, hi = w.ctx_range
    assert lay.context_lens.min() >= lo and lay.context_lens.max() <= hi
    # pool holds exactly the needed pages, each used once
    assert lay.used_pages.size == lay.num_pages
    assert np.array_equal(np.sort(lay.used_pages), np.arange(lay.num_pages))


def test_values_are_rounded_normals():
    inp = make_inputs("batch16")
    f = (inp.k.astype(np.uint32) << 16).view(np.float32)
    used = f[0, inp.layout.used_pages]
    assert abs(float(used.mean())) < 0.01 and abs(float(used.std()) - 1.0) < 0.01


def test_spikes_scale_k_rows_by_four():
    w = WORKLOADS["hd256_gqa4"]
    plain = workloads.Workload(**{**w.__dict__, "spike_frac": 0.0})
    a = make_inputs(w)
    # same draws up to the spike step: non-spiked K rows are identical
    b = make_inputs(plain)
    spikes = a.layout.spike_tokens
    assert 0.005 < spikes.mean() < 0.015
    fa = (a.k.astype(np.uint32) << 16).view(np.float32)
    fb = (b.k.astype(np.uint32) << 16).view(np.float32)
    pg, sl = workloads._token_slots(w, a.layout)
    assert np.array_equal(fa[0, pg[spikes], sl[spikes]], 4 * fb[0, pg[spikes], sl[spikes]])
    assert np.array_equal(fa[0, pg[~spikes], sl[~spikes]], fb[0, pg[~spikes], sl[~spikes]])


def test_poison_marks_only_unread_data():
    inp = make_inputs("tiny", poison_unused=True)
    clean = make_inputs("tiny")
    lay = inp.layout
    P = inp.w.page_size
    for b, L in enumerate(lay.context_lens):
        for t in range(L):
            pg = inp.block_tables[b, t // P]
            assert np.array_equal(inp.k[0, pg, t % P], clean.k[0, pg, t % P])
    assert np.sum(inp.k == workloads.BF16_NAN) > 0
    assert np.array_equal(inp.q, clean.q)


def test_single_seq_has_28_layers_of_32_calls():
    w = WORKLOADS["single_seq"]
    assert w.calls == 896 and w.layers == 28 and w.tokens == 32
    assert kv_bytes(w, [1152]) == 4_718_592
