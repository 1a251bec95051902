"""The benchmark's streaming-read probes (libpa_probe.so) run on the GPU:
both patterns over real workloads, nothing written but by chance (the sink
stays zero), the rows they read within the pools."""
import pytest
import torch

from paged_attention_decode_04_amd import probe
from workloads import make_inputs, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _dev(gpu):
    yield


def test_contiguous_probe_runs():
    buf = torch.ones(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    for n_wg in (1, 256, 1024):
        probe.read_contiguous(buf, n_wg, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


@pytest.mark.parametrize("name", ["tiny", "batch16", "hd256_gqa4"])
def test_paged_probe_runs(name):
    d = to_device(make_inputs(name, seed=0))
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    desc = probe.paged_desc(d.k[0], d.v[0], d.block_tables, d.context_lens)
    for n_wg in (1, 3, 256, 512):
        probe.read_paged(desc, n_wg, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


def test_issue_probe_runs():
    """Every mode of the issue-rate probe runs (few rounds, one and four waves
    per SIMD); it writes nothing but by chance."""
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    modes = probe.issue_modes()
    assert len(modes) >= 2 and all(nm + nv > 0 for nm, nv, _ in modes)
    for i in range(len(modes)):
        for n_wg in (256, 1024):
            probe.issue(i, n_wg, 64, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
