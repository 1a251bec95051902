"""Code-generation guard for the gfx950 kernels (CPU only: hipcc cross-compiles).

Cross-lane moves (permlane swaps, DPP) read other lanes' registers; under a
partial exec mask they read inactive lanes and return stale data.  The MFMA
kernel therefore evaluates every cross-lane move unconditionally.  This test
compiles the kernels to gfx950 assembly and checks that no permlane or DPP
instruction sits inside an exec-masked (divergent) region.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_attention_decode_04_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", ["pa_mfma.hip", "pa_valu.hip"])
def test_no_cross_lane_ops_under_divergent_exec(src, tmp_path):
    from paged_attention_decode_04_amd import build
    out = tmp_path / "k.s"
    cmd = [HIPCC, *build.CFLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    asm = out.read_text()
    kernels = re.findall(r"^(_ZN2pa\w+):", asm, flags=re.M)
    assert kernels
    for name in kernels:
        body = asm[asm.find(name + ":"):asm.find(".Lfunc_end", asm.find(name + ":"))]
        # Track regions opened by s_and_saveexec (keyed by the saved SGPR pair)
        # until their restore; a path ends at s_endpgm.
        open_regions, bad = set(), []
        for line in body.splitlines():
            t = line.strip()
            m = re.match(r"s_and_saveexec_b64 (s\[\d+:\d+\])", t)
            if m:
                open_regions.add(m.group(1))
                continue
            m = re.match(r"s_or_b64 exec, exec, (s\[\d+:\d+\])", t)
            if m:
                open_regions.discard(m.group(1))
                continue
            if t.startswith("s_endpgm"):
                open_regions.clear()
                continue
            if open_regions and ("permlane" in t or "_dpp" in t or " row_" in t):
                bad.append(t)
        assert not bad, f"{name}: cross-lane op under a partial exec mask: {bad[:3]}"
