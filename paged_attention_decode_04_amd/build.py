"""Build ``libpa_decode.so`` (gfx950) in place with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 VALU
instructions disabled in the device code, then linked into one shared
library next to this file.  The streaming-read probes (``include/pa_probe.h``,
measurement aids of the benchmark) go to a library of their own,
``libpa_probe.so``.  Usage: ``python -m paged_attention_decode_04_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpa_decode.so")
SOURCES = ["pa_api.hip", "pa_valu.hip", "pa_mfma.hip", "pa_append.hip", "pa_prefill.hip"]
PROBE_SOURCES = ["pa_probe.hip"]
PROBE_LIB = os.path.join(HERE, "libpa_probe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the online-softmax rescale touches
    # them with VALU ops, and the AGPR form costs a copy in and out each time.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]
# Per-source additions.  The several-query kernels assume no NaN in their
# arithmetic (no input NaN reaches it: rows outside a sequence are never
# loaded), so fmax needs no operand canonicalisation (one v_max per element
# instead of two in the VALU-bound softmax).  Infinities keep their meaning.
SOURCE_FLAGS = {"pa_prefill.hip": ["-fno-honor-nans"]}


def flags(src: str) -> list[str]:
    return [*CFLAGS, *SOURCE_FLAGS.get(src, [])]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *flags(src), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stderr or "").splitlines() if noise not in ln and "(ignoring feature)" not in ln]
    if any(m.strip() for m in msgs):
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
