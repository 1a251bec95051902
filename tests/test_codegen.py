"""Code-generation guard for the gfx950 kernels (CPU only: hipcc cross-compiles).

Cross-lane moves (permlane swaps, DPP) read other lanes' registers, and the
transposing LDS reads (ds_read_b64_tr_b16) gather through other lanes'
addresses; under a partial exec mask they read inactive lanes and return
stale data.  The MFMA
kernels therefore evaluate every cross-lane move unconditionally.  This test
compiles the kernels to gfx950 assembly and checks, by a data-flow pass over
each kernel's control-flow graph, that no permlane or DPP instruction can run
while an exec-masking region is open.

Exec save points nest: ``s_and_saveexec_b64 sX`` (an if), ``s_andn2_b64
exec, exec, sX`` (lanes leaving a divergent loop) and the split form
``s_mov_b64 sX, exec`` followed by any other write of exec open region sX
inside the current one; ``s_or_b64 exec, exec, sX`` (or ``s_mov_b64 exec,
sX``) restores the mask saved in sX, closing sX and every region opened
inside it; ``s_or_saveexec_b64 sY, sX`` (an else) closes sX and opens sY.
Each block's entry holds the set of save-point stacks that reach it along
some path.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_attention_decode_04_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

_PAIR = r"(s\[\d+:\d+\])"
_LABEL = re.compile(r"^(\.LBB\w+):")


def _blocks(body):
    """Split a kernel body into basic blocks: [(label, [instr...], succ_labels)]."""
    blocks, cur, label = [], [], "<entry>"
    lines = [l.split(";")[0].strip() for l in body.splitlines()]
    for t in lines:
        if not t or t.startswith("."):
            m = _LABEL.match(t)
            if m:
                blocks.append([label, cur])
                label, cur = m.group(1), []
            continue
        cur.append(t)
        if t.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append([label, cur])
            label, cur = f"<after:{len(blocks)}>", []
    blocks.append([label, cur])
    out = []
    for i, (lab, ins) in enumerate(blocks):
        nxt = blocks[i + 1][0] if i + 1 < len(blocks) else None
        last = ins[-1] if ins else ""
        succ = []
        if last.startswith("s_branch"):
            succ = [last.split()[1]]
        elif last.startswith("s_cbranch"):
            succ = [last.split()[1]] + ([nxt] if nxt else [])
        elif last.startswith(("s_endpgm", "s_setpc")):
            succ = []
        elif nxt:
            succ = [nxt]
        out.append((lab, ins, succ))
    return out


def _step(stack, t):
    """Apply one instruction to a stack of exec save points, innermost last.

    Entries are (sgpr_pair, narrowed): the pair holds a saved exec mask (or a
    loop's exit mask) and narrowed says exec has been cut down since.
    """
    def cut(pair):                      # restore pair: it and all inner save points end
        for k, (pp, _) in enumerate(stack):
            if pp == pair:
                return stack[:k]
        return stack

    def narrow():
        if stack:
            return stack[:-1] + ((stack[-1][0], True),)
        return (("<exec>", True),)

    m = re.match(r"s_and_saveexec_b64 " + _PAIR, t) or re.match(r"s_andn2_saveexec_b64 " + _PAIR, t)
    if m:
        return cut(m.group(1)) + ((m.group(1), True),)
    m = re.match(r"s_andn2_b64 exec, exec, " + _PAIR, t)       # lanes leaving a loop
    if m:
        return cut(m.group(1)) + ((m.group(1), True),)
    m = re.match(r"s_or_saveexec_b64 " + _PAIR + ", " + _PAIR, t)
    if m:
        return cut(m.group(2)) + ((m.group(1), True),)
    m = re.match(r"s_mov_b64 " + _PAIR + ", exec$", t)         # split save
    if m:
        return cut(m.group(1)) + ((m.group(1), False),)
    m = re.match(r"s_(?:or|mov)_b64 exec, (?:exec, )?" + _PAIR + "$", t)
    if m and any(pp == m.group(1) for pp, _ in stack):       # restore
        return cut(m.group(1))
    if re.match(r"s_mov_b64 exec, -1$", t):
        return ()
    if re.match(r"s_\w+_b64 exec, ", t):                      # any other exec write narrows
        return narrow()
    return stack


def cross_lane_under_divergence(body):
    """Cross-lane instructions that may execute inside an open exec region."""
    blocks = _blocks(body)
    index = {lab: i for i, (lab, _, _) in enumerate(blocks)}
    entry = [frozenset({()}) if i == 0 else frozenset() for i in range(len(blocks))]
    bad = set()
    work = [0]
    while work:
        i = work.pop()
        lab, ins, succ = blocks[i]
        states = set(entry[i])
        for t in ins:
            if any(nar for st in states for _, nar in st) and (
                    "permlane" in t or "_dpp" in t or " row_" in t or "_tr_b" in t):
                bad.add(t)
            states = {_step(st, t) for st in states}
        for s in succ:
            j = index.get(s)
            if j is None:
                continue
            new = entry[j] | frozenset(states)
            if new != entry[j]:
                entry[j] = new
                work.append(j)
    return sorted(bad)


def test_analysis_follows_loop_layout():
    # A region opened at the bottom of a loop and closed in a block laid out
    # above it (the loop latch) is closed on the path that reaches the DPP.
    body = """
    s_branch .LBB0_2
.LBB0_1:
    s_or_b64 exec, exec, s[4:5]
    s_cbranch_scc1 .LBB0_3
.LBB0_2:
    v_mov_b32 v0, v1
    s_and_saveexec_b64 s[4:5], vcc
    s_cbranch_execz .LBB0_1
    v_mov_b32 v2, v3
    s_branch .LBB0_1
.LBB0_3:
    v_mov_b32_dpp v1, v0 row_ror:8 row_mask:0xf bank_mask:0xf
    s_endpgm
"""
    assert cross_lane_under_divergence(body) == []


def test_analysis_catches_cross_lane_op_in_region():
    body = """
    s_and_saveexec_b64 s[4:5], vcc
    s_cbranch_execz .LBB0_1
    v_permlane32_swap_b32_e32 v1, v2
.LBB0_1:
    s_or_b64 exec, exec, s[4:5]
    s_endpgm
"""
    assert cross_lane_under_divergence(body) == ["v_permlane32_swap_b32_e32 v1, v2"]
    assert cross_lane_under_divergence(body.replace("v_permlane32_swap_b32_e32 v1, v2",
                                                    "ds_read_b64_tr_b16 v[1:2], v3")) == ["ds_read_b64_tr_b16 v[1:2], v3"]
    # the same through an else arm, and inside a divergent loop
    body_else = """
    s_and_saveexec_b64 s[4:5], vcc
    s_xor_b64 s[4:5], exec, s[4:5]
    s_cbranch_execz .LBB0_1
    v_mov_b32 v1, v2
.LBB0_1:
    s_or_saveexec_b64 s[6:7], s[4:5]
    v_mov_b32_dpp v1, v0 row_ror:8 row_mask:0xf bank_mask:0xf
    s_or_b64 exec, exec, s[6:7]
    s_endpgm
"""
    assert len(cross_lane_under_divergence(body_else)) == 1
    body_loop = """
.LBB0_1:
    v_mov_b32_dpp v1, v0 row_ror:8 row_mask:0xf bank_mask:0xf
    s_or_b64 s[4:5], vcc, s[4:5]
    s_andn2_b64 exec, exec, s[4:5]
    s_cbranch_execnz .LBB0_1
    s_or_b64 exec, exec, s[4:5]
    s_endpgm
"""
    assert len(cross_lane_under_divergence(body_loop)) == 1
    # the split save form: exec saved with a move, narrowed with another
    body_split = """
    s_mov_b64 s[10:11], exec
    s_and_b64 s[6:7], s[10:11], s[6:7]
    s_mov_b64 exec, s[6:7]
    s_cbranch_execz .LBB0_1
    v_permlane16_swap_b32_e32 v1, v2
.LBB0_1:
    s_or_b64 exec, exec, s[10:11]
    v_permlane32_swap_b32_e32 v3, v4
    s_endpgm
"""
    assert cross_lane_under_divergence(body_split) == ["v_permlane16_swap_b32_e32 v1, v2"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", ["pa_mfma.hip", "pa_valu.hip", "pa_prefill.hip", "pa_append.hip"])
def test_no_cross_lane_ops_under_divergent_exec(src, tmp_path):
    from paged_attention_decode_04_amd import build
    out = tmp_path / "k.s"
    cmd = [HIPCC, *build.flags(src), "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    asm = out.read_text()
    kernels = re.findall(r"^(_ZN2pa\w+):", asm, flags=re.M)
    assert kernels
    for name in kernels:
        start = asm.find(name + ":")
        body = asm[start + len(name) + 1:asm.find(".Lfunc_end", start)]
        bad = cross_lane_under_divergence(body)
        assert not bad, f"{name}: cross-lane op under a partial exec mask: {bad[:3]}"
