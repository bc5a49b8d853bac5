"""Device-code check on the CPU: MFMA operands written by inline assembly.

An MFMA on gfx950 may read a vector register only two wait states after a vector ALU
instruction has written it. hipcc inserts those waits after its own instructions, but
not after instructions inside inline assembly, which it does not inspect. The kernels
that build MFMA operands in inline assembly therefore end each such block with the
waits themselves. This test compiles every kernel source that holds inline assembly to
gfx950 assembly, with the library's own flags, and checks each MFMA: for every source
register last written inside an inline-assembly block, at least two wait states
(instructions issued in between, an `s_nop N` counting N + 1) separate that write from
the MFMA. The walk follows the text in order, across labels (the fall-through path).
"""
import os
import re
import shutil
import subprocess

import pytest

from unified_block_sparse_amd import build as ubs_build

HIPCC = ubs_build.HIPCC
NEEDED_WAIT_STATES = 2

pytestmark = pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                                reason="hipcc not available")


def _regs(tok: str) -> set:
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _operands(line: str) -> list:
    parts = line.split(None, 1)
    if len(parts) < 2:
        return []
    return [t.strip() for t in parts[1].split(",")]


def short_asm_to_mfma_gaps(asm_text: str) -> list:
    """(function, line, register, wait states) for every MFMA source register written by
    inline assembly fewer than NEEDED_WAIT_STATES wait states before the MFMA."""
    found = []
    func = None
    in_asm = False
    last_asm_write = {}   # register -> wait states issued since that write
    for lineno, raw in enumerate(asm_text.splitlines(), 1):
        line = raw.split(";", 1)[0].strip() if not raw.strip().startswith(";;#ASM") else raw.strip()
        if line.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if line.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = re.match(r"^([A-Za-z_.$][\w.$]*):", line)
        if m:
            if not m.group(1).startswith("."):
                func, last_asm_write = m.group(1), {}
            continue
        if not line or line.startswith("."):
            continue
        op = line.split()[0]
        ops = _operands(line)
        if op.startswith("v_mfma"):
            for tok in ops[1:4]:
                for r in _regs(tok):
                    w = last_asm_write.get(r)
                    if w is not None and w < NEEDED_WAIT_STATES:
                        found.append((func, lineno, r, w))
        issued = int(ops[0], 0) + 1 if op == "s_nop" and ops else 1
        for r in list(last_asm_write):
            last_asm_write[r] += issued
        dst = _regs(ops[0]) if ops else set()
        for r in dst:
            if in_asm:
                last_asm_write[r] = 0
            else:
                last_asm_write.pop(r, None)
    return found


def _sources_with_inline_asm():
    out = []
    for src in ubs_build.sources():
        text = open(src).read()
        if re.search(r"\basm\s*(volatile\s*)?\(\s*\"[^\"]", text):
            out.append(src)
    return out


def test_checker_flags_a_short_gap():
    """The checker itself: a write one instruction before the MFMA is flagged, two (or an
    s_nop 1 in the block) are not."""
    head = "k:\n;;#ASMSTART\n\tv_and_or_b32 v3, v0, s4, v5\n;;#ASMEND\n"
    mfma = "\tv_mfma_f32_16x16x32_f16 v[10:13], v[0:3], v[4:7], v[10:13]\n"
    assert short_asm_to_mfma_gaps(head + "\tv_mov_b32_e32 v20, v21\n" + mfma) == [("k", 6, ("v", 3), 1)]
    assert short_asm_to_mfma_gaps(head + "\tv_mov_b32_e32 v20, v21\n\ts_nop 0\n" + mfma) == []
    fenced = "k:\n;;#ASMSTART\n\tv_and_or_b32 v3, v0, s4, v5\n\ts_nop 1\n;;#ASMEND\n"
    assert short_asm_to_mfma_gaps(fenced + mfma) == []
    # a compiler-written definition after the assembly clears it (the compiler waits for
    # its own writes)
    assert short_asm_to_mfma_gaps(head + "\tv_mov_b32_e32 v3, v21\n" + mfma) == []


@pytest.mark.parametrize("src", _sources_with_inline_asm(), ids=os.path.basename)
def test_mfma_operands_from_inline_asm_have_their_wait_states(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, *ubs_build.FLAGS, *ubs_build.EXTRA_FLAGS.get(os.path.basename(src), []),
           "--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    gaps = short_asm_to_mfma_gaps(out.read_text())
    assert not gaps, f"{len(gaps)} MFMA operand(s) read too soon after inline assembly wrote them: {gaps[:5]}"
