"""Static check of the hand-placed MFMA hazards in the compiled gfx950 code.

MFMAs whose accumulators live in AGPRs are written as inline asm
(`common.hpp: mfma32_agpr`), so the compiler's hazard recognizer does not see
them. The hand-scheduled dK/dV step issues them without the `s_nop 1` that
would cover a VALU-written operand, because their operands are LDS reads or
VALU results produced well before. This test compiles the kernel sources to
assembly (hipcc cross-compiles without a GPU) and scans every such MFMA:

* no VALU instruction may write its A or B operand registers within the 2
  wait states before it (the rule the compiler applies to its own MFMAs: a
  VALU-written source needs 2 wait states; each instruction counts as one,
  `s_nop N` as N + 1);
* no VALU instruction may write the AGPRs of its accumulator within those 2
  wait states;
* no MFMA may write its A or B operand registers within 18 wait states
  before it (an MFMA result read as a source);
* no label may fall inside the window (a branch could enter with unknown
  history).

The scanner itself is pinned on small hand-written instruction sequences
with and without each hazard.
"""
import os
import re
import shutil
import subprocess

import pytest

from exact_attention_71_amd import build as b

VALU_WINDOW = 2
MFMA_WINDOW = 18
_REG = re.compile(r"^([va])(?:\[(\d+):(\d+)\]|(\d+))$")


def _regs(tok):
    """('v' | 'a', first, last) for a register operand token, else None."""
    m = _REG.match(tok.strip().rstrip(","))
    if not m:
        return None
    if m.group(2) is not None:
        return m.group(1), int(m.group(2)), int(m.group(3))
    return m.group(1), int(m.group(4)), int(m.group(4))


def _overlap(x, y):
    return x is not None and y is not None and x[0] == y[0] and x[1] <= y[2] and y[1] <= x[2]


def _parse(lines):
    """Instruction stream: ('label', name) or ('insn', opcode, operand tokens)."""
    out = []
    for raw in lines:
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":"):
            out.append(("label", line[:-1]))
            continue
        if line.startswith("."):
            continue
        parts = line.split(None, 1)
        ops = [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []
        out.append(("insn", parts[0], ops))
    return out


def _wait_states(entry):
    op = entry[1]
    if op == "s_nop":
        return int(entry[2][0], 0) + 1
    return 1


def scan(lines):
    """Hazards of AGPR-accumulating MFMAs in an assembly listing: a list of
    (index, reason) pairs, empty when every MFMA is covered."""
    stream = _parse(lines)
    bad = []
    for i, e in enumerate(stream):
        if e[0] != "insn" or not e[1].startswith("v_mfma") or len(e[2]) < 4:
            continue
        dst = _regs(e[2][0])
        if dst is None or dst[0] != "a":
            continue
        srcs = [_regs(t) for t in e[2][1:3]]
        acc = _regs(e[2][3]) if _regs(e[2][3]) is not None else dst
        ws = 0
        j = i - 1
        while j >= 0 and ws < MFMA_WINDOW:
            p = stream[j]
            if p[0] == "label":
                if ws < VALU_WINDOW:
                    bad.append((i, f"label {p[1]} within {ws} wait states"))
                break
            op, ops = p[1], p[2]
            w = _regs(ops[0]) if ops else None
            if op.startswith("v_mfma"):
                if any(_overlap(w, s) for s in srcs):
                    bad.append((i, f"{op} writes an operand {ws} wait states before"))
            elif op.startswith("v_") and ws < VALU_WINDOW:
                if any(_overlap(w, s) for s in srcs):
                    bad.append((i, f"{op} writes an operand {ws} wait states before"))
                if _overlap(w, acc):
                    bad.append((i, f"{op} writes the accumulator {ws} wait states before"))
            ws += _wait_states(p)
            j -= 1
    return bad


def count_agpr_mfma(lines):
    n = 0
    for e in _parse(lines):
        if e[0] == "insn" and e[1].startswith("v_mfma") and e[2]:
            r = _regs(e[2][0])
            n += r is not None and r[0] == "a"
    return n


# ---- pins of the scanner on hand-written sequences -------------------------

SAFE = """
  v_cvt_pk_bf16_f32 v12, v1, v2
  v_sub_f32_e32 v18, v18, v58
  v_mul_f32_e32 v240, v240, v18
  v_mfma_f32_32x32x16_bf16 a[16:31], v[42:45], v[10:13], a[16:31]
"""
VALU_RIGHT_BEFORE = """
  v_mul_f32_e32 v240, v240, v18
  v_cvt_pk_bf16_f32 v12, v1, v2
  v_mfma_f32_32x32x16_bf16 a[16:31], v[42:45], v[10:13], a[16:31]
"""
VALU_ONE_BETWEEN = """
  v_cvt_pk_bf16_f32 v43, v1, v2
  s_waitcnt lgkmcnt(1)
  v_mfma_f32_32x32x16_bf16 a[16:31], v[42:45], v[10:13], a[16:31]
"""
NOP_COVERS = """
  v_cvt_pk_bf16_f32 v12, v1, v2
  s_nop 1
  v_mfma_f32_32x32x16_bf16 a[16:31], v[42:45], v[10:13], a[16:31]
"""
MFMA_RESULT_AS_SOURCE = """
  v_mfma_f32_32x32x16_bf16 v[40:55], v[0:3], v[4:7], 0
  ds_read_b128 v[60:63], v200
  v_add_f32_e32 v100, v101, v102
  v_mfma_f32_32x32x16_bf16 a[16:31], v[42:45], v[10:13], a[16:31]
"""
LABEL_BEFORE = """
  v_add_f32_e32 v100, v101, v102
.LBB1_7:
  v_mfma_f32_32x32x16_bf16 a[16:31], v[42:45], v[10:13], a[16:31]
"""
ACC_WRITTEN = """
  v_accvgpr_write_b32 a20, v3
  v_mfma_f32_32x32x16_bf16 a[16:31], v[42:45], v[10:13], a[16:31]
"""


@pytest.mark.parametrize("text,hazard", [
    (SAFE, False), (VALU_RIGHT_BEFORE, True), (VALU_ONE_BETWEEN, True), (NOP_COVERS, False),
    (MFMA_RESULT_AS_SOURCE, True), (LABEL_BEFORE, True), (ACC_WRITTEN, True)])
def test_scanner_on_hand_written_sequences(text, hazard):
    assert bool(scan(text.splitlines())) == hazard


# ---- the compiled kernels ----------------------------------------------------

def _hipcc_or_skip():
    exe = b._hipcc()
    if not (os.path.exists(exe) or shutil.which(exe)):
        pytest.skip("hipcc not available")
    return exe


@pytest.mark.parametrize("src", ["bwd_dkdv.hip", "bwd.hip"])
def test_compiled_agpr_mfmas_have_no_uncovered_hazard(src, tmp_path):
    exe = _hipcc_or_skip()
    out = tmp_path / (src + ".s")
    cmd = [exe, *b.FLAGS, "-I", os.path.join(b.HERE, "..", "include"), "--cuda-device-only",
           "-S", "-o", str(out), os.path.join(b.CSRC, src)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = out.read_text().splitlines()
    assert count_agpr_mfma(lines) > 0 or src != "bwd_dkdv.hip"
    bad = scan(lines)
    assert not bad, bad[:10]
