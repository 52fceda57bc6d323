"""Wait states around the attention kernel's inline-asm MFMAs (CPU only: compiles to gfx950 assembly).

With two row halves per wave the kernel issues its MFMAs as inline asm, which the compiler's hazard recognizer
does not see through, so the kernel places the required wait states itself.  This test compiles attn.hip to
assembly with the library's own flags and checks every control-flow path of that kernel:
  * an MFMA result is not read or overwritten by another instruction within 12 wait states of the MFMA (the
    count the compiler itself inserts on gfx950 before a VALU read of an 8-pass MFMA result), except by an MFMA
    that accumulates into exactly the same registers;
  * a register written by a VALU instruction is not read by an MFMA within 2 wait states of the write.
A wait state is one instruction, or N + 1 for `s_nop N`.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

KERNEL = "_ZN4ulys12_GLOBAL__N_115attn_fwd_kernelILi128ELb0ELb0ELi2EEEvNS_8AttnArgsE"
RESULT_WAIT, OPERAND_WAIT = 12, 2


def _regs(tok):
    tok = tok.strip()
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _parse(op_line):
    op, _, rest = op_line.partition(" ")
    return op, [x.strip() for x in rest.split(",")] if rest.strip() else []


def _wait(line):
    op, ops = _parse(line)
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def _program(asm_lines):
    """Instructions of one function and the instruction index of each label."""
    ins, labels = [], {}
    for raw in asm_lines:
        t = raw.split(";")[0].strip()
        if not t:
            continue
        m = re.match(r"^(\.LBB\w+):$", t)
        if m:
            labels[m.group(1)] = len(ins)
            continue
        if t.startswith(".") or t.endswith(":"):
            continue
        ins.append(t)
    return ins, labels


def _successors(ins, labels, j):
    op, ops = _parse(ins[j])
    if op == "s_endpgm":
        return []
    if op == "s_branch":
        return [labels[ops[0]]]
    if op.startswith("s_cbranch"):
        return [j + 1, labels[ops[0]]]
    return [j + 1]


def hazards(asm_lines):
    """(kind, mfma line, other line, wait states) for every violation found."""
    ins, labels = _program(asm_lines)
    preds = {j: [] for j in range(len(ins) + 1)}
    for j in range(len(ins)):
        for s in _successors(ins, labels, j):
            preds.setdefault(s, []).append(j)
    found = []
    for i, line in enumerate(ins):
        op, ops = _parse(line)
        if not op.startswith("v_mfma"):
            continue
        dst = _regs(ops[0])
        srcs = set().union(*[_regs(o) for o in ops[1:4]])
        # forwards: nothing touches the result too early
        stack, seen = [(s, 0) for s in _successors(ins, labels, i)], {}
        while stack:
            j, w = stack.pop()
            if j >= len(ins) or w >= RESULT_WAIT or seen.get(j, RESULT_WAIT) <= w:
                continue
            seen[j] = w
            pj, oj = _parse(ins[j])
            if pj.startswith("v_mfma"):
                dj, sj = _regs(oj[0]), _regs(oj[1]) | _regs(oj[2])
                cj = _regs(oj[3]) if len(oj) > 3 else set()
                hit = bool(sj & dst) or ((dj & dst) and dj != dst) or ((cj & dst) and cj != dst)
            elif oj and re.match(r"(v_|ds_|global_|buffer_|flat_)", pj):
                hit = bool(set().union(*[_regs(o) for o in oj]) & dst)
            else:
                hit = False
            if hit:
                found.append(("mfma result", line, ins[j], w))
                continue
            for s in _successors(ins, labels, j):
                stack.append((s, w + _wait(ins[j])))
        # backwards: no VALU write of an operand too close before
        stack, seen = [(p, 0) for p in preds.get(i, [])], {}
        while stack:
            j, w = stack.pop()
            if w >= OPERAND_WAIT or seen.get(j, OPERAND_WAIT) <= w:
                continue
            seen[j] = w
            pj, oj = _parse(ins[j])
            if pj.startswith("v_mfma"):
                continue   # MFMA-to-MFMA dependences are the result rule's business
            if pj.startswith("v_") and oj and _regs(oj[0]) & srcs:
                found.append(("valu operand", line, ins[j], w))
                continue
            for p in preds.get(j, []):
                stack.append((p, w + _wait(ins[j])))
    return found


def test_checker_finds_planted_hazards():
    planted = [
        "v_cvt_pk_bf16_f32 v24, v1, v2",
        "v_mfma_f32_32x32x16_bf16 a[0:15], v[20:23], v[24:27], a[0:15]",   # operand written 1 wait state before
        "s_cbranch_scc1 .LBB0_2",
        "s_nop 7",
        ".LBB0_2:",
        "v_accvgpr_read_b32 v5, a3",                                        # result read 1 wait state after (taken branch)
        "s_endpgm",
    ]
    kinds = sorted(k for k, *_ in hazards(planted))
    assert kinds == ["mfma result", "valu operand"]
    clean = ["v_cvt_pk_bf16_f32 v24, v1, v2", "s_nop 1",
             "v_mfma_f32_32x32x16_bf16 a[0:15], v[20:23], v[24:27], a[0:15]",
             "v_mfma_f32_32x32x16_bf16 a[0:15], v[28:31], v[24:27], a[0:15]",   # accumulation chain: allowed
             "s_nop 7", "s_nop 3", "v_accvgpr_read_b32 v5, a3", "s_endpgm"]
    assert hazards(clean) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to compile the kernel to assembly")
def test_two_row_half_kernel_wait_states(tmp_path):
    from ulysses_sequence_attention_amd import build as B
    src = os.path.join(ROOT, "ulysses_sequence_attention_amd", "csrc", "attn.hip")
    out = tmp_path / "attn.s"
    flags = [f for f in B.FLAGS if f not in ("-fPIC",)]
    cmd = [B.HIPCC, *flags, *B.SOURCE_FLAGS.get("attn.hip", []), "-I", os.path.dirname(src),
           "--cuda-device-only", "-S", "-o", str(out), src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = out.read_text().split("\n")
    start = next(i for i, l in enumerate(lines) if l.startswith(KERNEL + ":"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    body = lines[start + 1:end]
    assert sum(1 for l in body if l.strip().startswith("v_mfma")) > 100
    found = hazards(body)
    assert found == [], found[:5]
