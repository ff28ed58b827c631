"""The attention kernel's S^T accumulation runs as a chain of MFMAs written
in inline asm (to keep its accumulator out of the AGPRs that hold O).  The
compiler's hazard tracking does not see into asm: it takes an asm MFMA's
result as ready, and its sources as free, once the instruction issues.  On
the hardware the result lands many cycles later and C is read late in the
instruction, so any instruction the compiler places between a link of the
chain and its wait (a register copy, a reuse of a dead source) reads
partial sums or corrupts C.

This test compiles the kernel source for gfx950 to assembly with the
library's own flags and checks every variant: between an asm MFMA's issue
and the asm wait that ends its chain, no other instruction reads or writes
its destination, nor writes its C operand.  The check runs on the CPU."""
import os
import re
import subprocess

import pytest

from sparse_attention_18_amd import build

SRC = os.path.join(build.CSRC, "sparse_attn.hip")


def _regs(tok):
    tok = tok.strip()
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


_NO_DEST = ("ds_write", "global_store", "buffer_store", "scratch_store", "s_")


def chain_hazards(body):
    """Lines of one kernel's assembly -> the offending instructions."""
    inflight, in_asm, bad = [], False, []
    for line in body:
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        t = line.split(";")[0].strip()
        if not t:
            continue
        mn, _, rest = t.partition(" ")
        args = [a.strip() for a in rest.split(",")] if rest else []
        if in_asm and mn == "s_nop":
            if int(args[0], 0) >= 15:      # the chain's wait (two of them)
                inflight = []
            continue
        if in_asm and mn.startswith("v_mfma"):
            dst = _regs(args[0])
            c = _regs(args[3]) if len(args) > 3 else set()
            # a link whose C is an earlier link's result consumes that link
            inflight = [x for x in inflight if x[0] != c] + [(dst, c)]
            continue
        if not inflight:
            continue
        touched = set().union(*(_regs(a) for a in args)) if args else set()
        written = _regs(args[0]) if args and not mn.startswith(_NO_DEST) else set()
        if any(touched & d or written & c for d, c in inflight):
            bad.append(t)
    return bad


def _kernels(asm):
    """(name, lines) of each attention kernel, up to its end-of-function label
    (blocks after an early s_endpgm belong to it too)."""
    lines = asm.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_Z\S*mla_sparse_attn_kernel\S*:", l)]
    for st in starts:
        en = next(i for i in range(st, len(lines)) if lines[i].startswith(".Lfunc_end"))
        yield lines[st].split(":")[0], lines[st:en]


def test_scanner_flags_a_copy_inside_a_chain():
    """The scanner itself: a copy of an accumulator between two links, and a
    write to the last link's C before its wait, are both found; the same
    chain without them is clean."""
    chain = [";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 v[16:31], v[0:3], v[40:43], v[16:31]", ";;#ASMEND"]
    wait = [";;#ASMSTART", "s_nop 15", "s_nop 15", ";;#ASMEND"]
    last = [";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 v[0:15], v[4:7], v[44:47], v[16:31]", ";;#ASMEND"]
    clean = chain + chain + last + wait + ["v_mov_b32_e32 v16, 0"]
    assert chain_hazards(clean) == []
    copy = chain + ["v_mov_b64_e32 v[32:33], v[16:17]"] + last + wait
    assert chain_hazards(copy) == ["v_mov_b64_e32 v[32:33], v[16:17]"]
    reuse = chain + last + ["v_add_u32_e32 v16, v1, v2"] + wait
    assert chain_hazards(reuse) == ["v_add_u32_e32 v16, v1, v2"]


@pytest.mark.timeout(600)
def test_attention_asm_chains_have_no_hazards(tmp_path):
    out = tmp_path / "sparse_attn.s"
    cmd = [build.hipcc()] + build.FLAGS + ["--cuda-device-only", "-S", SRC, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels = list(_kernels(out.read_text()))
    # 32/64/128 heads, packed and paged, with and without the gather lead
    assert len(kernels) == 12, [k for k, _ in kernels]
    report = {}
    for name, body in kernels:
        n_asm = sum(1 for i, l in enumerate(body) if "v_mfma" in l and i and ";;#ASMSTART" in body[i - 1])
        assert n_asm > 0, f"{name}: no asm MFMA chain found"
        bad = chain_hazards(body)
        if bad:
            report[name] = bad[:5]
    assert not report, report
