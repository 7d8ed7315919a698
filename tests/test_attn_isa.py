"""The attention kernel writes its score products as inline-asm MFMAs (VGPR
destinations).  The compiler does not know the result latency of an asm
instruction, so it would not insert the wait states a too-early read needs:
this test compiles csrc/k_attn.hip for gfx950 and checks, on the generated
code along every control-flow path (loop back-edges included), the wait
states the CDNA3/CDNA4 matrix cores need around an XDL MFMA of up to 16
passes, counting one wait state per instruction (the least an issued
instruction takes) and N + 1 for an s_nop N:

* READ_GAP: no instruction other than an MFMA accumulating into exactly the
  same registers reads an asm MFMA's destination sooner (a VALU, memory or
  export read needs passes + 4 wait states, at most 20);
* WAR_GAP: no non-MFMA instruction writes an asm MFMA's srcC registers
  (read in the MFMA's later passes) sooner (at most 15 wait states);
* VALU_GAP: no vector-ALU instruction writes a register an asm MFMA reads
  fewer than this many instructions before it (2 wait states).

CPU only: hipcc cross-compiles; nothing runs on a GPU."""
import os
import re
import shutil
import subprocess

import pytest

from sparse_bit_attention_amd import build

READ_GAP = 24
WAR_GAP = 16
VALU_GAP = 2
SRCS = ["k_attn.hip"]


def vregs(tok):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    if m:
        return {int(m.group(1))}
    return set()


def operands(text):
    parts = text.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [o.strip() for o in re.split(r",(?![^\[]*\])", parts[1].split(";")[0])]


STORES = ("global_store", "buffer_store", "ds_write", "scratch_store", "flat_store", "global_atomic",
          "buffer_atomic", "ds_add", "ds_max", "ds_min")


def reads_writes(text):
    """(registers read, registers written) of one instruction (VGPRs only)."""
    op, ops = operands(text)
    if not ops:
        return set(), set()
    if op.startswith(STORES) or op.startswith("s_"):
        return set().union(*[vregs(o.split()[0]) for o in ops]), set()
    dst = vregs(ops[0].split()[0])
    src = set().union(*[vregs(o.split()[0]) for o in ops[1:]]) if len(ops) > 1 else set()
    return src, dst


def parse(path):
    """kernel -> (instructions [(text, is_asm)], label -> index)"""
    kernels = {}
    cur = None
    in_asm = False
    for line in open(path):
        t = line.strip()
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = m.group(1)
            kernels[cur] = ([], {})
            continue
        if cur is None:
            continue
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if t.startswith(".Lfunc_end"):
            cur = None  # blocks may follow an s_endpgm until here
            continue
        m = re.match(r"^(\.?\w+):", t)
        if m:
            kernels[cur][1][m.group(1)] = len(kernels[cur][0])
            continue
        if not t or t.startswith((".", ";")):
            continue
        kernels[cur][0].append((t.split(";")[0].strip(), in_asm))
    return kernels


def wait_states(text):
    """Wait states an instruction provides: N + 1 for s_nop N, else 1."""
    op, ops = operands(text)
    return int(ops[0], 0) + 1 if op == "s_nop" and ops else 1


def successors(ins, labels, j):
    op, ops = operands(ins[j][0])
    if op == "s_endpgm":
        return []
    if op == "s_branch":
        return [labels[ops[0]]]
    if op.startswith("s_cbranch"):
        return [j + 1, labels[ops[0]]]
    return [j + 1]


def predecessors(ins, labels):
    pred = [[] for _ in ins]
    for j in range(len(ins)):
        for k in successors(ins, labels, j):
            if k < len(ins):
                pred[k].append(j)
    return pred


def violations(ins, labels):
    bad = []
    n_asm = 0
    pred = predecessors(ins, labels)
    for i, (text, is_asm) in enumerate(ins):
        if not (is_asm and text.startswith("v_mfma")):
            continue
        n_asm += 1
        _, ops = operands(text)
        dst, srcc = vregs(ops[0]), vregs(ops[3])
        srcs = vregs(ops[1]) | vregs(ops[2]) | srcc
        # vector-ALU writes of the operands just before, on every path in
        back = [(j, 1) for j in pred[i]]
        seen = set()
        while back:
            j, dist = back.pop()
            if dist > VALU_GAP or (j, dist) in seen:
                continue
            seen.add((j, dist))
            if ins[j][0].startswith("v_") and not ins[j][0].startswith("v_mfma"):
                if reads_writes(ins[j][0])[1] & srcs:
                    bad.append((ins[j][0], text, -dist, "VALU writes an operand"))
            back.extend((k, dist + wait_states(ins[j][0])) for k in pred[j])
        # walk every path for READ_GAP instructions; live: the result is still
        # this MFMA's (not yet taken over by an accumulation or overwritten)
        stack = [(j, 1, True) for j in successors(ins, labels, i)]
        seen = set()
        while stack:
            j, dist, live = stack.pop()
            if dist > READ_GAP or (j, dist, live) in seen or j >= len(ins):
                continue
            seen.add((j, dist, live))
            utext = ins[j][0]
            uop, uops = operands(utext)
            if uop.startswith("v_mfma"):
                udst, usrcc = vregs(uops[0]), vregs(uops[3])
                uab = vregs(uops[1]) | vregs(uops[2])
                chain = usrcc == dst and udst == dst
                if live and uab & dst:
                    bad.append((text, utext, dist, "MFMA A/B operand reads the result"))
                if live and usrcc & dst and not chain:
                    bad.append((text, utext, dist, "partial srcC overlap"))
                if chain:
                    live = False  # the next accumulation owns the result from here
            else:
                r, w = reads_writes(utext)
                if live and r & dst:
                    bad.append((text, utext, dist, "reads the result"))
                if w & srcc and dist <= WAR_GAP:
                    bad.append((text, utext, dist, "overwrites srcC"))
                if w & dst and not (r & dst):
                    live = False  # the result is dead on this path
            stack.extend((k, dist + wait_states(utext), live) for k in successors(ins, labels, j))
    return n_asm, bad


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    if not shutil.which(build.HIPCC) and not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    kernels = {}
    for src in SRCS:
        out = str(tmp_path_factory.mktemp("isa") / (src + ".s"))
        flags = [f for f in build.FLAGS if f not in ("-fPIC",)]
        cmd = [build.HIPCC, *flags, *build.EXTRA.get(src, []), "--cuda-device-only", "-S",
               os.path.join(build.CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        kernels.update(parse(out))
    return kernels


# the d = 128 pipelined (bound-path) instances, mangled:
# k_attn<128, LIN, true, QK8, FINE, DUMP>, including the int32 read-back form
HOT = ["_ZN3sla6k_attnILi128ELb1ELb1ELb1ELb0ELb0E", "_ZN3sla6k_attnILi128ELb1ELb1ELb1ELb1ELb0E",
       "_ZN3sla6k_attnILi128ELb1ELb1ELb0ELb0ELb0E", "_ZN3sla6k_attnILi128ELb0ELb1ELb1ELb0ELb0E",
       "_ZN3sla6k_attnILi128ELb0ELb1ELb1ELb0ELb1E", "_ZN3sla6k_attnILi128ELb0ELb1ELb1ELb1ELb1E"]


def test_asm_mfma_results_are_not_read_early(isa):
    total = 0
    problems = []
    per_kernel = {}
    for name, (ins, labels) in isa.items():
        n, bad = violations(ins, labels)
        total += n
        per_kernel[name] = n
        problems += [(name[:60],) + b for b in bad[:3]]
    assert total > 0, "no inline-asm MFMA found: the check no longer covers the kernel"
    for h in HOT:
        found = [n for k, n in per_kernel.items() if k.startswith(h)]
        assert found and found[0] > 0, f"{h}: the score products are no longer inline asm"
    assert not problems, "\n".join(map(str, problems))


def test_checker_catches_an_early_read():
    # a planted mistake: a VALU read two instructions after an asm MFMA
    ins = [("v_mfma_i32_16x16x64_i8 v[4:7], v[8:11], v[12:15], v[16:19]", True),
           ("v_mov_b32_e32 v0, 0", False),
           ("v_accvgpr_write_b32 a1, v7", False),
           ("s_endpgm", False)]
    n, bad = violations(ins, {})
    assert n == 1 and bad and bad[0][3] == "reads the result"
    # the same read after a loop back-edge is found too
    ins = [("v_mov_b32_e32 v0, v5", False)] + [("s_nop 0", False)] * 3 + [
        ("v_mfma_i32_16x16x64_i8 v[4:7], v[8:11], v[12:15], v[16:19]", True),
        ("s_cbranch_scc1 .LBB0_1", False), ("s_endpgm", False)]
    n, bad = violations(ins, {".LBB0_1": 0})
    assert bad and bad[0][2] == 2
    # an exact accumulation chain is allowed; a write to srcC is not
    ins = [("v_mfma_i32_16x16x64_i8 v[4:7], v[8:11], v[12:15], v[16:19]", True),
           ("v_mfma_i32_16x16x64_i8 v[4:7], v[20:23], v[12:15], v[4:7]", True),
           ("v_mov_b32_e32 v17, 0", False), ("s_endpgm", False)]
    n, bad = violations(ins, {})
    assert n == 2 and [b[3] for b in bad] == ["overwrites srcC"]
    # an s_nop 7 provides eight wait states: a read after three of them is far enough
    ins = [("v_mfma_i32_16x16x64_i8 v[4:7], v[8:11], v[12:15], v[16:19]", True)] + [
        ("s_nop 7", False)] * 3 + [("v_mov_b32_e32 v0, v5", False), ("s_endpgm", False)]
    n, bad = violations(ins, {})
    assert n == 1 and not bad
    ins = ins[:2] + ins[4:]
    n, bad = violations(ins, {})
    assert bad and bad[0][3] == "reads the result"
    # a vector write of an operand right before the MFMA
    ins = [("v_mov_b32_e32 v9, 0", False),
           ("v_mfma_i32_16x16x64_i8 v[4:7], v[8:11], v[12:15], v[16:19]", True),
           ("s_endpgm", False)]
    n, bad = violations(ins, {})
    assert [b[3] for b in bad] == ["VALU writes an operand"]
