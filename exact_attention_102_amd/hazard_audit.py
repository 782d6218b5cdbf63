"""Audit of MFMA result hazards in the compiled gfx950 kernels (host tool).

    python -m exact_attention_102_amd.hazard_audit [--keep DIR]

The matrix cores do not interlock their results: after a v_mfma_* writes its
accumulator registers, an instruction that reads them through the vector ALU
(v_accvgpr_read, any VALU, a store of the register) must follow at a distance of
enough wait states, which the compiler provides with independent instructions or
s_nop (s_nop N counts N + 1).  For the 8-pass v_mfma_f32_32x32x16_bf16 on gfx950
that distance is 12: the smallest the compiler inserts anywhere in these kernels
inside one basic block.  This tool compiles the kernels' device assembly, builds
each function's control-flow graph and, for every MFMA, walks every path forward
to each instruction that reads one of its result registers before they are
overwritten, reporting paths shorter than the required distance.  It also checks the
other direction: an MFMA may not read (as A, B or C) a register that a VALU instruction
wrote in the 2 wait states before it.  The compiler keeps both distances for the MFMAs it
emits; MFMAs written as inline assembly (vector-register results) are invisible to it,
and under register pressure it refilled their operand registers with v_accvgpr_read one
wait state before such a statement (a wrong dQ at d = 288 until every statement opened
with s_nop 1).  A compiler that
places the reads after a join whose other predecessor branches straight from the
MFMA's block can leave such a path; that is how a variant of the atomic dK/dV
kernel (its dS^T zeroing moved into a wave-uniform branch) read dK accumulators one
wait state after the MFMA that wrote them and produced a wrong dK.

Readers that are v_readfirstlane are not reported: these kernels use them only
for wave-uniform indices and addresses, and the one short path the scan finds
into a v_readfirstlane reads a loop value the compiler left undefined on that path.
"""
from __future__ import annotations

import argparse
import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
KERNEL_SOURCES = ["fa_fwd.hip", "fa_bwd.hip"]

# wait states between an MFMA writing its result and a VALU-side read of it, per opcode prefix
REQUIRED = {"v_mfma_f32_32x32x16": 12}
# wait states between a VALU instruction writing a register and an MFMA reading it (A, B or C)
VALU_TO_MFMA = 2
STORE_OPS = ("ds_write", "buffer_store", "global_store", "buffer_atomic", "global_atomic")


def regs(tok: str) -> set:
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def split(ins: str):
    parts = ins.split(None, 1)
    toks = [t.strip() for t in re.split(r",\s*", parts[1])] if len(parts) > 1 else []
    return parts[0], toks


def wait_states(ins: str) -> int:
    m = re.match(r"s_nop (\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def cfg(body: str):
    """Basic blocks {name: (instructions, successors)} of one function's assembly."""
    blocks, order, cur, fall = {}, [], None, {}
    for line in body.split("\n"):
        code = line.split(";")[0].strip()
        lab = re.match(r"^([.\w$]+):", code)
        bb = re.match(r"^; %bb\.(\d+):", line.strip())
        if lab or bb:
            name = lab.group(1) if lab else "bb" + bb.group(1)
            if cur is not None:
                fall[cur] = name
            cur = name
            blocks[cur] = []
            order.append(cur)
            continue
        if cur is None or not code or code.startswith("."):
            continue
        blocks[cur].append(code)
    out = {}
    for b in order:
        ins = blocks[b]
        last = ins[-1] if ins else ""
        if last.startswith("s_branch"):
            succ = [last.split()[1]]
        elif last.startswith("s_cbranch"):
            succ = [last.split()[1]] + ([fall[b]] if b in fall else [])
        elif last.startswith(("s_endpgm", "s_setpc")):
            succ = []
        else:
            succ = [fall[b]] if b in fall else []
        out[b] = (ins, [s for s in succ if s in blocks])
    return out


def _walk(g, b, i, x, live, need, is_hit, found):
    """Follows every control-flow path from instruction i + 1 of block b until `need` wait
    states have passed or the registers `live` are all overwritten, recording each
    instruction for which is_hit(op, operands, live) holds."""
    stack = [(b, i + 1, 0, frozenset(live))]
    seen = {}
    while stack:
        bb, j, w, live = stack.pop()
        if w >= need or not live:
            continue
        L, succ = g[bb]
        if j >= len(L):
            for s in succ:
                if seen.get((s, live), 1 << 30) > w:
                    seen[(s, live)] = w
                    stack.append((s, 0, w, live))
            continue
        y = L[j]
        op2, t2 = split(y)
        dst = regs(t2[0]) if t2 else set()
        if op2.startswith(STORE_OPS):
            dst = set()
        if is_hit(op2, t2, live):
            found.append((w, x, y, bb))
        stack.append((bb, j + 1, w + wait_states(y), frozenset(live - dst)))


def _reads_mfma_result(op, t, live):
    if op.startswith("v_mfma"):  # A or B operand (C = the same registers is a legal chain)
        return bool((regs(t[1]) | regs(t[2])) & live) if len(t) > 2 else False
    src = set()
    for tok in t[1:]:
        src |= regs(tok)
    if op.startswith(STORE_OPS) and t:
        src |= regs(t[0])
    return bool(src & live) and not op.startswith("v_readfirstlane")


def _mfma_reads(op, t, live):
    if not op.startswith("v_mfma") or len(t) < 4:
        return False
    return bool((regs(t[1]) | regs(t[2]) | regs(t[3])) & live)


def scan_function(body: str):
    """[(wait states, writer, reader, reader block)] for every read closer than required:
    an MFMA's result read by a VALU instruction, a store or another MFMA's A/B operand,
    and a VALU-written register read by an MFMA."""
    g = cfg(body)
    found = []
    for b, (ins, _) in g.items():
        for i, x in enumerate(ins):
            op, toks = split(x)
            if not toks:
                continue
            need = next((n for p, n in REQUIRED.items() if op.startswith(p)), None)
            if need is not None:
                _walk(g, b, i, x, regs(toks[0]), need, _reads_mfma_result, found)
            elif op.startswith("v_") and not op.startswith(("v_mfma", "v_readfirstlane", "v_readlane")):
                _walk(g, b, i, x, regs(toks[0]), VALU_TO_MFMA, _mfma_reads, found)
    return found


def scan_assembly(text: str) -> dict:
    """{function: findings} over every kernel in one assembly file."""
    res = {}
    for m in re.finditer(r"^(_Z\S+):", text, re.M):
        end = text.find(".Lfunc_end", m.end())
        f = scan_function(text[m.start():end])
        if f:
            res[m.group(1)] = f
    return res


def compile_asm(src: str, outdir: str) -> str:
    from exact_attention_102_amd.build import FLAGS, hipcc
    out = os.path.join(outdir, os.path.splitext(src)[0] + ".s")
    cmd = [hipcc()] + FLAGS + ["--cuda-device-only", "-S", "-x", "hip", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s" % (src, r.stderr))
    return out


def audit(keep: str | None = None) -> dict:
    """Compiles the kernel sources to device assembly and scans them; {source: {function: findings}}."""
    with tempfile.TemporaryDirectory() as tmp:
        d = keep or tmp
        os.makedirs(d, exist_ok=True)
        with ThreadPoolExecutor(max_workers=len(KERNEL_SOURCES)) as ex:
            paths = list(ex.map(lambda s: compile_asm(s, d), KERNEL_SOURCES))
        return {os.path.basename(p): scan_assembly(open(p).read()) for p in paths}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--keep", default=None, help="directory to keep the assembly in")
    a = ap.parse_args()
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    res = audit(a.keep)
    bad = 0
    for src, funcs in res.items():
        for fn, f in funcs.items():
            bad += 1
            w, x, y, bb = min(f)
            print("%s %s: %d short path(s), fewest %d wait states: %s -> %s [%s]" % (src, fn, len(f), w, x, y, bb))
    print("hazard audit: %d function(s) with a short MFMA-result or VALU-to-MFMA path" % bad)
    sys.exit(1 if bad else 0)


if __name__ == "__main__":
    main()
