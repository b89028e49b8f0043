"""Static check of the hand-scheduled parts of the library's gfx950 assembly.

The mainloop issues its LDS fragment reads and its MFMAs from inline asm, so the
compiler knows neither that those registers are written asynchronously nor the
MFMA result latency. This checker scans the device assembly of every kernel and
reports:

1. any instruction that reads (or non-LDS-writes) a VGPR/AGPR whose LDS load is
   still outstanding, i.e. not yet retired by an `s_waitcnt lgkmcnt(N)` (LDS
   operations of one wave complete in order and every one of them, writes
   included, counts; SMEM loads also count in lgkmcnt and are tracked the same
   way);
2. any non-MFMA instruction that touches a register an MFMA wrote fewer than
   MFMA_RESULT_STATES wait states earlier (s_nop N counts N+1, every other
   instruction 1), and any MFMA that reads as accumulator input a register a
   VALU instruction wrote fewer than VALU_TO_MFMA_STATES wait states earlier.

Control flow is followed with a fixed-point iteration over branch targets.

Usage: python tests/check_lds_waits.py [file.s]
(without a file it compiles the library's coda_kernels.hip to assembly first).
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

REG = re.compile(r"\b([vas])(?:\[(\d+):(\d+)\]|(\d+)\b)")
MFMA_RESULT_STATES = 19
VALU_TO_MFMA_STATES = 3
LGKM_LOADS = ("ds_read", "ds_load", "ds_bpermute", "ds_permute", "ds_swizzle", "s_load", "s_buffer_load")


def regs_of(text):
    out = set()
    for m in REG.finditer(text):
        kind = m.group(1)
        if kind == "s":
            continue
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            for r in range(int(m.group(2)), int(m.group(3)) + 1):
                out.add((kind, r))
    return out


def sregs_of(text):
    out = set()
    for m in REG.finditer(text):
        if m.group(1) != "s":
            continue
        if m.group(4) is not None:
            out.add(("s", int(m.group(4))))
        else:
            for r in range(int(m.group(2)), int(m.group(3)) + 1):
                out.add(("s", r))
    return out


def split_functions(asm: str):
    funcs = {}
    for m in re.finditer(r"^(\S+):\s*(?:;.*)?$", asm, re.M):
        name = m.group(1)
        if name.startswith(".") or name.startswith("__"):
            continue
        end = asm.find(".Lfunc_end", m.end())
        if end < 0:
            continue
        funcs[name] = asm[m.end():end]
    return funcs


def parse(body: str):
    insts = []
    for raw in body.split("\n"):
        line = raw.split(";")[0].strip()
        if not line or line.startswith(".") and not re.match(r"^\.LBB\S*:", line):
            continue
        insts.append(line)
    return insts


def check_function(name: str, body: str):
    insts = parse(body)
    labels = {l[:-1]: i for i, l in enumerate(insts) if l.endswith(":")}
    in_state = {}   # label -> (pending LDS queue, {reg: states since MFMA write}, {reg: states since VALU write})
    problems = []
    for _ in range(8):
        changed = False
        state, mf, va = (), {}, {}
        for i, ins in enumerate(insts):
            if ins.endswith(":"):
                prev = in_state.get(ins[:-1])
                if prev is not None:
                    state = merge(state, prev[0])
                    mf = merge_age(mf, prev[1])
                    va = merge_age(va, prev[2])
                continue
            op = ins.split()[0]
            args = ins[len(op):]
            if op == "s_waitcnt":
                m = re.search(r"lgkmcnt\((\d+)\)", args)
                if m:
                    n = int(m.group(1))
                    state = state[len(state) - n:] if n < len(state) else state
                    if n == 0:
                        state = ()
                mf, va = age(mf, 1), age(va, 1)
                continue
            if op == "s_nop":
                k = int(args.strip(), 0) + 1
                mf, va = age(mf, k), age(va, k)
                continue
            pending = set().union(*state) if state else set()
            ops = [a.strip() for a in args.split(",")]
            if op.startswith(LGKM_LOADS):
                dst = regs_of(ops[0]) | (sregs_of(ops[0]) if op.startswith("s_") else set())
                srcs = set()
                for a in ops[1:]:
                    srcs |= regs_of(a)
                bad = srcs & pending
                if bad:
                    problems.append((i, ins, "read of a register with a pending LDS/SMEM load", sorted(bad)))
                state = state + (frozenset(dst),)
            else:
                used = regs_of(args) | sregs_of(args)
                bad = used & pending
                if bad:
                    problems.append((i, ins, "use of a register with a pending LDS/SMEM load", sorted(bad)))
                if op.startswith("ds_"):  # LDS writes count in lgkmcnt too (no register returns)
                    state = state + (frozenset(),)
            if op.startswith("v_mfma"):
                srcc = regs_of(ops[3]) if len(ops) > 3 else set()
                hot = {r for r in srcc if va.get(r, 99) < VALU_TO_MFMA_STATES}
                if hot:
                    problems.append((i, ins, "MFMA reads an accumulator a VALU op just wrote", sorted(hot)))
                mf = age(mf, 1)
                va = age(va, 1)
                for r in regs_of(ops[0]):
                    mf[r] = 0
                    va.pop(r, None)
            elif op.startswith("v_"):
                hot = {r for r in regs_of(args) if mf.get(r, 99) < MFMA_RESULT_STATES}
                if hot:
                    problems.append((i, ins, "touches an MFMA result before it has landed", sorted(hot)))
                mf = age(mf, 1)
                va = age(va, 1)
                if ops and ops[0]:
                    for r in regs_of(ops[0]):
                        va[r] = 0
            else:
                mf, va = age(mf, 1), age(va, 1)
            if op.startswith(("s_branch", "s_cbranch")):
                tgt = args.strip().split()[-1]
                if tgt in labels:
                    old = in_state.get(tgt)
                    new = (state, mf, va) if old is None else (merge(old[0], state), merge_age(old[1], mf),
                                                               merge_age(old[2], va))
                    if new != old:
                        in_state[tgt] = new
                        changed = True
                if op == "s_branch":
                    state, mf, va = (), {}, {}
            if op == "s_endpgm":  # nothing falls through past the end of the program
                state, mf, va = (), {}, {}
        if not changed:
            break
    seen, uniq = set(), []
    for p in problems:
        if p[0] not in seen:
            seen.add(p[0])
            uniq.append(p)
    return uniq


def age(d, k):
    return {r: v + k for r, v in d.items() if v + k < 64}


def merge_age(a, b):
    out = dict(a)
    for r, v in b.items():
        out[r] = min(v, out.get(r, 99))
    return out


def merge(a, b):
    """Conservative union of two pending-load queues (aligned from the newest end)."""
    if not a:
        return b
    if not b:
        return a
    n = max(len(a), len(b))
    a2 = (frozenset(),) * (n - len(a)) + a
    b2 = (frozenset(),) * (n - len(b)) + b
    return tuple(x | y for x, y in zip(a2, b2))


def device_asm(src=None, extra_flags=()) -> str:
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    from transformer_gemm_epilogue_res_amd.build import CSRC, FLAGS, HIPCC
    src = src or os.path.join(CSRC, "coda_kernels.hip")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
        subprocess.run([HIPCC, *flags, *extra_flags, "--cuda-device-only", "-S", src, "-o", out], check=True,
                       capture_output=True)
        return open(out).read()


def check(asm: str):
    report = {}
    for name, body in split_functions(asm).items():
        probs = check_function(name, body)
        if probs:
            report[name] = probs
    return report


def main(argv):
    asm = open(argv[1]).read() if len(argv) > 1 else device_asm()
    rep = check(asm)
    for name, probs in rep.items():
        print(f"{name}: {len(probs)} problem(s)")
        for i, ins, why, regs in probs[:8]:
            print(f"   [{i}] {ins}    <- {why}: {regs[:6]}")
    print("OK" if not rep else f"{len(rep)} function(s) with problems")
    return 1 if rep else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
