"""Static check of the per-head prefill kernels' hand-scheduled loads.

Those kernels issue global loads in inline asm and wait for them later with
fixed `s_waitcnt vmcnt(N)` counts, so loads stay in flight across loop
iterations.  The compiler treats an asm output as written when the asm
statement ends; if it reused, copied or spilled such a register before the
wait, the load would land later and overwrite whatever the register then
holds.  This module compiles the source to gfx950 assembly and runs a
data-flow analysis over each kernel's control-flow graph: the state at a
point is the set of (load, vector-memory operations issued after it) pairs
that may still be outstanding, merged over all paths; `s_waitcnt vmcnt(N)`
retires the loads with N or more younger operations.  Any instruction other
than a later load into the same registers that reads or writes a register a
possibly-outstanding load writes is reported.
"""
from __future__ import annotations

import os
import re
import subprocess

_VMEM = re.compile(r"^(global_|scratch_|buffer_|flat_)")
_LOAD = re.compile(r"^(global_load|scratch_load|buffer_load|flat_load)")


def _vregs(tok: str) -> frozenset:
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return frozenset({int(m.group(1))}) if m else frozenset()


def compile_asm(src: str, out: str, flags: list[str]) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed:\n{r.stderr[-4000:]}")
    return open(out).read()


def kernels(asm: str) -> list[str]:
    return re.findall(r"^(_Z\w+):", asm, flags=re.M)


def check_kernel(asm: str, name: str) -> list[tuple[int, str, list[int]]]:
    """(asm line, instruction, registers) for every hazard found in `name`."""
    lines = asm.split("\n")
    start = next(i for i, l in enumerate(lines) if l.startswith(name + ":"))
    end = next(i for i in range(start + 1, len(lines)) if lines[i].startswith(".Lfunc_end"))
    # Basic blocks: a label starts one, a branch ends one.
    blocks: dict[str, list[tuple[int, str]]] = {"entry": []}
    order = ["entry"]
    cur = "entry"
    for i in range(start + 1, end):
        ins = lines[i].split(";")[0].strip()
        if not ins or (ins.startswith(".") and not ins.endswith(":")):
            continue
        if ins.endswith(":"):
            cur = ins[:-1]
            blocks[cur] = []
            order.append(cur)
            continue
        blocks[cur].append((i + 1, ins))
        if ins.split()[0].startswith(("s_cbranch", "s_branch")):
            cur = f"after{i + 1}"
            blocks[cur] = []
            order.append(cur)
    succ = {}
    for n, b in enumerate(order):
        out, falls = [], True
        for _, ins in blocks[b]:
            op = ins.split()[0]
            if op == "s_branch":
                out.append(ins.split()[1])
                falls = False
            elif op.startswith("s_cbranch"):
                out.append(ins.split()[1])
            elif op == "s_endpgm":
                falls = False
        if falls and n + 1 < len(order):
            out.append(order[n + 1])
        succ[b] = [s for s in out if s in blocks]

    dst_of: dict[int, frozenset] = {}

    def step(state, ln, ins, report):
        op = ins.split()[0]
        ops = [t for t in re.split(r"[ ,]+", ins)[1:] if t]
        if op == "s_waitcnt":
            m = re.search(r"vmcnt\((\d+)\)", ins)
            if m:
                n = int(m.group(1))
                state = frozenset((lid, k) for lid, k in state if k < n)
            return state
        used = frozenset().union(*(_vregs(t) for t in ops)) if ops else frozenset()
        live = {r: lid for lid, _ in state for r in dst_of.get(lid, ())}
        if _VMEM.match(op):
            dst = _vregs(ops[0]) if _LOAD.match(op) else frozenset()
            bad = (used - dst) & live.keys()
            if bad and report is not None:
                report.append((ln, ins, sorted(bad)))
            dst_of[ln] = dst
            return frozenset((lid, min(k + 1, 64)) for lid, k in state) | {(ln, 0)}
        bad = used & live.keys()
        if bad and report is not None:
            report.append((ln, ins, sorted(bad)))
        return state

    entry = {b: frozenset() for b in order}
    changed = True
    while changed:
        changed = False
        for b in order:
            st = entry[b]
            for ln, ins in blocks[b]:
                st = step(st, ln, ins, None)
            for s in succ[b]:
                merged = entry[s] | st
                if merged != entry[s]:
                    entry[s] = merged
                    changed = True
    report: list = []
    for b in order:
        st = entry[b]
        for ln, ins in blocks[b]:
            st = step(st, ln, ins, report)
    return report
