"""The cross-lane LDS traffic of the pair-symmetric and energy kernels, checked
on the gfx950 assembly the compiler makes from them (host only: hipcc
cross-compiles without a GPU).

In the LDS-carried pair-symmetric step, lane l reads, adds to and writes back
the j-side slot k = l + s; the next access to that slot is lane l - 1's read
at step s + 1.  No barrier separates them: one wave's LDS instructions
execute in the order they are issued, so the read is correct as long as the
write of step s is issued before the read of step s + 1.  The source keeps
that order with empty asm statements with a memory clobber; this test checks
that the code the compiler emitted still has it, so a compiler change that
moved one of these accesses would fail here instead of silently on the GPU.

In the energy pair pass every lane writes its j-body into the wave's tile
once per sweep and all lanes then read the tile: the writes must stay out of
the step loop, issued before it.
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from direct_all_pairs_softened_amd import build as hip_build

LABEL = re.compile(r"^(\.LBB\d+_\d+):")
BRANCH = re.compile(r"^s_c?branch\S*\s+(\.LBB\d+_\d+)")
DS = re.compile(r"^(ds_(read|write)\S*)\s+(.*?)\s*(?:offset:(\d+))?$")


def device_asm(tmp_path, source):
    """gfx950 assembly of one library source, built with the library's flags."""
    out = str(tmp_path / (os.path.basename(source) + ".s"))
    cmd = [hip_build.HIPCC, *hip_build.COMMON_FLAGS, "--cuda-device-only", "-S", "-x", "hip",
           os.path.join(hip_build.CSRC, source), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"hipcc could not build {source}: {r.stderr[-400:]}")
    with open(out) as f:
        return f.read()


def functions(asm, name):
    """(mangled name, instruction lines) of every kernel whose name contains name."""
    out = []
    for m in re.finditer(r"^(_Z\S*" + name + r"\S*):", asm, re.M):
        end = asm.index("s_endpgm", m.end())
        lines = [l.split(";")[0].strip() for l in asm[m.end():end].splitlines()]
        out.append((m.group(1), [l for l in lines if l and not l.startswith(".") or LABEL.match(l)]))
    assert out, f"no kernel named {name}"
    return out


def innermost_loops(lines):
    """(first, last) line indices of each loop (a label and a later branch back
    to it) that contains no other loop."""
    labels = {}
    loops = []
    for i, l in enumerate(lines):
        m = LABEL.match(l)
        if m:
            labels[m.group(1)] = i
        m = BRANCH.match(l)
        if m and m.group(1) in labels:
            loops.append((labels[m.group(1)], i))
    return [a for a in loops
            if not any(b != a and a[0] <= b[0] and b[1] <= a[1] for b in loops)]


def lds_ops(lines):
    """(kind, width, address register, offset) of each LDS instruction."""
    ops = []
    for l in lines:
        m = DS.match(l)
        if not m:
            continue
        op, kind, operands = m.group(1), m.group(2), m.group(3).rstrip(",")
        regs = [x.strip() for x in operands.split(",")]
        addr = regs[0] if kind == "write" else regs[1]
        ops.append((kind, op.split("_")[-1], addr, int(m.group(4) or 0), op))
    return ops


SYM = re.compile(r"symmetric_task_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb([01])"
                 r"ELi(\d+)ELi(\d+)E")


def test_pair_symmetric_slot_write_precedes_next_read(tmp_path):
    asm = device_asm(tmp_path, "symmetric.hip")
    checked = 0
    for name, lines in functions(asm, "symmetric_task_kernel"):
        K, KP, W, OCC, IL, POT, ML, JL = (int(x) for x in SYM.search(name).groups())
        if JL == 0:
            continue  # the rotated j-state has no LDS slots
        width = "b128" if POT else "b96"  # the slot: 3 sums, or 4 with the potential
        steps_seen = 0
        for a, b in innermost_loops(lines):
            ops = lds_ops(lines[a:b + 1])
            writes = [o for o in ops if o[0] == "write" and o[1] == width]
            if not writes:
                continue
            base = {o[2] for o in writes}
            assert len(base) == 1, (name, writes)
            offsets = {o[3] for o in writes}
            slot = [o for o in ops if o[1] == width and o[2] in base and o[3] in offsets]
            # read and write of one slot per step, steps in order: R0 W0 R1 W1 ...
            kinds = [o[0] for o in slot]
            assert kinds == ["read", "write"] * (len(slot) // 2), (name, slot)
            offs = [o[3] for o in slot]
            for u in range(len(slot) // 2):
                assert offs[2 * u] == offs[2 * u + 1], (name, slot)
                if u:
                    assert offs[2 * u] == offs[2 * u - 2] + 16, (name, slot)
            # nothing else in the loop writes LDS
            assert len(writes) == sum(1 for o in ops if o[0] == "write"), (name, ops)
            steps_seen += len(slot) // 2
        assert steps_seen >= JL, f"{name}: no step loop with {JL} slot updates found"
        checked += 1
    assert checked >= 5, checked  # the LDS-carried plain and potential variants


def test_energy_pairs_tile_written_outside_the_step_loop(tmp_path):
    asm = device_asm(tmp_path, "energy.hip")
    for name, lines in functions(asm, "energy_pairs_kernel"):
        loops = innermost_loops(lines)
        step_loops = [(a, b) for a, b in loops
                      if any(o[0] == "read" and o[1] == "b128" for o in lds_ops(lines[a:b + 1]))]
        assert step_loops, name
        for a, b in step_loops:
            assert not [o for o in lds_ops(lines[a:b + 1]) if o[0] == "write"], (name, a, b)
            # the sweep's tile store comes before the loop that reads it
            before = [o for o in lds_ops(lines[:a]) if o[0] == "write" and o[1] == "b128"]
            assert before, (name, a)
