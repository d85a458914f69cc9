"""Build-time check of the MFMA instructions written as inline assembly.

score_tile_kernel issues part of its MFMAs (those whose accumulators live in
VGPRs) as inline assembly, where the compiler cannot see the instruction and
so inserts none of the wait states CDNA requires around it. The kernel is
written so that none are needed; this check proves it on the code the
compiler actually produced, for every instantiation, and fails the build
otherwise. It reads the device assembly of score.hip (our own build) and, for
every MFMA that came from an inline-assembly block and writes VGPRs, rejects:

  * a VALU instruction writing any of its A, B or C/D registers within the 4
    instruction slots before it (VALU write -> MFMA read needs 2 wait states);
  * within the 20 slots after it, a VALU instruction reading or writing its
    D registers, a store reading them, or an MFMA reading them as A or B (an
    8-pass XDL result needs about 11 wait states before other readers, and
    its C read needs them before a VALU overwrite).

Slots are counted conservatively: each instruction is one, `s_nop n` is n+1.
"""

from __future__ import annotations

import re

_VREG = re.compile(r"v\[(\d+):(\d+)\]|v(\d+)\b")
_STORES = ("ds_write", "buffer_store", "global_store", "scratch_store", "flat_store")
BEFORE_SLOTS = 4
AFTER_SLOTS = 20


def _regs(text: str) -> set[int]:
    out: set[int] = set()
    for m in _VREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _split(line: str) -> tuple[str, list[str]]:
    parts = line.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [t.strip() for t in parts[1].split(";")[0].split(",")]


def _slots(op: str, ops: list[str]) -> int:
    if op == "s_nop" and ops:
        try:
            return int(ops[0], 0) + 1
        except ValueError:
            return 1
    return 1


def _kernel_lines(asm: str, name: str) -> list[tuple[str, bool]]:
    i = asm.find(name + ":")
    j = asm.find(".Lfunc_end", i)
    lines: list[tuple[str, bool]] = []
    in_asm = False
    for raw in asm[i:j].split("\n")[1:]:
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        lines.append((t, in_asm))
    return lines


def check_asm(asm: str, kernel_filter: str = "score_tile_kernel") -> list[str]:
    """Return one message per violation in the kernels whose name contains
    kernel_filter; an empty list means the code is clean."""
    problems: list[str] = []
    names = [k for k in re.findall(r"\.amdhsa_kernel (\S+)", asm) if kernel_filter in k]
    if not names:
        problems.append(f"no kernel matching {kernel_filter!r} in the assembly")
    for name in names:
        lines = _kernel_lines(asm, name)
        n_asm_mfma = 0
        for n, (t, from_asm) in enumerate(lines):
            op, ops = _split(t)
            if not (from_asm and op.startswith("v_mfma") and len(ops) >= 4
                    and ops[0].startswith("v")):
                continue
            n_asm_mfma += 1
            D, A, B = _regs(ops[0]), _regs(ops[1]), _regs(ops[2])
            slots = 0
            for m in range(n - 1, -1, -1):
                pt, _ = lines[m]
                pop, pops = _split(pt)
                if (pop.startswith("v_") and not pop.startswith("v_mfma") and pops
                        and _regs(pops[0]) & (A | B | D)):
                    problems.append(f"{name}: VALU write '{pt}' just before '{t}'")
                slots += _slots(pop, pops)
                if slots >= BEFORE_SLOTS:
                    break
            slots = 0
            for m in range(n + 1, len(lines)):
                pt, _ = lines[m]
                pop, pops = _split(pt)
                used = _regs(",".join(pops))
                if pop.startswith("v_mfma"):
                    if len(pops) >= 3 and (_regs(pops[1]) | _regs(pops[2])) & D:
                        problems.append(f"{name}: '{pt}' reads the result of '{t}' too early")
                elif pop.startswith("v_") and used & D:
                    problems.append(f"{name}: VALU '{pt}' touches the result of '{t}' too early")
                elif pop.startswith(_STORES) and used & D:
                    problems.append(f"{name}: store '{pt}' reads the result of '{t}' too early")
                slots += _slots(pop, pops)
                if slots >= AFTER_SLOTS:
                    break
        if n_asm_mfma == 0:
            problems.append(f"{name}: no inline-assembly MFMA found (check is stale)")
    return problems


# ---------------------------------------------------------------------------
# Cross-lane reductions of the comparison kernel: its butterflies run on DPP
# row operations, ds_swizzle and readlane, never on ds_bpermute (the LDS
# crossbar), which this check enforces on the built assembly.
# ---------------------------------------------------------------------------

def kernel_bodies(asm: str, name_part: str) -> dict[str, str]:
    """Assembly text of every kernel whose symbol contains name_part."""
    out = {}
    for m in re.finditer(r"^(_Z\S*%s\S*):" % re.escape(name_part), asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        out[m.group(1)] = asm[m.end():end if end >= 0 else len(asm)]
    return out


def check_no_bpermute(asm: str, name_part: str = "compare_kernel") -> list[str]:
    """Problems: a missing kernel, or ds_bpermute / ds_permute inside it."""
    bodies = kernel_bodies(asm, name_part)
    if not bodies:
        return [f"no kernel matching {name_part!r} in the assembly"]
    problems = []
    for name, body in bodies.items():
        n = len(re.findall(r"^\s*ds_(?:b)?permute_b32", body, re.M))
        if n:
            problems.append(f"{name}: {n} ds_bpermute/ds_permute instruction(s)")
    return problems


# ---------------------------------------------------------------------------
# Buffer -> LDS copies written as inline assembly (both tile kernels' operand
# stages, the comparison kernel's window ring): the compiler inserts no wait
# states around an inline-assembly instruction, and CDNA requires 5 between a
# VALU instruction that writes an SGPR (v_readlane restoring a spilled
# resource, a v_cmp writing a lane mask) and a vector memory instruction that
# reads that SGPR as its resource or offset. The copies carry their own
# s_nop; this check proves on the built code that no such write sits closer.
# ---------------------------------------------------------------------------

VMEM_SGPR_SLOTS = 5
_SREG = re.compile(r"s\[(\d+):(\d+)\]|\bs(\d+)\b")


def _sregs(text: str) -> set[int]:
    out: set[int] = set()
    for m in _SREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def check_lds_dma_sgpr(asm: str, name_part: str = "") -> list[str]:
    """Problems: a VALU write of an SGPR that a buffer -> LDS load reads,
    fewer than 5 wait states before it, in any kernel whose symbol contains
    name_part."""
    problems: list[str] = []
    names = [k for k in re.findall(r"\.amdhsa_kernel (\S+)", asm) if name_part in k]
    for name in names:
        lines = _kernel_lines(asm, name)
        for n, (t, _) in enumerate(lines):
            op, ops = _split(t)
            if not (op.startswith("buffer_load") and " lds" in t and len(ops) >= 3):
                continue
            used = _sregs(ops[1]) | _sregs(ops[2])
            slots = 0
            for m in range(n - 1, -1, -1):
                pt, _ = lines[m]
                pop, pops = _split(pt)
                if pop.startswith("v_") and pops and _sregs(pops[0]) & used:
                    problems.append(f"{name}: VALU '{pt}' writes an SGPR that '{t}' reads "
                                    f"fewer than {VMEM_SGPR_SLOTS} wait states later")
                slots += _slots(pop, pops)
                if slots >= VMEM_SGPR_SLOTS:
                    break
    return problems
