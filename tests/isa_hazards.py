"""Matrix-core hazard check on gfx950 assembly (test helper, no GPU needed).

The dK/dV kernel issues its matrix-core products from inline assembly (to
keep accumulators and stationary operands in the register files it needs).
The compiler inserts no wait states around inline assembly, so the code it
generates around those products must be checked for the hazards the
hardware does not interlock. This module compiles a source file to gfx950
assembly and scans every function for them, following the control flow.

Hazard classes and the wait states each needs (`RULES`). The values are
what the compiler's own hazard recognizer inserts for the same instruction
pairs written with the matrix-core builtins (`tests/isa/hazard_rules.hip`,
checked by `tests/test_isa_hazards.py`), for v_mfma_f32_32x32x16_{bf16,f16}:

* valu_to_srcab: a vector-ALU write of a register, then a product that
  reads it as its A or B operand;
* valu_to_srcc:  a vector-ALU write, then a product that reads it as its
  accumulator input;
* xdl_to_read:   a product's result register, then any other instruction
  that reads it (vector ALU, LDS or memory instruction, or another product
  reading it as A or B). A product that reads the result as its own
  accumulator input with the same destination (a chain of accumulations)
  needs none.
* xdl_to_write:  a product's result register, then a vector-ALU write of it.

Loads from LDS or memory into operand registers are ordered by s_waitcnt,
which the compiler places around inline assembly like around any other use.

A wait state is one instruction slot: every instruction counts one, and
s_nop N counts N + 1. Branches count one, and at a join the check assumes
the nearest write over all incoming paths.
"""

from __future__ import annotations

import functools
import os
import re
import subprocess

RULES = {"valu_to_srcab": 2, "valu_to_srcc": 2, "xdl_to_read": 12, "xdl_to_write": 12}
FAR = 64  # distances at or above this never matter

_REG = re.compile(r"(?<![\w])([va])(?:(\d+)\b|\[(\d+):(\d+)\])")
_LABEL = re.compile(r"^([.\w$]+):")


def compile_to_asm(src: str, include_dirs, extra_flags=()) -> str:
    """hipcc -S of one source file for gfx950 (device code only)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *extra_flags]
    for d in include_dirs:
        cmd += ["-I", d]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += [src, "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed: {' '.join(cmd)}\n{r.stderr[-4000:]}")
    return r.stdout


@functools.lru_cache(maxsize=None)
def library_asm(name: str) -> str:
    """gfx950 assembly of one of the library's sources (cached per process)."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    csrc = os.path.join(root, "exact_attention_115_amd", "csrc")
    return compile_to_asm(os.path.join(csrc, name), [os.path.join(root, "include"), csrc])


def kernel_resources(asm: str) -> dict:
    """Kernel name -> its code-object metadata entries (vgpr_count,
    vgpr_spill_count, sgpr_spill_count, private_segment_fixed_size,
    group_segment_fixed_size) as ints."""
    out = {}
    for block in asm.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        vals = {}
        for key in ("vgpr_count", "vgpr_spill_count", "sgpr_spill_count",
                    "private_segment_fixed_size", "group_segment_fixed_size"):
            m = re.search(r"\.%s:\s+(\d+)" % key, block)
            vals[key] = int(m.group(1)) if m else None
        out[name] = vals
    return out


def functions(asm: str) -> dict:
    """Function name -> list of its lines (from the label to s_endpgm)."""
    out, cur, name = {}, None, None
    for line in asm.splitlines():
        m = re.match(r"^([A-Za-z_][\w.$]*):", line)
        if m and not m.group(1).startswith(".L"):
            name, cur = m.group(1), []
            out[name] = cur
            continue
        if cur is not None:
            cur.append(line)
            if line.strip().startswith("s_endpgm"):
                cur = None
    return out


def _regs(text: str):
    """Registers named in an operand string: ('v', n) / ('a', n)."""
    regs = []
    for m in _REG.finditer(text):
        kind = m.group(1)
        if m.group(2) is not None:
            regs.append((kind, int(m.group(2))))
        else:
            regs.extend((kind, i) for i in range(int(m.group(3)), int(m.group(4)) + 1))
    return regs


def _split_operands(rest: str):
    """Operands of an instruction (top-level commas; modifiers dropped)."""
    ops, depth, cur = [], 0, ""
    for ch in rest:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            ops.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        ops.append(cur.strip())
    # The last operand may carry space-separated modifiers ("v1 offset:16").
    if ops:
        ops[-1] = ops[-1].split(" ")[0] if not ops[-1].startswith("[") else ops[-1]
    return ops


class Instr:
    __slots__ = ("text", "op", "ops", "cost", "label", "is_xdl", "is_valu", "dst", "srcs",
                 "src_ab", "src_c", "branch", "target", "ends")

    def __init__(self, text):
        self.text = text
        self.label = None
        parts = text.split(None, 1)
        self.op = parts[0]
        rest = parts[1] if len(parts) > 1 else ""
        self.ops = _split_operands(rest) if rest else []
        self.cost = 1
        if self.op == "s_nop":
            self.cost = int(self.ops[0], 0) + 1 if self.ops else 1
        self.is_xdl = self.op.startswith("v_mfma")
        valu = self.op.startswith("v_") and not self.is_xdl
        self.is_valu = valu
        self.dst, self.srcs, self.src_ab, self.src_c = [], [], [], []
        if self.is_xdl:
            self.dst = _regs(self.ops[0])
            self.src_ab = _regs(self.ops[1]) + _regs(self.ops[2])
            self.src_c = _regs(self.ops[3]) if len(self.ops) > 3 else []
        elif valu:
            writes_sgpr = (self.op.startswith(("v_cmp", "v_readlane", "v_readfirstlane")))
            if self.ops and not writes_sgpr:
                self.dst = _regs(self.ops[0])
                self.srcs = [r for o in self.ops[1:] for r in _regs(o)]
            else:
                self.srcs = [r for o in self.ops for r in _regs(o)]
        else:
            # Loads write their VGPRs asynchronously (ordered by s_waitcnt);
            # every register they name is read at issue except a load's
            # destination.
            is_load = ("_load" in self.op or self.op.startswith("ds_read")) and "lds" not in rest
            ops = self.ops[1:] if is_load else self.ops
            self.srcs = [r for o in ops for r in _regs(o)]
        self.branch = self.op.startswith(("s_branch", "s_cbranch"))
        self.target = self.ops[0] if self.branch and self.ops else None
        self.ends = self.op in ("s_endpgm", "s_branch", "s_setpc_b64")


def parse(lines):
    """Instructions and the index of each label."""
    instrs, labels = [], {}
    for line in lines:
        s = line.strip()
        if not s or s.startswith(";") or s.startswith("."):
            m = _LABEL.match(s)
            if m and s.startswith(".L"):
                labels[m.group(1)] = len(instrs)
            continue
        m = _LABEL.match(s)
        if m:
            labels[m.group(1)] = len(instrs)
            continue
        s = s.split(";")[0].strip()
        if s:
            instrs.append(Instr(s))
    return instrs, labels


def distances(lines):
    """For every instruction that reads a register recently written by the
    vector ALU or by a product: (index, text, {kind: nearest distance}),
    kinds 'valu_to_srcab', 'valu_to_srcc' (products' operands written by the
    vector ALU), 'xdl_to_read' (a product's result read by another
    instruction; an accumulation chain into the same registers excepted) and
    'xdl_to_write' (a vector-ALU write of a product's result). Distances are
    in wait states, over every path through the control flow."""
    instrs, labels = parse(lines)
    n = len(instrs)
    if n == 0:
        return []
    # Basic blocks: starts at labels, after branches and at 0.
    starts = sorted({0, *labels.values(), *(i + 1 for i, x in enumerate(instrs) if x.branch)})
    starts = [s for s in starts if s < n]
    block_of = {}
    blocks = []
    for bi, s in enumerate(starts):
        e = starts[bi + 1] if bi + 1 < len(starts) else n
        blocks.append((s, e))
        block_of[s] = bi
    succ = []
    for s, e in blocks:
        last = instrs[e - 1]
        out = []
        if last.branch and last.target in labels and labels[last.target] in block_of:
            out.append(block_of[labels[last.target]])
        if not last.ends and e < n:
            out.append(block_of[e])
        succ.append(out)
    # State: reg -> (dist since VALU write, dist since product write), kept
    # only for registers written less than FAR wait states ago.
    entry = [None] * len(blocks)
    entry[0] = {}
    found = {}
    work = [0]

    def merge(a, b):
        out = dict(a)
        for r, (dv, dx) in b.items():
            if r in out:
                ov, ox = out[r]
                out[r] = (min(ov, dv), min(ox, dx))
            else:
                out[r] = (dv, dx)
        return out

    def note(i, kind, d):
        if d < FAR:
            cur = found.setdefault(i, {})
            cur[kind] = min(cur.get(kind, FAR), d)

    while work:
        bi = work.pop()
        state = dict(entry[bi])
        s, e = blocks[bi]
        for i in range(s, e):
            x = instrs[i]
            if x.is_xdl:
                for r in x.src_ab:
                    dv, dx = state.get(r, (FAR, FAR))
                    note(i, "valu_to_srcab", dv)
                    note(i, "xdl_to_read", dx)
                chain = set(x.src_c) == set(x.dst)
                for r in x.src_c:
                    dv, dx = state.get(r, (FAR, FAR))
                    note(i, "valu_to_srcc", dv)
                    if not chain:
                        note(i, "xdl_to_read", dx)
            else:
                for r in x.srcs:
                    note(i, "xdl_to_read", state.get(r, (FAR, FAR))[1])
                if x.is_valu:
                    for r in x.dst:
                        note(i, "xdl_to_write", state.get(r, (FAR, FAR))[1])
            w = x.cost
            state = {r: (dv + w, dx + w) for r, (dv, dx) in state.items()
                     if dv + w < FAR or dx + w < FAR}
            if x.is_xdl:
                for r in x.dst:
                    state[r] = (state.get(r, (FAR, FAR))[0], 0)
            elif x.is_valu:
                for r in x.dst:
                    state[r] = (0, state.get(r, (FAR, FAR))[1])
        for sb in succ[bi]:
            new = state if entry[sb] is None else merge(entry[sb], state)
            if entry[sb] is None or new != entry[sb]:
                entry[sb] = new
                work.append(sb)
    return [(i, instrs[i].text, found[i]) for i in sorted(found)]


def check(lines, rules=RULES):
    """Hazard violations in one function: a list of strings (empty if none)."""
    out = []
    for i, text, kinds in distances(lines):
        for kind, d in kinds.items():
            if d < rules[kind]:
                out.append(f"[{i}] {kind}: {d} wait states (needs {rules[kind]}): {text}")
    return out
