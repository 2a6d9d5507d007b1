"""The library's own gfx950 assembly, as the build keeps it (hipcc
-save-temps): each kernel's instructions and resource use, and a hash of its
machine code.

Two users:
* the stored HBM counter readings (profiles/traffic.json) name the kernels
  they were taken on by a hash of their code, so a reading is dropped as
  soon as any instruction of those kernels changes -- and kept when only a
  comment or an unrelated kernel changed;
* the static checks of the barrier schedule (tests/test_asm_schedule.py).

Nothing here runs on the GPU or takes part in any computation.
"""
from __future__ import annotations

import hashlib
import json
import re

import yaml

_LABEL = re.compile(r"^([A-Za-z_][\w.$]*):")


def _normalise(line: str) -> str:
    """An instruction or directive with its comment, numbering of local
    labels and compilation-unit id removed."""
    line = line.split(";", 1)[0].strip()
    line = re.sub(r"\.LBB\d+_(\d+)", r".LBB_\1", line)
    line = re.sub(r"\.Lfunc_end\d+", ".Lfunc_end", line)
    line = re.sub(r"\.Ltmp\d+", ".Ltmp", line)
    line = re.sub(r"__hip_cuid_[0-9a-f]+", "__hip_cuid", line)
    return re.sub(r"\s+", " ", line)


def kernels(text: str) -> dict:
    """name -> {"lines": instruction/directive lines of the kernel (its code
    and its kernel descriptor), "meta": resource use from the code object
    metadata}."""
    meta = {}
    m = re.search(r"\.amdgpu_metadata\n(---\n.*?\n\.\.\.)\n", text, re.S)
    if m:
        doc = yaml.safe_load(m.group(1))
        for k in doc.get("amdhsa.kernels", []):
            meta[k[".name"]] = {
                "private_segment_fixed_size": k.get(".private_segment_fixed_size"),
                "group_segment_fixed_size": k.get(".group_segment_fixed_size"),
                "vgpr_count": k.get(".vgpr_count"),
                "agpr_count": k.get(".agpr_count"),
                "sgpr_count": k.get(".sgpr_count"),
                "vgpr_spill_count": k.get(".vgpr_spill_count"),
                "sgpr_spill_count": k.get(".sgpr_spill_count"),
            }
    out = {}
    cur = None
    body = []
    for raw in text.splitlines():
        if cur is None:
            lm = _LABEL.match(raw)
            if lm and lm.group(1) in meta:
                cur, body = lm.group(1), []
            continue
        if raw.startswith(".Lfunc_end"):
            out[cur] = {"lines": body, "meta": meta[cur]}
            cur = None
            continue
        n = _normalise(raw)
        if n:
            body.append(n)
    return out


def code_hash(k: dict) -> str:
    """Hash of a kernel's normalised code and descriptor."""
    h = hashlib.sha256()
    for line in k["lines"]:
        h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def base_name(name: str) -> str | None:
    """The template (function) name of a kernel from its mangled name
    (_ZN3bpt17gemm_apair_kernelI...) or from a demangled one
    (void bpt::gemm_apair_kernel<...>(...)), as profilers print either."""
    m = re.match(r"_ZN3bpt(\d+)", name)
    if m:
        n = int(m.group(1))
        start = m.end()
        return name[start:start + n]
    m = re.search(r"bpt::([A-Za-z_]\w*)\s*[<(]", name)
    return m.group(1) if m else None


def template_hash(hashes: dict, base: str) -> str | None:
    """Hash over every instance of one kernel template (name -> code hash of
    all kernels); None when the library has no such kernel."""
    items = sorted((n, h) for n, h in hashes.items() if base_name(n) == base)
    if not items:
        return None
    return hashlib.sha256(json.dumps(items).encode()).hexdigest()[:16]


_BRANCH = re.compile(r"^s_(cbranch_\w+|branch) (\.LBB_\d+)$")


def basic_blocks(lines: list) -> tuple:
    """A kernel's basic blocks (split at labels and after branches and
    s_endpgm): their first line indices, their end indices (exclusive) and
    each block's successors (branch target, and the next block unless the
    block ends in an unconditional branch or s_endpgm)."""
    starts = [0]
    for i, l in enumerate(lines):
        if l.endswith(":") and i != 0:
            starts.append(i)
        elif (_BRANCH.match(l) or l == "s_endpgm") and i + 1 < len(lines):
            starts.append(i + 1)
    starts = sorted(set(starts))
    ends = starts[1:] + [len(lines)]
    label_block = {}
    for b, s in enumerate(starts):
        if lines[s].endswith(":"):
            label_block[lines[s][:-1]] = b
    succ = {b: [] for b in range(len(starts))}
    for b, (s, e) in enumerate(zip(starts, ends)):
        last = lines[e - 1] if e > s else ""
        m = _BRANCH.match(last)
        if m:
            if m.group(2) in label_block:
                succ[b].append(label_block[m.group(2)])
            if m.group(1) != "branch" and b + 1 < len(starts):
                succ[b].append(b + 1)
        elif last != "s_endpgm" and b + 1 < len(starts):
            succ[b].append(b + 1)
    return starts, ends, succ


def natural_loops(lines: list) -> list:
    """The loops of a kernel's control flow: for every back edge (a branch to
    a block that dominates it) the set of line indices of the loop's blocks.
    Built from basic blocks, so a backward jump that only reflects block
    placement is not a loop."""
    starts, ends, succ = basic_blocks(lines)
    n = len(starts)
    pred = {b: [] for b in range(n)}
    for b, ss in succ.items():
        for t in ss:
            pred[t].append(b)
    # dominators (iterative, entry = block 0)
    dom = [set(range(n)) for _ in range(n)]
    dom[0] = {0}
    changed = True
    while changed:
        changed = False
        for b in range(1, n):
            ps = [dom[p] for p in pred[b]]
            new = set.intersection(*ps) | {b} if ps else {b}
            if new != dom[b]:
                dom[b] = new
                changed = True
    loops = []
    for u in range(n):
        for h in succ[u]:
            if h in dom[u]:                      # back edge u -> h
                body = {h, u}
                stack = [u]
                while stack:
                    x = stack.pop()
                    if x == h:
                        continue
                    for p in pred[x]:
                        if p not in body:
                            body.add(p)
                            stack.append(p)
                loops.append({i for b in body for i in range(starts[b], ends[b])})
    return loops
