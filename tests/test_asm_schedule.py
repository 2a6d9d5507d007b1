"""Static checks of the barrier schedule and resources on the library's own
gfx950 assembly (kept by the build).  No GPU.

What the pages ask of a split-barrier pipeline, checked on the code the
compiler actually produced:
* every wave executes the same barriers ("Xe2 ESIMD GEMM", Hardware limits;
  "Xe2 Nbarrier Pipelining", What Doesn't Work: Double-Arrive Deadlock): no
  s_barrier sits in code that only some lanes run (under a saved exec mask),
  and no loop that holds a barrier changes exec;
* each publish is one s_barrier right after its wait ("Xe2 Nbarrier
  Pipelining", Checklist for Adding Split Barriers, steps 6-7): in every
  kernel that stages tiles by LDS-DMA the barrier follows an
  s_waitcnt vmcnt(n) lgkmcnt(0), with n one of the wait counts the kernel's
  ring implies (closed forms of its template parameters below), the steady
  count inside the K-loop, and the K-loop holds exactly one barrier per
  K-tile it runs per iteration; in the persistent kernel with wave roles
  only the copy waves wait on vmcnt, and the other roles publish with
  lgkmcnt(0) alone (its own check);
* no kernel spills ("Xe2 ESIMD GEMM", Workflow step 2): the GEMM kernels use
  no scratch and spill no VGPR or SGPR;
* the race-detection build (libbpt_gemm_poison.so, run by
  tests/test_lds_poison_gpu.py) fills every LDS-DMA copy's destination with
  NaN, and waits for the fill, before issuing the copy.
"""
import os
import re

import pytest

from barrier_pipelined_tiled_amd import asm_info, build


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(build.ASM_PATH):
        build.build()
    with open(build.ASM_PATH) as f:
        return asm_info.kernels(f.read())


def _ints(name):
    """The integer template arguments of a mangled kernel name, in order."""
    return [int(x) for x in re.findall(r"Li(\d+)E", name)]


def expected_waits(name):
    """(wait counts a publish of this kernel may use, the steady count of its
    K-loop, barriers per K-loop iteration), from the ring's layout; None for
    kernels that stage nothing by LDS-DMA."""
    base = asm_info.base_name(name)
    if base == "gemm_pipelined_kernel":
        BM, BN, BK, S = _ints(name)[:4]
        lps = (BM * BK + BK * BN) // 2048           # 1 KiB copies per wave per stage (4 waves)
        allowed = {lps * (S - 1)} | {lps * (S - 2 - d) for d in range(S - 1)} | {0}
        return allowed, lps * (S - 2), 1
    if base == "gemm_apair_kernel":
        le, lo = 8 + 4, 4                           # even group: A pair + B; odd group: B
        return {lo + le + lo, le + lo, lo, 0}, le + lo, 2
    if base == "gemm_persist_kernel":
        (nk,) = _ints(name)
        lps = (256 * 32 + 32 * 128) // 2048
        return {lps * 2 + lps // 2, lps * 2, 0}, lps * 2, nk
    if base == "gemm_persist_apair_kernel":
        # windows of 2 B copies (even K-tiles) or 2 B + 8 A-pair copies (odd);
        # the publish after an even K-tile lets an even and an odd window
        # fly, after an odd one only an even window; the prologue's lets an
        # even window and half an odd one
        (nk,) = _ints(name)
        even, odd = 2, 2 + 8
        return {even + odd // 2, even + odd, even, 0}, {even + odd, even}, nk
    if base == "gemm_persist_ares_kernel":
        # 3 B stages of 2 copies per wave at K = 256, 4 at K = 128: publish
        # lets BSTAGES-2 windows fly, the prologue's half a window more; a
        # new group's panel sits between two full publishes in the loop body
        (nk,) = _ints(name)
        vm = 2 * ((3 if nk == 8 else 4) - 2)
        return {vm + 1, vm, 0}, {vm, 0}, nk + 2
    if base == "gemm_skinny_ring_kernel":
        kc, s = _ints(name)[:2]
        lps = (64 * kc * 2) // 4096 + (kc * 128 * 2) // 4096
        return {(s - 2) * lps}, (s - 2) * lps, 1
    if base == "attention_fwd_kernel":
        d, waves, bn, s = _ints(name)[:4]
        copies = bn * d * 2 // 1024 // waves
        return {(s - 2) * 2 * copies}, (s - 2) * 2 * copies, 1
    return None


_EXEC_WRITE = re.compile(r"^(s_\w+_saveexec_b64|v_cmpx_\w+|s_\w+_b64 exec,|s_mov_b64 exec,)")


def _loops(lines):
    """Line-index sets of the kernel's loops (natural loops of its control flow)."""
    return asm_info.natural_loops(lines)


def _barrier_kernels(kernels):
    return {n: k for n, k in kernels.items() if "s_barrier" in k["lines"]}


def test_every_barrier_kernel_is_recognised(kernels):
    names = _barrier_kernels(kernels)
    assert names
    for n in names:
        if asm_info.base_name(n) not in ("gemm_generic_kernel", "gemm_skinny_kernel", "gemm_persist_roles_kernel"):
            assert expected_waits(n) is not None, n           # the roles kernel: its own test below


_SAVEEXEC = re.compile(r"s_and_saveexec_b64 (s\[\d+:\d+\])")
_RESTORE = re.compile(r"s_or_b64 exec, exec, (s\[\d+:\d+\])")


def check_no_barrier_under_saved_exec(kernels):
    for n, k in _barrier_kernels(kernels).items():
        lines = k["lines"]
        starts, ends, succ = asm_info.basic_blocks(lines)
        # masks still open on entry to each block, joined over every path
        into = {0: frozenset()}
        work = [0]
        while work:
            b = work.pop()
            open_masks = set(into[b])
            for l in lines[starts[b]:ends[b]]:
                m = _SAVEEXEC.match(l)
                if m:
                    open_masks.add(m.group(1))
                    continue
                m = _RESTORE.match(l)
                if m:
                    open_masks.discard(m.group(1))
                    continue
                if l == "s_barrier":
                    assert not open_masks, f"{n}: s_barrier under saved exec {sorted(open_masks)}"
            for t in succ[b]:
                joined = into.get(t, frozenset()) | open_masks
                if t not in into or joined != into[t]:
                    into[t] = frozenset(joined)
                    work.append(t)


def test_no_barrier_under_a_saved_exec_mask(kernels):
    """s_and_saveexec opens a region only some lanes run, the s_or_b64 exec
    that restores the saved mask closes it; the open masks follow the
    control flow from block to block (a region that never closes runs to
    the end of the program).  No barrier may be reachable inside one."""
    check_no_barrier_under_saved_exec(kernels)


def check_publish_waits(kernels):
    for n, k in _barrier_kernels(kernels).items():
        exp = expected_waits(n)
        if exp is None:
            continue
        allowed, steady, per_iter = exp
        L = k["lines"]
        bars = [i for i, l in enumerate(L) if l == "s_barrier"]
        seen = set()
        for i in bars:
            m = re.match(r"s_waitcnt vmcnt\((\d+)\) lgkmcnt\(0\)$", L[i - 1])
            assert m, f"{n}: barrier not preceded by a publish wait: {L[i - 1]!r}"
            seen.add(int(m.group(1)))
        assert seen <= allowed, f"{n}: wait counts {sorted(seen)} not in {sorted(allowed)}"
        assert (steady <= seen) if isinstance(steady, set) else (steady in seen), n
        # the innermost loop around each barrier is the K-loop: per_iter
        # barriers, all with the steady count, no exec writes
        loops = _loops(L)
        k_loops = []
        for i in bars:
            around = [lp for lp in loops if i in lp]
            if not around:
                continue                       # prologue, drain or epilogue publish
            inner = min(around, key=len)
            if inner not in k_loops:
                k_loops.append(inner)
        assert k_loops, f"{n}: no loop holds a barrier"
        for lp in k_loops:
            idx = sorted(i for i in lp if L[i] == "s_barrier")
            assert len(idx) == per_iter, f"{n}: {len(idx)} barriers per K-loop iteration, expected {per_iter}"
            steady_set = steady if isinstance(steady, set) else {steady}
            for j in idx:
                m = re.match(r"s_waitcnt vmcnt\((\d+)\) lgkmcnt\(0\)$", L[j - 1])
                assert m and int(m.group(1)) in steady_set, (n, L[j - 1])
            writes = [L[i] for i in sorted(lp) if _EXEC_WRITE.match(L[i])]
            assert not writes, f"{n}: the K-loop writes exec: {writes[:3]}"


def test_publish_waits_match_the_ring(kernels):
    check_publish_waits(kernels)


def check_roles_barriers(kernels):
    """The persistent kernel with wave roles: only its copy waves issue
    copies, so only their publish waits on vmcnt, for the ring's two younger
    windows (2 x 8 copies; the pieces of a new A panel ride on the same
    waits); the compute and store waves publish with lgkmcnt(0) alone.  The
    compute loop (one tile, unrolled) holds one publish per K-tile, the copy
    and store loops one each; no loop with a barrier writes exec."""
    seen = 0
    for n, k in kernels.items():
        if asm_info.base_name(n) != "gemm_persist_roles_kernel":
            continue
        seen += 1
        (nk,) = _ints(n)
        L = k["lines"]
        bars = [i for i, l in enumerate(L) if l == "s_barrier"]
        allowed = {"s_waitcnt vmcnt(16) lgkmcnt(0)", "s_waitcnt lgkmcnt(0)"}
        kinds = {}
        for i in bars:
            assert L[i - 1] in allowed, (n, L[i - 1])
            kinds[L[i - 1]] = kinds.get(L[i - 1], 0) + 1
        assert kinds.get("s_waitcnt vmcnt(16) lgkmcnt(0)", 0) >= 1, kinds
        per_loop = sorted(sum(1 for i in lp if L[i] == "s_barrier") for lp in _loops(L)
                          if any(L[i] == "s_barrier" for i in lp))
        assert per_loop == [1, 1, nk], (n, per_loop)
        for lp in _loops(L):
            if any(L[i] == "s_barrier" for i in lp):
                writes = [L[i] for i in sorted(lp) if _EXEC_WRITE.match(L[i])]
                assert not writes, (n, writes[:3])
    assert seen == 4                           # {f16, bf16} x {K = 128, 256}


def test_roles_kernel_barriers(kernels):
    check_roles_barriers(kernels)


APAIR = "_ZN3bpt17gemm_apair_kernelIDF16_DF16_Lb0EEEvNS_8GemmArgsE"


def _planted(kernels, edit):
    k = dict(kernels[APAIR])
    lines = list(k["lines"])
    loop = min((lp for lp in _loops(lines) if any(lines[i] == "s_barrier" for i in lp)), key=len)
    a, b = min(loop), max(loop)
    edit(lines, a, b)
    k["lines"] = lines
    return {APAIR: k}


def test_the_checks_catch_planted_mistakes(kernels):
    """Each mistake, planted in a copy of the 4096^3 kernel's K-loop, fails a
    check: a dropped barrier, a wait that lets one copy too many fly, a wait
    for LDS reads dropped, an exec write, a barrier in a divergent region."""
    def first(lines, a, b, what):
        return next(i for i in range(a, b + 1) if lines[i] == what)

    def drop_barrier(lines, a, b):
        del lines[first(lines, a, b, "s_barrier")]

    def off_by_one(lines, a, b):
        i = first(lines, a, b, "s_barrier")
        lines[i - 1] = "s_waitcnt vmcnt(17) lgkmcnt(0)"

    def no_lds_wait(lines, a, b):
        i = first(lines, a, b, "s_barrier")
        lines[i - 1] = "s_waitcnt vmcnt(16)"

    def exec_write(lines, a, b):
        lines.insert(a + 1, "s_and_saveexec_b64 s[60:61], vcc")

    def divergent(lines, a, b):
        i = first(lines, a, b, "s_barrier")
        lines.insert(i - 1, "s_and_saveexec_b64 s[60:61], vcc")

    check_publish_waits({APAIR: kernels[APAIR]})
    check_no_barrier_under_saved_exec({APAIR: kernels[APAIR]})
    for edit in (drop_barrier, off_by_one, no_lds_wait, exec_write):
        with pytest.raises(AssertionError):
            check_publish_waits(_planted(kernels, edit))
    with pytest.raises(AssertionError):
        check_no_barrier_under_saved_exec(_planted(kernels, divergent))


GEMM_TEMPLATES = ("gemm_pipelined_kernel", "gemm_apair_kernel", "gemm_persist_kernel", "gemm_persist_apair_kernel",
                  "gemm_persist_ares_kernel", "gemm_persist_roles_kernel", "gemm_skinny_kernel",
                  "gemm_skinny_ring_kernel", "gemm_generic_kernel", "skinny_sum_kernel", "splitk_sum_kernel",
                  "repack_pad_kernel", "fill_zero_kernel")


def test_gemm_kernels_use_no_scratch_and_spill_nothing(kernels):
    seen = set()
    for n, k in kernels.items():
        base = asm_info.base_name(n)
        if base not in GEMM_TEMPLATES:
            continue
        seen.add(base)
        m = k["meta"]
        assert m["private_segment_fixed_size"] == 0, (n, m)
        assert m["vgpr_spill_count"] == 0, (n, m)
        if base not in ("gemm_persist_kernel", "gemm_persist_apair_kernel", "gemm_persist_ares_kernel"):   # SGPRs: below
            assert m["sgpr_spill_count"] == 0, (n, m)
    assert seen == set(GEMM_TEMPLATES)


@pytest.mark.xfail(strict=True, reason="the persistent short-K kernels still spill a few SGPRs into VGPR lanes "
                                       "(v_writelane/v_readlane at the tile switch, no memory traffic)")
def test_persistent_kernel_spills_no_sgpr(kernels):
    for n, k in kernels.items():
        if asm_info.base_name(n) in ("gemm_persist_kernel", "gemm_persist_apair_kernel", "gemm_persist_ares_kernel"):
            assert k["meta"]["sgpr_spill_count"] == 0, (n, k["meta"])


def test_kernels_fit_one_workgroup_in_lds(kernels):
    for n, k in kernels.items():
        assert k["meta"]["group_segment_fixed_size"] <= 160 * 1024, n


def test_attention_without_a_ragged_tail_spills_nothing(kernels):
    """The attention instances for Skv a multiple of the key block (the
    workload's 4096 keys) have no masked copy of the block code after the
    loop, use no scratch and spill nothing; the RAGGED instances may spill
    around their masked last block."""
    seen = 0
    for n, k in kernels.items():
        if asm_info.base_name(n) == "attention_fwd_kernel" and n.endswith("Lb0EEEvNS_8AttnArgsE"):
            seen += 1
            m = k["meta"]
            assert m["private_segment_fixed_size"] == 0 and m["vgpr_spill_count"] == 0, (n, m)
    assert seen == 16                          # {f16, bf16} x {16-bit, fp32 out} x {+,- scale} x {D 128, 256}


def _is_copy(line):
    return line.startswith("buffer_load_dwordx4") and line.endswith(" lds")


@pytest.fixture(scope="module")
def poison_kernels():
    if not os.path.exists(build.POISON_ASM_PATH):
        build.build_poison()
    with open(build.POISON_ASM_PATH) as f:
        return asm_info.kernels(f.read())


def test_poison_build_fills_every_copy_destination_first(kernels, poison_kernels):
    """Per kernel the poison build has the normal build's copies and exactly
    one more ds_write_b128 per copy, and walking its code, no copy comes
    without a ds_write_b128 and an lgkmcnt(0) wait since the previous copy
    (the fill and the copy are adjacent statements, so no label separates
    them)."""
    assert set(poison_kernels) == set(kernels)
    copies = 0
    for n, k in poison_kernels.items():
        lines, normal = k["lines"], kernels[n]["lines"]
        nc = sum(map(_is_copy, lines))
        assert nc == sum(map(_is_copy, normal)), n
        writes = sum(l.startswith("ds_write_b128") for l in lines)
        assert writes - sum(l.startswith("ds_write_b128") for l in normal) == nc, n
        filled = waited = False
        for l in lines:
            if l.endswith(":"):
                filled = waited = False
            elif l.startswith("ds_write_b128"):
                filled, waited = True, False
            elif filled and l.startswith("s_waitcnt") and "lgkmcnt(0)" in l:
                waited = True
            elif _is_copy(l):
                assert filled and waited, f"{n}: a copy without its fill"
                filled = waited = False
        copies += nc
    assert copies > 0
