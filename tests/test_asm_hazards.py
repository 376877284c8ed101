"""Wait states in front of the hand-written LDS-DMA loads (CPU: compiles to
gfx950 assembly, runs nothing).

The direct global->LDS loads are inline assembly, and the compiler's hazard
pass does not look inside inline assembly.  The gfx9 family needs, in front
of a buffer load that writes LDS:
  - 5 wait states after a VALU instruction writes an SGPR that the load
    reads (its buffer resource; v_readlane does that when a spilled resource
    is restored), and
  - 1 wait state after a SALU write of M0 (the LDS address).
A missing wait lets the load read a half-updated resource: wrong addresses,
zeros or a memory fault, depending on how the compiler allocated registers
that day.  This test checks every such load of every kernel.
"""
import re

import pytest

from warp_specialized_pipelined_amd import build as _build

LDS_LOAD = re.compile(r"^\s*buffer_load_dwordx4 v\d+, s\[(\d+):(\d+)\], 0 offen(?: nt)? lds")
NEEDED_SGPR = 5
NEEDED_M0 = 1


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    path = _build.dump_asm(str(tmp_path_factory.mktemp("asm")))
    text = open(path).read()
    out = {}
    # gemm_kernel<...> and gemm_kernel_m192<...> (mangled with their name lengths, 11 and 16)
    for m in re.finditer(r"^(_ZN6migemm\d+gemm_kernel\w*?I\S*):[^\n]*\n(.*?)^\.Lfunc_end", text,
                         re.S | re.M):
        out[m.group(1)] = m.group(2).split("\n")
    assert len(out) == 36, f"expected the 36 GEMM kernel instantiations, found {len(out)}"
    assert sum("gemm_kernel_m192" in k for k in out) == 4
    return out


def _writes(inst):
    """Destination registers of one instruction, as written (first operand)."""
    parts = inst.split(None, 1)
    if len(parts) < 2:
        return parts[0], ""
    return parts[0], parts[1].split(",")[0].strip()


def _sgprs(dst):
    m = re.fullmatch(r"s(\d+)", dst)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", dst)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def check_load(lines, i):
    """Problems with the wait states in front of the LDS load at lines[i]."""
    lo, hi = map(int, LDS_LOAD.match(lines[i]).groups())
    rsrc = set(range(lo, hi + 1))
    waits = 0
    j = i - 1
    while j >= 0 and waits < NEEDED_SGPR:
        t = lines[j].split(";")[0].strip()  # drop comments (";;#ASMSTART", "; %bb.3:")
        j -= 1
        if t.endswith(":"):  # a branch target: its predecessors are not all above
            return ["block boundary %d wait states before the load" % waits]
        if not t or t.startswith("."):  # directives
            continue
        op, dst = _writes(t)
        if op.startswith("v_") and _sgprs(dst) & rsrc:
            return ["%s writes the resource %d wait states before the load" % (op, waits)]
        if dst == "m0" and waits < NEEDED_M0:
            return ["%s writes M0 %d wait states before the load" % (op, waits)]
        waits += int(t.split()[1], 0) + 1 if op == "s_nop" else 1
    return []


def test_lds_dma_loads_have_their_wait_states(kernels):
    bad = []
    for name, lines in kernels.items():
        n_loads = 0
        for i, line in enumerate(lines):
            if LDS_LOAD.match(line):
                n_loads += 1
                for p in check_load(lines, i):
                    bad.append("%s line %d: %s" % (name[:60], i, p))
        # every kernel has a K-loop prologue and loop body full of them
        assert n_loads >= 24, (name, n_loads)
    assert not bad, "\n".join(bad[:20])


def test_checker_sees_the_hazard():
    # The pattern the compiler produced once, with the wait states removed:
    # a spilled resource restored right in front of the load.
    lines = [
        "\tv_readlane_b32 s88, v254, 58",
        "\ts_mov_b32 m0, s34",
        "\tv_readlane_b32 s91, v254, 61",
        "\tbuffer_load_dwordx4 v22, s[88:91], 0 offen lds",
    ]
    assert check_load(lines, 3)
    m0_only = ["\tv_add_u32_e32 v1, v2, v3", "\ts_mov_b32 m0, s34",
               "\tbuffer_load_dwordx4 v22, s[88:91], 0 offen lds"]
    assert check_load(m0_only, 2)
    ok = ["\tv_readlane_b32 s91, v254, 61", "\ts_mov_b32 m0, s34", "\ts_nop 4",
          "\tbuffer_load_dwordx4 v22, s[88:91], 0 offen lds"]
    assert not check_load(ok, 3)
    # the non-temporal form is checked the same way
    nt = [x.replace("offen lds", "offen nt lds") for x in lines]
    assert LDS_LOAD.match(nt[3]) and check_load(nt, 3)


def _innermost_k_loops(lines):
    """(first, last) line of every innermost loop that holds MFMAs: the K
    loops (a back-edge branch to an earlier label closes a loop)."""
    labels = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(\.LBB\w+):", l)
        if m:
            labels[m.group(1)] = i
    loops = []
    for i, l in enumerate(lines):
        m = re.search(r"s_c?branch\w*\s+(\.LBB\w+)", l)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            loops.append((labels[m.group(1)], i))
    inner = [(a, b) for a, b in loops
             if not any(a <= c and d <= b and (c, d) != (a, b) for c, d in loops)]
    return [(a, b) for a, b in inner if sum("v_mfma" in x for x in lines[a:b]) >= 16]


def test_no_scratch_access_inside_a_k_loop(kernels):
    """A scratch reload inside a K loop waits (vmcnt) for every stage load in
    flight, which stalls the ring; spills may only sit in per-tile code."""
    bad = {}
    for name, lines in kernels.items():
        loops = _innermost_k_loops(lines)
        assert loops, f"no K loop found in {name}"
        hits = [i for a, b in loops for i in range(a, b) if "scratch_" in lines[i]]
        if hits:
            bad[name] = [lines[i].strip() for i in hits[:3]]
    assert not bad, bad
