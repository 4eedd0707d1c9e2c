"""Static check of the LDS-DMA ring's waits in the compiled int8 kernels.

The int8 kernels stage operands through a ring of LDS buffers filled by
LDS-DMA loads (buffer_load ... lds) and synchronise with a hand-placed
`s_waitcnt vmcnt(N)` followed by `s_barrier`.  vmcnt counts every vector
memory load and retires in issue order, so in a kernel that also loads into
registers such a wait is only correct if, in the instruction order the
compiler finally emits, every DMA of the stage about to be read lies more
than N loads back.  The compiler may move ordinary loads between blocks (it
once sank the prologue's filter loads behind the first wait), so this is
checked on the emitted assembly: the prologue followed by several passes of
the stage loop is replayed in text order and, at the j-th ring wait, every
DMA of stages 0..j-1 must have retired.  A loop whose blocks the compiler
laid out out of order fails the structural asserts rather than passing.

No GPU is needed: hipcc cross-compiles the sources to gfx950 assembly.
"""
import os
import re
import shutil

import pytest

from convolution_forward_gemm_amd import build as hip_build

pytestmark = pytest.mark.skipif(not os.path.exists(hip_build.HIPCC) and not shutil.which("hipcc"),
                                reason="hipcc not available")

VMEM = re.compile(r"^\s*(buffer_load|global_load|buffer_store|global_store|flat_)")
WAIT = re.compile(r"^\s*s_waitcnt\s.*vmcnt\((\d+)\)")


def _functions(asm, prefix):
    """{mangled kernel name: [instruction lines]} for kernels matching prefix."""
    out, cur, body = {}, None, []
    for line in asm.splitlines():
        m = re.match(r"^(_ZN9convfprop\w+):", line)
        if m:
            cur, body = m.group(1), []
            continue
        if cur is None:
            continue
        if line.startswith(".Lfunc_end"):
            if cur.startswith(prefix):
                out[cur] = body
            cur = None
            continue
        body.append(line)
    return out


def _template_ints(name):
    return [int(v) for v in re.findall(r"Li(\d+)E", name)]


def _split(body):
    """(prologue lines, loop-body lines).  The prologue is the path from the
    kernel's entry to the first loop header, walked in execution order: an
    unconditional branch is followed; a conditional one is followed into a
    loop header, or towards one when the fall-through path does not lead to
    one (the compiler may place the loop after the epilogue), and otherwise
    falls through.  The loop body runs from that header's label to
    the branch back to it."""
    labels, headers = {}, set()
    for i, line in enumerate(body):
        m = re.match(r"^(\.LBB\w+):", line)
        if m:
            labels[m.group(1)] = i
            if "Loop Header" in line:
                headers.add(m.group(1))
    def reaches_header(k):
        # straight-line code from line k (passing labels and conditional
        # branches) arrives at a loop header
        while k < len(body):
            m = re.match(r"^(\.LBB\w+):", body[k])
            if m and m.group(1) in headers:
                return True
            if re.match(r"^\s*(s_branch|s_endpgm|s_setpc)", body[k]):
                return False
            k += 1
        return False

    pro, i, steps = [], 0, 0
    while i < len(body) and steps < 100000:
        steps += 1
        line = body[i]
        m = re.match(r"^(\.LBB\w+):", line)
        if m and m.group(1) in headers:
            label = m.group(1)
            for j in range(i + 1, len(body)):
                if re.match(r"^\s*s_c?branch\w*\s+%s\s*$" % re.escape(label), body[j]):
                    return pro, body[i:j + 1]
            return pro, []
        m = re.match(r"^\s*s_branch\s+(\.LBB\w+)\s*$", line)
        if m:
            i = labels[m.group(1)]
            continue
        m = re.match(r"^\s*s_cbranch\w*\s+(\.LBB\w+)\s*$", line)
        if m and (m.group(1) in headers or
                  (not reaches_header(i + 1) and reaches_header(labels[m.group(1)]))):
            i = labels[m.group(1)]
            continue
        if re.match(r"^\s*s_endpgm", line):
            break
        pro.append(line)
        i += 1
    return body, []


def _loops(body):
    """Every (header index, loop lines) of the body, in text order."""
    out = []
    for i, line in enumerate(body):
        m = re.match(r"^(\.LBB\w+):.*Loop Header", line)
        if m:
            label = m.group(1)
            for j in range(i + 1, len(body)):
                if re.match(r"^\s*s_c?branch\w*\s+%s\s*$" % re.escape(label), body[j]):
                    out.append((i, body[i:j + 1]))
                    break
    return out


def _events(lines):
    """Sequence of ('load', is_dma) and ('ringwait', n) events."""
    ev = []
    instr = [l for l in lines if l.strip() and not l.strip().startswith(";")
             and not re.match(r"^\s*\.", l) and not re.match(r"^\.LBB", l)]
    for i, line in enumerate(instr):
        if VMEM.match(line):
            ev.append(("load", " lds" in line))
        m = WAIT.match(line)
        if m and i + 1 < len(instr) and re.match(r"^\s*s_barrier\b", instr[i + 1]):
            ev.append(("ringwait", int(m.group(1))))
    return ev


def _check_kernel(name, body, ns, extra0=0, batch=None):
    """extra0: DMAs that follow stage 0's batch in the prologue and must have
    landed at the first wait too (the register-filter kernel's prologue
    filter taps).  batch: DMAs per wave per stage; by default the prologue
    holds NS-1 whole batches (stages 0..NS-2), else it may also run the
    first ring stages ahead of the loop (each issuing one batch more)."""
    pro, loop = _split(body)
    pro_ev, loop_ev = _events(pro), _events(loop)
    n_dma_pro = sum(1 for e in pro_ev if e == ("load", True))
    if batch is None:
        assert (n_dma_pro - extra0) % (ns - 1) == 0, (name, n_dma_pro)
        batch = (n_dma_pro - extra0) // (ns - 1)
    assert (n_dma_pro - extra0) % batch == 0 and n_dma_pro - extra0 >= (ns - 1) * batch, (
        name, n_dma_pro)
    assert batch > 0, name
    assert loop_ev, "%s: no stage loop found" % name
    seq = []            # per load: DMA batch index or None
    dmas = 0
    waits = 0
    for kind, val in pro_ev + loop_ev * 4:
        if kind == "load":
            if val:
                seq.append(0 if dmas < batch + extra0 else (dmas - extra0) // batch)
                dmas += 1
            else:
                seq.append(None)
            continue
        waits += 1
        retired = len(seq) - val
        pending = [b for b in seq[max(retired, 0):] if b is not None]
        assert all(b >= waits for b in pending), (
            "%s: ring wait %d (vmcnt(%d)) leaves a DMA of stage %d in flight"
            % (name, waits, val, min(pending)))
    assert waits >= 5, (name, waits)


@pytest.fixture(scope="module")
def halo_asm():
    return hip_build.device_asm("conv_i8_halo.hip")


def test_register_filter_kernels_ring_waits(halo_asm):
    # The kernels that mix LDS-DMAs with ordinary loads into registers.  In
    # the all-DMA kernels every vmcnt event is a DMA, and DMAs (LDS writes)
    # keep their program order, so their counts cannot be disturbed.
    fns = _functions(halo_asm, "_ZN9convfprop22conv_i8_halo_ad_kernel")
    assert len(fns) >= 3
    for name, body in fns.items():
        ints = _template_ints(name)  # <WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, AL, SW, PT, RG>
        wk, wp, fk, _, r, s, ns = ints[:7]
        if len(ints) > 13 and ints[13]:
            # halo through registers: the ring has no LDS-DMA (the compiler
            # places the waits for its ordinary loads); only the prologue's
            # filter taps come by DMA, awaited in full before the first barrier
            for _, lp in _loops(body):
                assert not any(VMEM.match(l) and " lds" in l for l in lp), name
            continue
        # the prologue's filter taps 0..A-1, A = min(R*S-1, 4) taps ahead (the
        # kernel's halo_filter_ahead): A*WK*FK blocks over WK*WP waves; with
        # the filter in the LDS ring (AL) they are part of stage 0
        ahead = min(r * s - 1, 4)
        aj = 0 if ints[10] else (ahead * wk * fk + wk * wp - 1) // (wk * wp)
        # DMAs per wave per stage: the halo blocks of its CPS channel blocks,
        # and with AL the filter blocks of its taps
        hj, cps = ints[7], ints[9]
        fj = ((r * s * cps) * (wk * fk) + wk * wp - 1) // (wk * wp) if ints[10] else 0
        _check_kernel(name, body, ns, aj, batch=hj * cps + fj)
        # A tile with a short last wave column runs its main loop twice over
        # (full and short waves): both loops must issue the same loads and
        # waits in the same order, so the check of the first covers both.
        loops = [lp for _, lp in _loops(body) if any("v_mfma" in l for l in lp)]
        pt = ints[12] if len(ints) > 12 else 0
        if pt:
            assert len(loops) == 2, (name, len(loops))
        for lp in loops[1:]:
            assert _events(lp) == _events(loops[0]), name


def test_checker_catches_a_wait_that_is_too_loose():
    # Prologue: 2 stages of 2 DMAs in flight; vmcnt(3) lets stage 0's second
    # DMA retire late, vmcnt(2) does not.  In the loop one register load
    # follows the last batch, so vmcnt(1) covers stage 1 but vmcnt(2) would
    # not.
    body = [
        "\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds",
        "\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds",
        "\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds",
        "\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds",
        "\ts_waitcnt vmcnt(3) lgkmcnt(0)",
        "\ts_barrier",
        ".LBB0_1:  ; =>This Inner Loop Header: Depth=1",
        "\tbuffer_load_dwordx4 v[2:5], v1, s[0:3], 0 offen",
        "\ts_waitcnt vmcnt(1) lgkmcnt(0)",
        "\ts_barrier",
        "\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds",
        "\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds",
        "\ts_cbranch_scc1 .LBB0_1",
        "\ts_endpgm",
    ]
    with pytest.raises(AssertionError, match="ring wait 1"):
        _check_kernel("synthetic", body, 3)
    body[4] = "\ts_waitcnt vmcnt(2) lgkmcnt(0)"
    _check_kernel("synthetic", body, 3)
    body[8] = "\ts_waitcnt vmcnt(2) lgkmcnt(0)"
    with pytest.raises(AssertionError, match="ring wait 2"):
        _check_kernel("synthetic", body, 3)


def test_checker_counts_prologue_extras_into_stage_0():
    # Stage 0 (1 DMA) plus one extra DMA that must land with it, then stage 1.
    body = [
        "\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds",
        "\tbuffer_load_dwordx4 v1, s[4:7], 0 offen lds",
        "\ts_waitcnt vmcnt(0) lgkmcnt(0)",
        "\ts_barrier",
        "\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds",
        ".LBB0_1:  ; =>This Inner Loop Header: Depth=1",
        "\ts_waitcnt vmcnt(0) lgkmcnt(0)",
        "\ts_barrier",
        "\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds",
        "\ts_cbranch_scc1 .LBB0_1",
        "\ts_endpgm",
    ]
    _check_kernel("synthetic", body, 3, extra0=1)
    body[2] = "\ts_waitcnt vmcnt(1) lgkmcnt(0)"   # the extra DMA may still be in flight
    with pytest.raises(AssertionError, match="ring wait 1"):
        _check_kernel("synthetic", body, 3, extra0=1)
