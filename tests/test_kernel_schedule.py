"""The product kernels' hand-counted memory waits against their compiled code.

The 8-bit tile kernels load each k-step's weight slice straight into LDS
(buffer_load ... lds) and publish it to the other waves with an explicit
vmcnt(N) wait plus a barrier: loads complete in order, so vmcnt(N) means
every load but the last N has landed.  That count is only right if the
compiler issues the loads where the source puts them; a compiler that peeled
the first loop iteration and sank its activation loads past the exit test
once left too few loads behind two slices, so other waves could read a slice
before it had landed.

These tests compile k_gemm.hip for gfx950 with the library's flags (no GPU
needed), take each 8-bit tile kernel's prologue and k loop from the
assembly, and replay the wave's issue order: at every barrier, each slice
that the next step reads must be covered by a wait issued before it (slice s
is read from step s - 1 on, and before the loop for s = 0).  Three loop
iterations are replayed, so the steady state is checked too.  The 4-bit
tile kernel, which stages its slices with LDS stores and an lgkmcnt wait,
is checked the same way on its LDS operations.
"""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "w8a8_post_quantization_sq_amd", "csrc", "k_gemm.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    sys.path.insert(0, ROOT)
    from w8a8_post_quantization_sq_amd import build
    out = str(tmp_path_factory.mktemp("asm") / "k_gemm.s")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.hipcc(), *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.dirname(SRC), "-x", "hip", SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def kernel_body(text, mangled_prefix):
    """Assembly lines of every kernel whose symbol starts with the prefix."""
    out = {}
    for m in re.finditer(r"^(" + re.escape(mangled_prefix) + r"\w*):", text, re.M):
        end = text.find(".Lfunc_end", m.end())
        out[m.group(1)] = text[m.end():end].split("\n")
    return out


def events(lines):
    """The wave's memory events in issue order: D (load into LDS), L (other
    vector memory access, counted by vmcnt), W<n> (s_waitcnt with vmcnt),
    B (s_barrier), plus loop markers ('H', label) and back-branches ('J', label)."""
    ev = []
    label = None
    for raw in lines:
        s = raw.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":") and s.startswith(".LBB"):
            label = s[:-1]
            if "Loop Header" in raw:
                ev.append(("H", label))
            continue
        op = s.split()[0]
        if op.startswith("buffer_load") and s.split()[-1] == "lds":
            ev.append(("D", None))
        elif op.startswith(("buffer_load", "global_load", "buffer_store", "global_store",
                            "buffer_atomic", "global_atomic")):
            ev.append(("L", None))
        elif op == "s_waitcnt" and "vmcnt(" in s:
            ev.append(("W", int(s.split("vmcnt(")[1].split(")")[0])))
        elif op == "s_barrier":
            ev.append(("B", None))
        elif op.startswith("s_cbranch") or op == "s_branch":
            ev.append(("J", s.split()[-1]))
    return ev


def prologue_and_loop(ev):
    """Events before the k loop's header (from the first LDS load on) and the
    loop body up to its back-branch."""
    first = next(i for i, e in enumerate(ev) if e[0] == "D")
    hdr = next(i for i in range(first, len(ev)) if ev[i][0] == "H")
    label = ev[hdr][1]
    back = next(i for i in range(hdr + 1, len(ev)) if ev[i] == ("J", label))
    pro = [e for e in ev[first:hdr] if e[0] in "DLWB"]
    body = [e for e in ev[hdr + 1:back] if e[0] in "DLWB"]
    return pro, body


def replay(pro, body, slice_dmas, iterations=3):
    """Checks that at barrier k (0 = the prologue's, k = the end of step k - 1)
    every load of slices 0 .. k + 1 is complete.  A wait vmcnt(n) completes
    every access issued before it except the last n.  slice_dmas: LDS loads
    per slice and wave."""
    seq = pro + body * iterations
    issued = []          # kinds of the accesses issued so far
    done = 0             # accesses known complete (a prefix, loads complete in order)
    barrier = 0
    checked = 0
    for kind, arg in seq:
        if kind in "DL":
            issued.append(kind)
        elif kind == "W":
            done = max(done, len(issued) - arg)
        elif kind == "B":
            dmas_done = sum(1 for k in issued[:done] if k == "D")
            need = (barrier + 2) * slice_dmas        # slices 0 .. barrier + 1
            dmas_issued = issued.count("D")
            if need <= dmas_issued or barrier < 2:
                assert dmas_done >= min(need, dmas_issued), (
                    f"barrier {barrier}: slices up to {barrier + 1} need {need} LDS loads "
                    f"complete, only {dmas_done} of {dmas_issued} are")
                checked += 1
            barrier += 1
    return checked


def test_tile_kernel_waits_cover_every_slice(asm):
    kernels = kernel_body(asm, "_ZN2sq11k_gemm_tileIL")
    eight_bit = {k: v for k, v in kernels.items() if re.match(r"_ZN2sq11k_gemm_tileILb[01]ELb0E", k)}
    assert len(eight_bit) == 2, sorted(kernels)
    for name, lines in eight_bit.items():
        pro, body = prologue_and_loop(events(lines))
        # the source's shape: 4 slices and 3 activation steps before the loop,
        # 1 slice and 2 activation fragments per step, 4 steps per iteration
        assert [k for k, _ in pro].count("D") == 4, name
        assert [k for k, _ in body].count("D") == 4 and [k for k, _ in body].count("B") == 4, name
        assert [k for k, _ in body].count("L") == 8, name
        # no peeled steps between the prologue's barrier and the loop
        assert [k for k, _ in pro].count("B") == 1, name
        assert replay(pro, body, slice_dmas=1) >= 12, name


def test_wide_kernel_waits_cover_every_slice(asm):
    kernels = kernel_body(asm, "_ZN2sq11k_gemm_wideIL")
    assert len(kernels) == 2, sorted(kernels)
    for name, lines in kernels.items():
        pro, body = prologue_and_loop(events(lines))
        assert [k for k, _ in pro].count("D") == 8, name
        assert [k for k, _ in body].count("D") == 8 and [k for k, _ in body].count("B") == 4, name
        assert [k for k, _ in pro].count("B") == 1, name
        assert replay(pro, body, slice_dmas=2) >= 12, name


def lds_events(lines):
    """LDS-side events in issue order: S (LDS store), R (LDS read), M (scalar
    memory load, which also counts in lgkmcnt and completes out of order),
    G<n> (s_waitcnt with lgkmcnt), B (s_barrier), plus loop markers."""
    ev = []
    for raw in lines:
        s = raw.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":") and s.startswith(".LBB"):
            if "Loop Header" in raw:
                ev.append(("H", s[:-1]))
            continue
        op = s.split()[0]
        if op.startswith(("ds_write", "ds_store")):
            ev.append(("S", None))
        elif op.startswith(("ds_read", "ds_load")):
            ev.append(("R", None))
        elif op.startswith(("s_load", "s_buffer_load")):
            ev.append(("M", None))
        elif op == "s_waitcnt" and "lgkmcnt(" in s:
            ev.append(("G", int(s.split("lgkmcnt(")[1].split(")")[0])))
        elif op == "s_barrier":
            ev.append(("B", None))
        elif op.startswith("s_cbranch") or op == "s_branch":
            ev.append(("J", s.split()[-1]))
    return ev


def test_four_bit_tile_kernel_publishes_each_staged_slice(asm):
    """The 4-bit tile kernel stages each widened weight slice with an LDS
    store and ends the step on lgkmcnt(n) and a barrier: LDS operations of a
    wave complete in order, so the store has landed if at least n LDS
    operations follow it before the wait (and no scalar load, which counts
    in the same counter out of order, is pending in the loop)."""
    kernels = kernel_body(asm, "_ZN2sq11k_gemm_tileIL")
    four_bit = {k: v for k, v in kernels.items() if re.match(r"_ZN2sq11k_gemm_tileILb[01]ELb1E", k)}
    assert len(four_bit) == 2, sorted(kernels)
    for name, lines in four_bit.items():
        ev = lds_events(lines)
        hdr = next(i for i, e in enumerate(ev) if e[0] == "H")
        back = next(i for i in range(hdr + 1, len(ev)) if ev[i] == ("J", ev[hdr][1]))
        body = [e for e in ev[hdr + 1:back] if e[0] in "SRMGB"]
        assert not any(k == "M" for k, _ in body), name
        steps, cur = [], []
        for e in body:
            if e[0] == "B":
                steps.append(cur)
                cur = []
            else:
                cur.append(e)
        assert len(steps) == 4, name
        for step in steps:
            kinds = [k for k, _ in step]
            assert kinds.count("S") == 1, (name, kinds)
            s = kinds.index("S")
            waits = [i for i, (k, _) in enumerate(step) if k == "G" and i > s]
            assert waits, (name, kinds)
            w = waits[-1]
            after = sum(1 for k in kinds[s + 1:w] if k in "SR")
            assert after >= step[w][1], (name, kinds)


def test_replay_catches_a_peeled_first_iteration():
    """The checker itself: the schedule the compiler once produced (steps 1..3
    of the first iteration issuing their slice but not their activation
    fragments, with vmcnt(8) at step ends) must fail, and the intended
    one must pass."""
    D, L, B = ("D", None), ("L", None), ("B", None)
    W = lambda n: ("W", n)
    pro = [D, L, L, D, L, L, D, L, L, D, W(0), B]
    step = [D, L, L, W(8), B]
    assert replay(pro, step * 4, slice_dmas=1) >= 12
    peeled = pro + [D, L, L, W(6), B, D, W(6), B, D, W(8), B, D, W(8), B] + [L] * 6
    with pytest.raises(AssertionError):
        replay(peeled, step * 4, slice_dmas=1)
