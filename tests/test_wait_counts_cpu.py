"""The hand-set memory waits of the multi-stage tile loops, checked on the compiler's output.

The direct-to-LDS tile kernels (three or four LDS stages, `lds_ring`) keep NST - 1 K-steps
of loads in flight and, before a step's barrier, wait with an explicit
`s_waitcnt vmcnt(N)` for the stage the next step reads.  N is set from the number of
loads a wave issues per step.  Loads complete in issue order, so the wait is safe exactly
when N is at most the number of loads issued after that stage's: the loads of the
current step plus those of the NST - 3 steps before it.  If the compiler moved a load
across a wait or a barrier, or a loader issued a different number of loads than the wait
assumes, the next step could read a stage that has not landed.

The one-token weight-streaming kernel (X row staged in LDS) has the same hazard: each
wave owns a four-stage ring with three stages in flight and waits explicitly for the
stage it reads (no barriers there; its waves never synchronise inside the loop).

This test compiles the kernels to gfx950 assembly (hipcc, no GPU needed), finds each
ring kernel's steady-state loop, and replays its body (three trips, so that the groups
before the first waits come from the previous trips) with a count of loads per step
(steps are delimited by the barriers, or for the per-wave rings by the waits),
checking every vmcnt wait against that bound.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "semi_structured_sparse_amd", "csrc")


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _assembly(src, tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           "-o", str(out), os.path.join(CSRC, src)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return out.read_text()


def _functions(asm, name):
    """(mangled name, body lines) of every kernel whose name contains `name`."""
    out = []
    for m in re.finditer(r"^(_Z\w*" + name + r"\w*):", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        out.append((m.group(1), asm[m.end():end].splitlines()))
    return out


def _template_ints(mangled):
    """Integer and bool template arguments of a mangled kernel name, in order."""
    args = re.search(r"I((?:L[ib]n?\d+E)+)E", mangled).group(1)
    return [int(v.replace("n", "-")) for v in re.findall(r"L[ib](n?\d+)E", args)]


def _loops(lines):
    """Bodies (instruction lines) of the innermost loops: from a loop header label to the
    branch back to it."""
    loops = []
    for i, ln in enumerate(lines):
        m = re.match(r"^(\.LBB\w+):.*Loop Header", ln)
        if not m:
            continue
        label = m.group(1)
        for j in range(i + 1, len(lines)):
            if re.match(r"^\s*s_cbranch_\w+\s+" + re.escape(label) + r"\s*$", lines[j]):
                loops.append(lines[i + 1:j + 1])
                break
    return loops


def _events(body):
    ev = []
    for ln in body:
        t = ln.strip()
        if t.startswith("global_load_lds_"):
            ev.append(("load",))
        elif t.startswith("s_barrier"):
            ev.append(("bar",))
        elif t.startswith("s_waitcnt"):
            m = re.search(r"vmcnt\((\d+)\)", t)
            if m:
                ev.append(("wait", int(m.group(1))))
        elif t.startswith(("global_load", "buffer_load", "flat_load")):
            ev.append(("vload",))   # any other vector-memory load also counts in vmcnt
    return ev


def _check_ring_loop(ev, nst, label):
    """Replay three trips of a loop body; at each vmcnt wait after the first trip, the
    loads issued after the stage the next step reads (this step's, and those of the
    nst - 3 steps before it) must number at least N."""
    groups, cur, trip_len = [], 0, len(ev)
    checked = 0
    for idx, e in enumerate(ev * 3):
        if e[0] in ("load", "vload"):
            cur += 1
        elif e[0] == "bar":
            groups.append(cur)
            cur = 0
        elif e[0] == "wait" and idx >= trip_len:
            later = cur + sum(groups[len(groups) - (nst - 3):]) if nst > 3 else cur
            assert e[1] <= later, (f"{label}: s_waitcnt vmcnt({e[1]}) lets the loads of a stage still in flight "
                                   f"({later} loads issued after it)")
            checked += 1
    return checked


def _check_stream_loop(ev, depth, label):
    """Per-wave rings with no barriers (the one-token weight-streaming kernels): each stage
    issues its loads, then waits for the stage it reads, issued `depth` stages earlier.
    Intervals between waits hold one stage's loads, so at each wait N must not exceed the
    loads of the last `depth` intervals (this one included)."""
    intervals, cur, trip_len, checked = [], 0, len(ev), 0
    for idx, e in enumerate(ev * 3):
        if e[0] in ("load", "vload"):
            cur += 1
        elif e[0] == "wait":
            intervals.append(cur)
            cur = 0
            if idx >= trip_len:
                later = sum(intervals[-depth:])
                assert e[1] <= later, (f"{label}: s_waitcnt vmcnt({e[1]}) lets the loads of a stage still in flight "
                                       f"({later} loads issued after it)")
                checked += 1
    return checked


def test_stream_waits_cover_their_stage(tmp_path):
    """The weight-streaming kernel with its X row staged in LDS (one token): the four-
    stage per-wave ring's explicit waits (three stages in flight), on its steady-state loop."""
    asm = _assembly("decode.hip", tmp_path)
    # k_fewd<TB, WK0, XL0, NS, WK1, XS, SELM, QNS, RWV>: XS is the sixth argument
    kernels = [(n, b) for n, b in _functions(asm, "k_fewdI") if _template_ints(n)[5] == 1]
    assert kernels, "no k_fewd instantiation with the staged X row"
    n_loops = 0
    for name, body in kernels:
        for lp in _loops(body):
            ev = _events(lp)
            n_load = sum(1 for e in ev if e[0] == "load")
            n_wait = sum(1 for e in ev if e[0] == "wait")
            if n_load >= 8 and n_wait >= 4:   # the steady state: four stages per trip
                assert _check_stream_loop(ev, 3, name) >= 4
                n_loops += 1
    assert n_loops > 0, "no steady-state ring loop found"


@pytest.mark.parametrize("src,kernel,nst_index", [
    ("gemm_lds.hip", "k_gemm_lds", 7),      # <BM, BN, WM, WN, PRO, W8, KH, NST>
    ("gemm_lds_sp.hip", "k_gemm_lds_sp", 6),  # <BM, BN, WM, WN, MB, F8, NST>
])
def test_ring_waits_cover_their_stage(src, kernel, nst_index, tmp_path):
    asm = _assembly(src, tmp_path)
    kernels = [(n, b) for n, b in _functions(asm, kernel + "I") if _template_ints(n)[nst_index] >= 3]
    assert kernels, f"no {kernel} instantiation with three or more stages"
    for name, body in kernels:
        nst = _template_ints(name)[nst_index]
        rings = []
        for lp in _loops(body):
            ev = _events(lp)
            if any(e[0] == "load" for e in ev) and any(e[0] == "bar" for e in ev):
                rings.append(ev)
        assert rings, f"{name}: no loop with direct-to-LDS loads and barriers"
        for ev in rings:
            n_bar = sum(1 for e in ev if e[0] == "bar")
            n_wait = sum(1 for e in ev if e[0] == "wait")
            # a whole trip: NST steps, each one barrier and one wait for its stage
            assert n_bar == nst and n_wait >= nst, (name, n_bar, n_wait)
            assert _check_ring_loop(ev, nst, name) >= nst
