"""Instruction-order property of the packed-layout GEMV that its correctness
rests on, checked on the gfx950 assembly the compiler produces (no GPU).

The K-chunk-0 workgroup of a row block zeroes the block's outputs, then issues
its first weight loads, then waits with a hand-written ``s_waitcnt vmcnt(N)``
before it advances the generation words that let the other K chunks add into
those outputs.  vmcnt counts vector-memory operations in issue order, so the
wait covers the zero store only if exactly N vector-memory operations -- the
weight loads -- sit between the zero store and the wait.  A compiler that
moved a load above the zero store, or added a memory operation in between,
would turn the wait into a race; this test fails instead.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gemm_hadamard_rotated_amd", "csrc")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def packed_asm(tmp_path_factory):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    from gemm_hadamard_rotated_amd import build
    out = tmp_path_factory.mktemp("isa") / "gemv_packed.s"
    flags = [f for f in build.flags_for("gemv_packed.hip") if f not in ("-fPIC",)]
    cmd = [cc, *flags, "--cuda-device-only", "-S", "-o", str(out),
           os.path.join(CSRC, "gemv_packed.hip")]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout[-4000:]
    return out.read_text()


def _kernels(asm, name):
    return re.findall(rf"^(_ZN\w*{name}\w+):[^\n]*\n(.*?)s_endpgm", asm, re.S | re.M)


def test_zeroing_wait_counts_exactly_the_weight_loads(packed_asm):
    kernels = _kernels(packed_asm, "gemv_packed_kernel")
    assert len(kernels) >= 18, "expected every packed GEMV instantiation in the assembly"
    checked = 0
    for name, body in kernels:
        lines = [l.strip() for l in body.splitlines()]
        waits = [(i, int(m.group(1))) for i, l in enumerate(lines)
                 if (m := re.match(r"s_waitcnt vmcnt\((\d+)\)$", l)) and i > 0
                 and lines[i - 1] == ";;#ASMSTART"]
        hand = [(i, n) for i, n in waits if n > 0]
        assert len(hand) == 1, f"{name}: expected one hand-written non-zero vmcnt wait"
        i, n = hand[0]
        stores = [j for j in range(i) if lines[j].startswith("global_store_dword") and "sc1" in lines[j]]
        assert stores, f"{name}: no coherent zero store before the wait"
        z = stores[-1]
        vmem = [lines[j].split()[0] for j in range(z + 1, i)
                if re.match(r"(global_|buffer_|flat_|scratch_)", lines[j])]
        assert len(vmem) == n, f"{name}: {len(vmem)} memory operations between the zero store " \
                               f"and vmcnt({n}): {vmem}"
        assert all("load" in v for v in vmem), f"{name}: non-load between zero store and wait: {vmem}"
        checked += 1
    assert checked == len(kernels)


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    from gemm_hadamard_rotated_amd import build
    out = tmp_path_factory.mktemp("isa") / "gemm.s"
    flags = [f for f in build.flags_for("gemm.hip") if f not in ("-fPIC",)]
    cmd = [cc, *flags, "--cuda-device-only", "-S", "-o", str(out), os.path.join(CSRC, "gemm.hip")]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout[-4000:]
    return out.read_text()


def test_gemm_barrier_waits_cover_the_lds_copies(gemm_asm):
    """The prefill GEMM tiles copy the next group of X straight into LDS
    (buffer loads with the `lds` modifier), then load the weights and scale
    two groups ahead into registers, and wait with vmcnt(n) before the
    group's barrier: n leaves those register loads in flight.  vmcnt counts
    vector-memory operations in issue order, so the copies have landed only
    if at least n vector-memory operations follow the last copy before the
    wait.  A compiler that moved a register load above the copies would make
    the barrier release waves into a half-written tile; this test fails
    instead."""
    kernels = _kernels(gemm_asm, "gemm_xg")
    assert len(kernels) == 2, "expected the two tile kernels"
    for name, body in kernels:
        lines = [l.strip() for l in body.splitlines()]
        barriers = [i for i, l in enumerate(lines) if l == "s_barrier"]
        assert len(barriers) >= 12, f"{name}: expected the unrolled loop's barriers"
        partial = 0
        for b in barriers:
            # the last wait before the barrier (the compiler may merge it with an
            # earlier LDS wait); no vector-memory operation may lie between them
            w = next(j for j in range(b - 1, -1, -1) if lines[j].startswith("s_waitcnt"))
            between = [lines[j] for j in range(w + 1, b)
                       if re.match(r"(global_|buffer_|flat_|scratch_)", lines[j])]
            assert not between, f"{name}: memory operations between the wait and the barrier " \
                                f"at line {b}: {between}"
            m = re.search(r"vmcnt\((\d+)\)", lines[w])
            if not m:
                continue
            n = int(m.group(1))
            dma = [j for j in range(w) if re.match(r"(buffer|global)_load\w* .*\blds\b", lines[j])]
            assert dma, f"{name}: no LDS copy before the wait at line {w}"
            after = [lines[j].split()[0] for j in range(dma[-1] + 1, w)
                     if re.match(r"(global_|buffer_|flat_|scratch_)", lines[j])]
            assert len(after) >= n, f"{name}: vmcnt({n}) at line {w} but only {len(after)} memory " \
                                    f"operations after the last LDS copy: {after}"
            partial += n > 0
        assert partial >= 6, f"{name}: expected the loop's barriers to leave loads in flight"
