"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments before touching the HIP
runtime (validation returns an error code without any device work)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT, gpu_available

HEADER = os.path.join(ROOT, "include", "pq1.h")


@pytest.fixture(scope="module")
def lib():
    from gemm_hadamard_rotated_amd import pq1
    if not os.path.exists(pq1.LIB_PATH):
        from gemm_hadamard_rotated_amd import build
        build.build()
    return pq1.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pq1_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("pq1_rotate", "pq1_gemv", "pq1_gemm", "pq1_rotate_gemv", "pq1_gemv_ex",
              "pq1_gemv_workspace_bytes", "pq1_status_str", "pq1_abi_version",
              "pq1_last_hip_error", "pq1_pack_weights", "pq1_gemv_packed",
              "pq1_rotate_gemv_packed", "pq1_packed_bits_bytes", "pq1_packed_scales_bytes",
              "pq1_pack_weights_rows", "pq1_embed", "pq1_packed_scales_bytes_ex",
              "pq1_pack_weights_ex", "pq1_gemv_packed_ex", "pq1_rotate_gemv_packed_ex",
              "pq1_gemm_ex", "pq1_set_test_flags"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from gemm_hadamard_rotated_amd import pq1
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(pq1.EXPORTS)


def test_abi_version_and_status_strings(lib):
    assert lib.pq1_abi_version() == 4
    for code in range(0, 10):
        s = lib.pq1_status_str(code)
        assert s and len(s) > 1
    assert lib.pq1_status_str(1234) == b"unknown status"


def test_counter_region_constant_matches_header():
    from gemm_hadamard_rotated_amd import pq1
    m = re.search(r"#define\s+PQ1_GEMV_COUNTER_BYTES\s+(\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == pq1.PQ1_GEMV_COUNTER_BYTES


def test_workspace_bytes(lib):
    f = lib.pq1_gemv_workspace_bytes
    assert f(0, 1024) == 0 and f(16, 100) == 0 and f(16, 0) == 0
    for N, K in ((256, 1024), (17408, 5120), (5120, 17408), (5120, 6144), (1000, 640)):
        b = f(N, K)
        assert b % 256 == 0 and b >= 262144
        # counters + at most one fp32 partial per row and K-tile of 256
        assert b <= 262144 + ((K + 255) // 256) * N * 4 + 256


A = 0x10000  # fake, 16-byte aligned "device" addresses: never dereferenced


def P(v):
    return ctypes.c_void_p(v)


def test_rotate_validation(lib):
    from gemm_hadamard_rotated_amd.pq1 import Pq1Perm
    r = lib.pq1_rotate
    assert r(None, P(A), None, P(2 * A), 0, 1, 1024, None) == 1           # NULL x
    assert r(P(A), P(2 * A), None, None, 0, 1, 1024, None) == 1           # NULL out
    assert r(P(A), P(2 * A), None, P(3 * A), 0, 1, 1000, None) == 2       # K % 1024
    assert r(P(A), P(2 * A), None, P(3 * A), 0, 0, 1024, None) == 2       # M < 1
    assert r(P(A), P(2 * A), None, P(3 * A), 7, 1, 1024, None) == 8       # bad dtype
    assert r(P(A), P(2 * A), None, P(3 * A), 3, 1, 1024, None) == 8
    assert r(P(A + 4), P(2 * A), None, P(3 * A), 0, 1, 1024, None) == 3   # misaligned
    bad = Pq1Perm(128, 16, 3)                                              # 6144 != 5120
    assert r(P(A), P(2 * A), ctypes.byref(bad), P(3 * A), 0, 1, 5120, None) == 4
    odd = Pq1Perm(130, 16, 3)
    assert r(P(A), P(2 * A), ctypes.byref(odd), P(3 * A), 0, 1, 6240, None) == 2  # 6240 % 1024
    neg = Pq1Perm(0, 16, 3)
    assert r(P(A), P(2 * A), ctypes.byref(neg), P(3 * A), 0, 1, 6144, None) == 4
    assert r(P(A), P(A + 4096), None, P(A), 0, 1, 1024, None) == 5         # out == x


def test_gemv_validation(lib):
    g = lib.pq1_gemv_ex
    x, w, s, y, ws = A, 2 * A, 4 * A, 8 * A, 1 << 40
    big = 1 << 30
    assert g(None, P(w), P(s), P(y), 16, 1024, 0, P(ws), big, None) == 1
    assert g(P(x), None, P(s), P(y), 16, 1024, 0, P(ws), big, None) == 1
    assert g(P(x), P(w), P(s), P(y), 16, 100, 0, P(ws), big, None) == 2      # K % 128
    assert g(P(x), P(w), P(s), P(y), 0, 1024, 0, P(ws), big, None) == 2      # N < 1
    assert g(P(x), P(w), P(s + 8), P(y), 16, 1024, 0, P(ws), big, None) == 3
    assert g(P(x), P(w), P(s), P(y), 16, 1024, 9, P(ws), big, None) == 8     # algo
    assert g(P(x), P(w), P(s), P(w), 16, 1024, 0, P(ws), big, None) == 5     # y over w_bits
    # a split-K plan needs a 256-byte-aligned workspace of sufficient size
    need = lib.pq1_gemv_workspace_bytes(5120, 17408)
    assert g(P(x), P(w), P(s), P(y), 5120, 17408, 0, None, big, None) == 1
    assert g(P(x), P(w), P(s), P(y), 5120, 17408, 0, P(ws + 16), big, None) == 3
    assert g(P(x), P(w), P(s), P(y), 5120, 17408, 0, P(ws), need - 256, None) == 8
    # workspace overlapping the output
    assert g(P(x), P(w), P(s), P(y), 5120, 17408, 0, P(y - 256), big, None) == 5


def test_gemm_and_fused_validation(lib):
    # pq1_gemm(x_rot_bf16, w_bits, scales, y, M, N, K, stream): the argument
    # order of the problem statement's call
    g = lib.pq1_gemm
    x, w, s, y = A, 2 * A, 4 * A, 8 * A
    assert g(None, P(w), P(s), P(y), 4, 16, 1024, None) == 1
    assert g(P(x), None, P(s), P(y), 4, 16, 1024, None) == 1
    assert g(P(x), P(w), None, P(y), 4, 16, 1024, None) == 1
    assert g(P(x), P(w), P(s), None, 4, 16, 1024, None) == 1
    assert g(P(x), P(w), P(s), P(y), 0, 16, 1024, None) == 2
    assert g(P(x), P(w), P(s), P(y), 4, 0, 1024, None) == 2
    assert g(P(x), P(w), P(s), P(y), 4, 16, 1000, None) == 2
    assert g(P(x + 2), P(w), P(s), P(y), 4, 16, 1024, None) == 3
    assert g(P(x), P(w + 4), P(s), P(y), 4, 16, 1024, None) == 3
    assert g(P(x), P(w), P(s), P(x), 4, 16, 1024, None) == 5      # y over x
    assert g(P(x), P(w), P(s), P(w), 4, 16, 1024, None) == 5      # y over w_bits
    assert g(P(x), P(w), P(s), P(y), 1, 1, 1 << 28, None) == 2   # K too large
    assert g(P(x), P(w), P(s), P(y), 1, 1, (1 << 28) - 128, None) != 2
    ge = lib.pq1_gemm_ex
    assert ge(P(x), P(w), P(s), P(y), 4, 16, 1024, 7, None) == 8   # unknown layout
    assert ge(P(x), P(w), P(s), P(y), 4, 16, 1024, -1, None) == 8
    assert ge(None, P(w), P(s), P(y), 4, 16, 1024, 1, None) == 1
    assert ge(P(x), P(w), P(s), P(y), 4, 16, 1000, 1, None) == 2
    f = lib.pq1_rotate_gemv
    assert f(P(x), P(A // 2), None, P(w), P(s), P(y), 16, 1152, P(16 * A), 1 << 30, None) == 2
    assert f(None, P(A // 2), None, P(w), P(s), P(y), 16, 1024, P(16 * A), 1 << 30, None) == 1


def test_gemv_plans_beyond_the_counters_are_refused(lib):
    # With K split into tiles the canonical-layout kernels have one arrival
    # counter per row block (8192 of them): N = 3,000,000 rows at K = 2048
    # needs 11,719 row blocks of 256 rows.  Every kernel is compiled for its K
    # tile, so the call must refuse the shape rather than drop the split.
    B = 1 << 40  # made-up, far-apart device addresses
    x, w, s, y, ws = B, 2 * B, 3 * B, 4 * B, 5 * B
    for algo in (0, 1, 2):
        assert lib.pq1_gemv_ex(P(x), P(w), P(s), P(y), 3_000_000, 2048, algo, P(ws), 1 << 40,
                               None) == 2
    assert lib.pq1_rotate_gemv(P(x), P(x + (1 << 20)), None, P(w), P(s), P(y), 3_000_000, 2048,
                               P(ws), 1 << 40, None) == 2
    # one K tile needs no counters: any row count the element limit allows
    big = 16_000_000
    if not gpu_available():
        assert lib.pq1_gemv_ex(P(x), P(w), P(s), P(y), big, 1024, 0, None, 0, None) == 6
        assert lib.pq1_rotate_gemv(P(x), P(x + (1 << 20)), None, P(w), P(s), P(y), big, 1024,
                                   None, 0, None) == 6
    # the largest split plans still pass validation
    if not gpu_available():
        assert lib.pq1_gemv_ex(P(x), P(w), P(s), P(y), 8192 * 256, 2048, 1, P(ws), 1 << 40,
                               None) == 6
        assert lib.pq1_gemv_ex(P(x), P(w), P(s), P(y), 8192 * 256 + 1, 2048, 1, P(ws), 1 << 40,
                               None) == 2
        assert lib.pq1_gemv_ex(P(x), P(w), P(s), P(y), 8192 * 128, 2048, 2, P(ws), 1 << 40,
                               None) == 6
        assert lib.pq1_gemv_ex(P(x), P(w), P(s), P(y), 8192 * 128 + 1, 2048, 2, P(ws), 1 << 40,
                               None) == 2


def test_status_word_constants_match_header():
    from gemm_hadamard_rotated_amd import pq1
    text = open(HEADER).read()
    for name in ("PQ1_GEMV_STATUS_OFFSET", "PQ1_SPLITK_WAIT_GAVE_UP", "PQ1_SPLITK_OUT_OF_STEP",
                 "PQ1_TEST_WITHHOLD_PUBLISH"):
        m = re.search(rf"#define\s+{name}\s+(\d+)u?", text)
        assert m and int(m.group(1)) == getattr(pq1, name), name
    m = re.search(r"PQ1_ERR_SPLITK\s*=\s*(\d+)", text)
    assert m and int(m.group(1)) == pq1.PQ1_ERR_SPLITK
    # the status word sits inside the counter region, past every generation /
    # seen pair of the packed layout and 4-byte aligned
    assert pq1.PQ1_GEMV_STATUS_OFFSET % 256 == 0
    assert pq1.PQ1_GEMV_STATUS_OFFSET + 4 <= pq1.PQ1_GEMV_COUNTER_BYTES


def test_test_flags_round_trip(lib):
    assert lib.pq1_set_test_flags(1) == 0
    assert lib.pq1_set_test_flags(0) == 1


def test_pack_rows_and_embed_validation(lib):
    w, s, pb, ps = A, 2 * A, 4 * A, 8 * A
    r = lib.pq1_pack_weights_rows
    assert r(None, P(s), 16, 1024, P(pb), P(ps), 32, 0, None) == 1
    assert r(P(w), P(s), 16, 1024, P(pb), P(ps), 32, 17, None) == 2     # row0 + N > N_total
    assert r(P(w), P(s), 16, 1024, P(pb), P(ps), 32, -1, None) == 2
    assert r(P(w), P(s), 16, 1024, P(pb + 4), P(ps), 32, 0, None) == 3
    assert r(P(w), P(s), 16, 1024, P(w), P(ps), 32, 0, None) == 5
    e = lib.pq1_embed
    tok, sg, out = 16 * A, 17 * A, 18 * A
    assert e(None, 1, P(w), P(s), P(sg), P(out), 16, 1024, None) == 1
    assert e(P(tok), 1, P(w), P(s), P(sg), P(out), 16, 1536, None) == 2   # K % 1024
    assert e(P(tok), 0, P(w), P(s), P(sg), P(out), 16, 1024, None) == 2   # M < 1
    assert e(P(tok + 2), 1, P(w), P(s), P(sg), P(out), 16, 1024, None) == 3
    assert e(P(tok), 1, P(w), P(s), P(sg), P(out + 4), 16, 1024, None) == 3
    assert e(P(tok), 1, P(w), P(s), P(sg), P(w), 16, 1024, None) == 5      # out over the table


def test_packed_sizes_and_validation(lib):
    assert lib.pq1_packed_bits_bytes(130, 640) == 3 * 5 * 64 * 16
    assert lib.pq1_packed_scales_bytes(130, 640) == 3 * 5 * 64 * 4
    assert lib.pq1_packed_bits_bytes(0, 640) == 0 and lib.pq1_packed_scales_bytes(5, 100) == 0
    p = lib.pq1_pack_weights
    w, s, pb, ps = A, 2 * A, 4 * A, 8 * A
    assert p(None, P(s), 16, 1024, P(pb), P(ps), None) == 1
    assert p(P(w), P(s), 16, 1000, P(pb), P(ps), None) == 2
    assert p(P(w), P(s), 16, 1024, P(pb + 4), P(ps), None) == 3
    assert p(P(w), P(s), 16, 1024, P(w), P(ps), None) == 5
    g = lib.pq1_gemv_packed
    assert g(None, P(pb), P(ps), P(A), 16, 1024, P(1 << 40), 1 << 30, None) == 1
    assert g(P(A), P(pb), P(ps), P(pb), 16, 1024, P(1 << 40), 1 << 30, None) == 5
    f = lib.pq1_rotate_gemv_packed
    assert f(P(A), None, None, P(pb), P(ps), P(16 * A), 16, 1024, P(1 << 40), 1 << 30, None) == 1
    assert f(P(A), P(2 * A), None, P(pb), P(ps), P(16 * A), 16, 1152, P(1 << 40), 1 << 30,
             None) == 2


def test_f16_scale_sizes_match_the_pages(lib):
    import json
    facts = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_facts.json")))
    vt, row = facts["vocab_table"], facts["row_bytes_f16_scales_5120"]
    V, K = vt["rows"], vt["width"]
    assert V % 64 == 0  # no band padding: the packed arrays hold exactly the table
    bits = lib.pq1_packed_bits_bytes(V, K)
    sc16 = lib.pq1_packed_scales_bytes_ex(V, K, 1)
    assert bits == V * row["bits_bytes"] and sc16 == V * row["scale_bytes"]
    assert bits + sc16 == vt["bytes_f16_scales"] == V * row["value"]
    # 1.125 bits per weight with f16 scales, 1.25 with fp32 ones
    assert 8 * (bits + sc16) / (V * K) == 1.125
    assert 8 * (bits + lib.pq1_packed_scales_bytes_ex(V, K, 0)) / (V * K) == 1.25
    assert lib.pq1_packed_scales_bytes_ex(130, 640, 1) == 3 * 5 * 64 * 2
    assert lib.pq1_packed_scales_bytes_ex(130, 640, 0) == lib.pq1_packed_scales_bytes(130, 640)
    assert lib.pq1_packed_scales_bytes_ex(130, 640, 2) == 0
    assert lib.pq1_packed_scales_bytes_ex(130, 640, -1) == 0
    assert lib.pq1_packed_scales_bytes_ex(0, 640, 1) == 0


def test_f16_scale_entry_points_validation(lib):
    w, s, pb, ps = A, 2 * A, 4 * A, 8 * A
    p = lib.pq1_pack_weights_ex
    assert p(None, P(s), 16, 1024, P(pb), P(ps), 1, 32, 0, None) == 1
    assert p(P(w), P(s), 16, 1024, P(pb), P(ps), 2, 32, 0, None) == 8       # scale dtype
    assert p(P(w), P(s), 16, 1024, P(pb), P(ps), -1, 32, 0, None) == 8
    assert p(P(w), P(s), 16, 1024, P(pb), P(ps), 1, 32, 17, None) == 2      # row0 + N > N_total
    assert p(P(w), P(s), 16, 1000, P(pb), P(ps), 1, 16, 0, None) == 2
    assert p(P(w), P(s), 16, 1024, P(pb), P(ps + 2), 1, 32, 0, None) == 3
    # f16 scales of 32 x 1024 take 64 x 8 x 2 bytes: ending 16 bytes into
    # packed_bits overlaps (the adjacent, valid placement is in the no-device test)
    nsc = lib.pq1_packed_scales_bytes_ex(32, 1024, 1)
    assert p(P(w), P(s), 16, 1024, P(pb), P(pb - nsc + 16), 1, 32, 0, None) == 5
    g = lib.pq1_gemv_packed_ex
    assert g(None, P(pb), P(ps), 1, P(A), 16, 1024, P(1 << 40), 1 << 30, None) == 1
    assert g(P(A), P(pb), P(ps), 3, P(16 * A), 16, 1024, P(1 << 40), 1 << 30, None) == 8
    assert g(P(A), P(pb), P(ps), 1, P(pb), 16, 1024, P(1 << 40), 1 << 30, None) == 5
    assert g(P(A), P(pb), P(ps + 2), 1, P(16 * A), 16, 1024, P(1 << 40), 1 << 30, None) == 3
    f = lib.pq1_rotate_gemv_packed_ex
    assert f(P(A), None, None, P(pb), P(ps), 1, P(16 * A), 16, 1024, P(1 << 40), 1 << 30,
             None) == 1
    assert f(P(A), P(2 * A), None, P(pb), P(ps), 1, P(16 * A), 16, 1152, P(1 << 40), 1 << 30,
             None) == 2
    assert f(P(A), P(2 * A), None, P(pb), P(ps), 9, P(16 * A), 16, 1024, P(1 << 40), 1 << 30,
             None) == 8


@pytest.mark.skipif(gpu_available(), reason="checks the no-device path")
def test_valid_call_without_device_reports_device_error(lib):
    # all arguments valid: the call reaches the device check and fails there
    assert lib.pq1_rotate(P(A), P(2 * A), None, P(3 * A), 0, 1, 1024, None) == 6
    assert lib.pq1_gemm(P(A), P(2 * A), P(4 * A), P(8 * A), 4, 16, 1024, None) == 6
    assert lib.pq1_gemm_ex(P(A), P(2 * A), P(4 * A), P(8 * A), 4, 16, 1024, 1, None) == 6
    assert lib.pq1_pack_weights_ex(P(A), P(2 * A), 16, 1024, P(4 * A), P(8 * A), 1, 16, 0,
                                   None) == 6
    # f16 scales placed right before packed_bits: adjacent, not overlapping
    nsc = lib.pq1_packed_scales_bytes_ex(32, 1024, 1)
    assert lib.pq1_pack_weights_ex(P(A), P(2 * A), 16, 1024, P(4 * A), P(4 * A - nsc), 1, 32, 0,
                                   None) == 6
