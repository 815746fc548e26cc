"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: every check uses a library
routine, a different construction, a closed form, a value printed on the
pages (tests/golden), or pure-Python brute force on tiny inputs.  The
mutation tests at the end plant plausible mistakes in the oracle and show
that at least one pin catches each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle.pq1_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


FACTS = _load("pages_facts.json")
RNG = np.random.default_rng(20261202)


# ----------------------------------------------------------------------------
# Pin functions (also used by the mutation tests)
# ----------------------------------------------------------------------------
def pin_constants():
    assert orc.WHT_BLOCK == FACTS["wht_block"]["value"]
    assert orc.WHT_SCALE == FACTS["wht_scale"]["value"]
    assert orc.GROUP == FACTS["group"]["value"]
    w = FACTS["sign_widths"]
    assert sum(w["value"]) == w["total"]
    for width in w["value"]:
        assert width % orc.WHT_BLOCK == 0 and width % orc.GROUP == 0


def pin_hadamard_library():
    # scipy.linalg.hadamard builds the natural-order Sylvester matrix.
    for n in (2, 8, 64, 1024):
        assert np.array_equal(orc.sylvester_hadamard(n), scipy.linalg.hadamard(n).astype(float))


def pin_hadamard_recursion():
    # H_{2n} = [[H_n, H_n], [H_n, -H_n]], built with Kronecker products.
    H = np.array([[1.0]])
    base = np.array([[1.0, 1.0], [1.0, -1.0]])
    for _ in range(10):
        H = np.kron(base, H)
    assert np.array_equal(orc.sylvester_hadamard(1024), H)


def pin_rotate_against_scipy():
    # rotate() with a block-diagonal dense matrix from scipy's Hadamard.
    K = 2048
    x = RNG.standard_normal(K)
    s = RNG.choice([-1.0, 1.0], size=K)
    Hs = scipy.linalg.hadamard(1024).astype(float) / 32.0
    ref = np.concatenate([Hs @ (s[:1024] * x[:1024]), Hs @ (s[1024:] * x[1024:])])
    got = orc.rotate(x, s)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(orc.rotate_normalizer(x, s))


def pin_rotate_closed_forms():
    ones = np.ones(1024)
    e0 = np.zeros(1024)
    e0[0] = 1.0
    # H e0 = (1/32) * 1 ; H 1 = 32 e0 (normalized transform).
    assert np.allclose(orc.rotate(e0, ones), ones / 32.0, atol=0, rtol=0)
    assert np.allclose(orc.rotate(ones, ones), 32.0 * e0, atol=1e-12, rtol=0)
    # A sign flip on one input flips that input's contribution only.
    s = ones.copy()
    s[0] = -1.0
    assert np.allclose(orc.rotate(e0, s), -ones / 32.0, atol=0, rtol=0)


def pin_rotate_orthogonal():
    # The rotation (permutation, signs, normalized Hadamard) preserves norms
    # and the normalized Hadamard is an involution.
    x = RNG.standard_normal(6144)
    s = RNG.choice([-1.0, 1.0], size=6144)
    y = orc.rotate(x, s, perm=(128, 16, 3))
    assert abs(np.linalg.norm(y) - np.linalg.norm(x)) <= 1e-12 * np.linalg.norm(x)
    ones = np.ones(1024)
    z = RNG.standard_normal(1024)
    assert np.max(np.abs(orc.rotate(orc.rotate(z, ones), ones) - z)) < 1e-12


def pin_rotate_block_diagonal():
    K = 5120
    x = RNG.standard_normal(K)
    s = RNG.choice([-1.0, 1.0], size=K)
    base = orc.rotate(x, s)
    for b in range(5):
        x2 = x.copy()
        x2[b * 1024 + 17] += 3.0
        d = np.abs(orc.rotate(x2, s) - base).reshape(5, 1024).max(axis=1)
        assert d[b] > 0.05
        assert all(d[j] == 0.0 for j in range(5) if j != b)


def pin_fwht_matches_dense():
    v = RNG.standard_normal((3, 1024))
    dense = v @ scipy.linalg.hadamard(1024).astype(float)
    assert np.max(np.abs(orc.fwht_fp64(v) - dense)) < 1e-10


def pin_permutation_semantics():
    p = FACTS["ssm_out_perm"]
    hd, nk, rep = p["hd"], p["nk"], p["rep"]
    assert hd * nk * rep == p["width"]
    src = orc.head_source_index(hd, nk, rep)
    # a bijection that moves whole heads
    assert np.array_equal(np.sort(src), np.arange(hd * nk * rep))
    heads = src.reshape(nk * rep, hd)
    assert np.all(heads % hd == np.arange(hd))
    src_head = heads[:, 0] // hd
    for dst_head, sh in enumerate(src_head):
        # tiled layout: key head is h % nk (interleaved); grouped layout:
        # key head is h // rep (blocked).  The permutation keeps each value
        # under the key head it belongs to.
        assert sh % nk == dst_head // rep
    # within a key group, repeats keep ascending order
    for n in range(nk):
        grp = src_head[n * rep:(n + 1) * rep]
        assert list(grp) == sorted(grp)
    # rep == 1 means no permutation
    x = RNG.standard_normal(6144)
    s = np.ones(6144)
    assert np.array_equal(orc.rotate(x, s, perm=(128, 48, 1)), orc.rotate(x, s))


def pin_bit_order_golden():
    g = _load("bit_order.json")
    for case in g["cases"]:
        words = np.array([case["words"]], dtype=np.uint32)
        K = 32 * len(case["words"])
        want = -np.ones(K, dtype=np.int8)
        want[case["plus_positions"]] = 1
        assert np.array_equal(orc.weight_signs(words, K)[0], want)


def pin_bit_order_unpackbits():
    words = RNG.integers(0, 2 ** 32, size=(7, 8), dtype=np.uint32)
    # On a little-endian host the bytes of each word come LSB byte first, and
    # unpackbits(bitorder="little") emits each byte LSB first.
    le = words.astype("<u4").view(np.uint8).reshape(7, 32)
    bits = np.unpackbits(le, axis=1, bitorder="little")
    assert np.array_equal(orc.weight_signs(words, 256), bits.astype(np.int8) * 2 - 1)


def pin_scale_groups_one_hot():
    # Row pattern: weight k is +1 exactly when k % 3 == 0.  Scales differ per
    # group.  A one-hot x' at k must return scale[k // 128] * (+-1).
    K = 512
    words = np.zeros((1, K // 32), dtype=np.uint32)
    for k in range(0, K, 3):
        words[0, k // 32] |= np.uint32(1 << (k % 32))
    scales = np.array([[0.5, 0.25, 0.125, 2.0]], dtype=np.float32)
    for k in range(K):
        e = np.zeros(K)
        e[k] = 1.0
        y = orc.gemv(e, words, scales)[0]
        want = [0.5, 0.25, 0.125, 2.0][k // 128] * (1.0 if k % 3 == 0 else -1.0)
        assert y == want


def pin_group_norm():
    # Every group of 128 dequantized weights has length sqrt(128) * scale.
    fac = FACTS["group_norm_factor"]["value"]
    words = RNG.integers(0, 2 ** 32, size=(5, 40), dtype=np.uint32)
    scales = RNG.uniform(0.005, 0.05, size=(5, 10)).astype(np.float32)
    W = orc.dequantize(words, scales, 1280).reshape(5, 10, 128)
    norms = np.linalg.norm(W, axis=2)
    assert np.allclose(norms / scales.astype(np.float64), math.sqrt(128))
    assert abs(math.sqrt(128) - fac) < 5e-4
    # and a 5120-wide row holds at most 2 * 40 distinct values
    w5120 = RNG.integers(0, 2 ** 32, size=(1, 160), dtype=np.uint32)
    s5120 = RNG.uniform(0.005, 0.05, size=(1, 40)).astype(np.float32)
    vals = np.unique(orc.dequantize(w5120, s5120, 5120))
    assert len(vals) <= FACTS["distinct_values_per_5120_row"]["value"]


def pin_all_ones_and_zeros():
    K, N = 1024, 6
    x = RNG.standard_normal(K)
    scales = RNG.uniform(0.005, 0.05, size=(N, K // 128)).astype(np.float32)
    T = x.reshape(-1, 128).sum(axis=1)
    ones = np.full((N, K // 32), 0xFFFFFFFF, dtype=np.uint32)
    zeros = np.zeros((N, K // 32), dtype=np.uint32)
    want = scales.astype(np.float64) @ T
    assert np.allclose(orc.gemv(x, ones, scales), want, rtol=0, atol=1e-12)
    assert np.allclose(orc.gemv(x, zeros, scales), -want, rtol=0, atol=1e-12)
    # normalizer: with all-ones bits and |x| the product is the normalizer
    assert np.allclose(orc.normalizer(x, ones, scales), orc.gemv(np.abs(x), ones, scales))


def _popcount_parity(v):
    return bin(v).count("1") & 1


def pin_pipeline_bruteforce():
    # Pure-Python loops: y[n] = sum_k scale[n][k>>7] * (+-1) * x'[k], with
    # x'[i] = (1/32) sum_j (-1)^popcount(i&j) * s[j] * x[j]; K = 1024, N = 2.
    K, N = 1024, 2
    rng = np.random.default_rng(7)
    x = rng.standard_normal(K)
    s = rng.choice([-1.0, 1.0], size=K)
    words = rng.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint32)
    scales = rng.uniform(0.005, 0.05, size=(N, K // 128)).astype(np.float32)
    xs = [float(s[j]) * float(x[j]) for j in range(K)]
    xr = []
    for i in range(K):
        acc = 0.0
        for j in range(K):
            acc += -xs[j] if _popcount_parity(i & j) else xs[j]
        xr.append(acc / 32.0)
    got_r = orc.rotate(x, s)
    assert max(abs(got_r[i] - xr[i]) for i in range(K)) < 1e-11
    y = []
    for n in range(N):
        acc = 0.0
        for k in range(K):
            bit = (int(words[n, k >> 5]) >> (k & 31)) & 1
            acc += float(scales[n, k >> 7]) * (1.0 if bit else -1.0) * xr[k]
        y.append(acc)
    got = orc.gemv(orc.rotate(x, s), words, scales)
    A = orc.normalizer(orc.rotate(x, s), words, scales)
    assert all(abs(got[n] - y[n]) <= 1e-12 * A[n] for n in range(N))


def pin_folded_form():
    # Wq . WHT(s * P x)  ==  (Wq . H_blk . D . P) . x with dense matrices:
    # fixes the order permutation -> signs -> transform.
    for K, perm in ((1024, None), (2048, None), (6144, (128, 16, 3))):
        N = 16 if K < 6144 else 64
        rng = np.random.default_rng(K)
        x = rng.standard_normal(K)
        s = rng.choice([-1.0, 1.0], size=K)
        words = rng.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint32)
        scales = rng.uniform(0.005, 0.05, size=(N, K // 128)).astype(np.float32)
        Wq = orc.dequantize(words, scales, K)
        Hblk = np.kron(np.eye(K // 1024), scipy.linalg.hadamard(1024).astype(float) / 32.0)
        D = np.diag(s)
        P = np.eye(K)
        if perm is not None:
            hd, nk, rep = perm
            P = np.zeros((K, K))
            for n in range(nk):
                for r in range(rep):
                    for d in range(hd):
                        P[hd * (r + rep * n) + d, hd * (n + nk * r) + d] = 1.0
        folded = Wq @ Hblk @ D @ P
        want = folded @ x
        got = orc.gemv(orc.rotate(x, s, perm=perm), words, scales)
        A = np.abs(folded) @ np.abs(x)
        assert np.max(np.abs(got - want) / A) < 1e-12


def pin_embedding_inverse():
    # The embedding-side order (transform, then signs) undoes the forward
    # rotation; the forward order applied twice does not.
    K = 2048
    x = RNG.standard_normal(K)
    s = RNG.choice([-1.0, 1.0], size=K)
    z = orc.rotate(x, s)
    assert np.max(np.abs(orc.inverse_rotate(z, s) - x)) < 1e-12
    assert np.max(np.abs(orc.rotate(z, s) - x)) > 0.1


def pin_bf16_rounding():
    import torch
    v = np.concatenate([RNG.standard_normal(4096) * 10.0 ** RNG.integers(-6, 6, 4096),
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0, -0.0,
                         1.0 + 2.0 ** -8 + 2.0 ** -20]])
    f32 = v.astype(np.float32)
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.round_to_bf16(v), ref)
    # ties go to even: 1 + 2^-8 -> 1.0, 1 + 3*2^-8 -> 1 + 2^-6
    assert orc.bf16_bits_to_float(orc.round_to_bf16(np.array([1.0 + 2.0 ** -8])))[0] == 1.0
    assert orc.bf16_bits_to_float(orc.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8])))[0] == 1.0 + 2.0 ** -6


def pin_gemm_rows_are_gemv():
    K, N, M = 1024, 8, 3
    X = RNG.standard_normal((M, K))
    words = RNG.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint32)
    scales = RNG.uniform(0.005, 0.05, size=(N, K // 128)).astype(np.float32)
    Y = orc.gemm(X, words, scales)
    for m in range(M):
        assert np.allclose(Y[m], orc.gemv(X[m], words, scales), rtol=0, atol=1e-12)
    ms, ns = np.array([0, 2, 1]), np.array([7, 0, 3])
    assert np.allclose(orc.gemm_entries(X, words, scales, ms, ns), Y[ms, ns], rtol=0, atol=1e-12)


def _dense_perm(K, perm):
    """The head permutation as a dense 0/1 matrix, written out from the
    reading (grouped head r + rep*n takes tiled head n + nk*r)."""
    P = np.eye(K)
    if perm is not None:
        hd, nk, rep = perm
        P = np.zeros((K, K))
        for n in range(nk):
            for r in range(rep):
                for d in range(hd):
                    P[hd * (r + rep * n) + d, hd * (n + nk * r) + d] = 1.0
    return P


def pin_rotate_normalizer_bruteforce():
    # A'[i] is the sum of the absolute values of the terms of output i of the
    # rotation, from the dense block-diagonal scipy Hadamard (Pulse
    # ARCHITECTURE-SPEC method notes: errors are scaled by sum |terms|).
    for K, perm in ((2048, None), (6144, (128, 16, 3))):
        rng = np.random.default_rng(K + 11)
        x = rng.standard_normal(K)
        x[rng.choice(K, 4, replace=False)] *= 20.0  # outlier channels
        s = rng.choice([-1.0, 1.0], size=K)
        Hblk = np.kron(np.eye(K // 1024), scipy.linalg.hadamard(1024).astype(float) / 32.0)
        v = s * (_dense_perm(K, perm) @ x)          # the transform's inputs
        want = np.abs(Hblk) @ np.abs(v)             # sum_j |H_ij v_j| per output i
        got = orc.rotate_normalizer(x, s, perm)
        assert got.shape == (K,)
        assert np.max(np.abs(got - want)) <= 1e-12 * np.max(want)
        # and a few outputs by pure-Python loops over the terms
        for i in (0, 1023, 1024, K - 1, 3 * K // 5):
            b = i // 1024
            acc = 0.0
            for j in range(1024 * b, 1024 * (b + 1)):
                acc += abs(((-1.0) ** _popcount_parity(i % 1024 & j % 1024)) / 32.0 * v[j])
            assert abs(got[i] - acc) <= 1e-12 * acc
    # rows of a matrix input are independent
    X = RNG.standard_normal((3, 2048))
    s = RNG.choice([-1.0, 1.0], size=2048)
    A = orc.rotate_normalizer(X, s)
    for m in range(3):
        assert np.array_equal(A[m], orc.rotate_normalizer(X[m], s))


def _brute_normalizer_row(x, words, scales, n):
    """sum_k |scale[n][k>>7] * (+-1) * x[k]| by a loop over k."""
    acc = 0.0
    for k in range(len(x)):
        bit = (int(words[n, k >> 5]) >> (k & 31)) & 1
        acc += abs(float(scales[n, k >> 7]) * (1.0 if bit else -1.0) * float(x[k]))
    return acc


def _brute_gemv_row(x, words, scales, n):
    acc = 0.0
    for k in range(len(x)):
        bit = (int(words[n, k >> 5]) >> (k & 31)) & 1
        acc += float(scales[n, k >> 7]) * (1.0 if bit else -1.0) * float(x[k])
    return acc


def pin_normalizer_bruteforce():
    # A[n] = sum_k |W[n][k] x'[k]| by loops, for a vector and a matrix input.
    K, N = 384, 5
    rng = np.random.default_rng(31)
    x = rng.standard_normal(K)
    words = rng.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint32)
    scales = rng.uniform(0.005, 0.05, size=(N, K // 128)).astype(np.float32)
    A = orc.normalizer(x, words, scales)
    for n in range(N):
        want = _brute_normalizer_row(x, words, scales, n)
        assert abs(A[n] - want) <= 1e-12 * want
    X = rng.standard_normal((2, K))
    A2 = orc.normalizer(X, words, scales)
    assert A2.shape == (2, N)
    for m in range(2):
        for n in range(N):
            assert abs(A2[m, n] - _brute_normalizer_row(X[m], words, scales, n)) <= 1e-12 * A2[m, n]


def pin_row_and_entry_subsets():
    # The row / entry forms the full-size parity tests use, against loops over
    # the chosen rows and entries (rows unsorted, repeated, and at the ends).
    K, N, M = 256, 9, 4
    rng = np.random.default_rng(32)
    x = rng.standard_normal(K)
    X = rng.standard_normal((M, K))
    words = rng.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint32)
    scales = rng.uniform(0.005, 0.05, size=(N, K // 128)).astype(np.float32)
    rows = np.array([8, 0, 3, 3, 5])
    g = orc.gemv_rows(x, words, scales, rows)
    a = orc.normalizer_rows(x, words, scales, rows)
    for i, n in enumerate(rows):
        assert abs(g[i] - _brute_gemv_row(x, words, scales, n)) <= 1e-12 * a[i]
        assert abs(a[i] - _brute_normalizer_row(x, words, scales, n)) <= 1e-12 * a[i]
    ms, ns = np.array([3, 0, 2, 3, 1]), np.array([8, 8, 0, 4, 5])
    ge = orc.gemm_entries(X, words, scales, ms, ns)
    ae = orc.normalizer_entries(X, words, scales, ms, ns)
    for i, (m, n) in enumerate(zip(ms, ns)):
        want_a = _brute_normalizer_row(X[m], words, scales, n)
        assert abs(ae[i] - want_a) <= 1e-12 * want_a
        assert abs(ge[i] - _brute_gemv_row(X[m], words, scales, n)) <= 1e-12 * want_a
    # embedding rows: entry k of table row r is +-scale[r][k>>7], by loops
    emb = orc.embedding_rows(words, scales, K, rows)
    assert emb.shape == (len(rows), K)
    for i, r in enumerate(rows):
        for k in range(0, K, 7):
            bit = (int(words[r, k >> 5]) >> (k & 31)) & 1
            assert emb[i, k] == float(scales[r, k >> 7]) * (1.0 if bit else -1.0)


def _f16_value_from_fields(bits):
    """binary16 value from its fields, written out: sign, 5-bit exponent with
    bias 15, 10-bit fraction; exponent 0 is subnormal (fraction * 2^-24)."""
    bits = np.asarray(bits, dtype=np.int64)
    sign = np.where(bits >> 15, -1.0, 1.0)
    e, m = (bits >> 10) & 31, bits & 1023
    normal = sign * (1.0 + m / 1024.0) * np.exp2(e - 15.0)
    return np.where(e == 0, sign * m * 2.0 ** -24, normal)


def pin_f16_rounding_bruteforce():
    # every finite non-negative binary16 value, in increasing order (patterns
    # 0x0000 .. 0x7BFF); the nearest one by search, ties to the even pattern,
    # beyond the midpoint above 65504 infinity
    grid_bits = np.arange(0x7C00, dtype=np.int64)
    grid = _f16_value_from_fields(grid_bits)
    assert np.all(np.diff(grid) > 0) and grid[-1] == 65504.0
    mags = np.concatenate([
        np.exp2(RNG.uniform(-27, 16.2, 6000)),
        (grid[1:] + grid[:-1]) / 2,                     # exact ties
        RNG.choice(grid, 500),                          # exact values
        [0.0, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 65519.99, 65520.0, 1e6]])
    v = np.concatenate([mags, -mags]).astype(np.float32).astype(np.float64)
    a = np.abs(v)
    hi = np.clip(np.searchsorted(grid, a), 1, len(grid) - 1)
    lo = hi - 1
    dl, dh = a - grid[lo], grid[hi] - a
    pick = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a <= grid[0], 0, pick)
    expect = pick.astype(np.uint32)
    # above 65504 the next step would be 65536: below the midpoint 65520 the
    # value rounds down to 65504, from it on (the tie goes to the even,
    # infinite pattern) it overflows
    expect = np.where(a >= 65520.0, 0x7C00, np.where(a > 65504.0, 0x7BFF, expect))
    expect = (expect | np.where(np.signbit(v), 0x8000, 0)).astype(np.uint16)
    got = orc.round_to_f16(v)
    assert np.array_equal(got, expect), np.flatnonzero(got != expect)[:5]
    # the decode is exact
    assert np.array_equal(orc.f16_bits_to_float(grid_bits.astype(np.uint16)), grid)


def pin_f16_pages_facts():
    sub = FACTS["f16_smallest_subnormal"]
    b = orc.round_to_f16(np.array([2.0 ** -24]))
    assert int(b[0]) == sub["bits"]
    assert f"{orc.f16_bits_to_float(b)[0]:.2e}" == f"{sub['value']:.2e}"
    # half of the smallest subnormal is a tie and goes to (even) zero
    assert int(orc.round_to_f16(np.array([2.0 ** -25]))[0]) == 0
    # bf16 keeps 7 explicit mantissa bits and f16 keeps 10, so an f16 holding a
    # bf16 value (in f16's exponent range) has 3 trailing zero mantissa bits
    # ("Inside the One-Bit Engine", station "The one-bit quantizer never
    # quantized anything")
    fp = FACTS["f16_from_bf16_fingerprint"]
    assert fp["f16_mantissa_bits"] - fp["bf16_mantissa_bits"] == fp["zero_low_mantissa_bits"]
    bf = orc.bf16_bits_to_float(orc.round_to_bf16(np.exp2(RNG.uniform(-14, 15.9, 4000))))
    b16 = orc.round_to_f16(bf)
    assert np.array_equal(orc.f16_bits_to_float(b16), bf)  # exact: no rounding happened
    assert np.all((b16 & 7) == 0)
    assert orc.scales_as_f16(np.array([0.1]))[0] != 0.1  # 0.1 is not an f16
    assert abs(orc.scales_as_f16(np.array([0.1]))[0] - 0.1) <= 2.0 ** -14 / 2


PINS = [pin_constants, pin_hadamard_library, pin_hadamard_recursion, pin_rotate_against_scipy,
        pin_rotate_closed_forms, pin_rotate_orthogonal, pin_rotate_block_diagonal,
        pin_fwht_matches_dense, pin_permutation_semantics, pin_bit_order_golden,
        pin_bit_order_unpackbits, pin_scale_groups_one_hot, pin_group_norm,
        pin_all_ones_and_zeros, pin_pipeline_bruteforce, pin_folded_form,
        pin_embedding_inverse, pin_bf16_rounding, pin_gemm_rows_are_gemv,
        pin_f16_rounding_bruteforce, pin_f16_pages_facts, pin_rotate_normalizer_bruteforce,
        pin_normalizer_bruteforce, pin_row_and_entry_subsets]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# Mutation tests: a planted mistake in the oracle must fail at least one pin.
# ----------------------------------------------------------------------------
def _fails_some_pin():
    for p in PINS:
        try:
            p()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


def _msb_first_signs(w_bits, K):
    words = np.asarray(w_bits, dtype=np.uint32)
    k = np.arange(K)
    bits = (words[:, k >> 5] >> (31 - (k & 31)).astype(np.uint32)) & np.uint32(1)
    return (bits.astype(np.int8) * 2 - 1).astype(np.int8)


def _inverted_convention(w_bits, K):
    words = np.asarray(w_bits, dtype=np.uint32)
    k = np.arange(K)
    bits = (words[:, k >> 5] >> (k & 31).astype(np.uint32)) & np.uint32(1)
    return (1 - bits.astype(np.int8) * 2).astype(np.int8)


def _sequency_hadamard(n=1024):
    H = scipy.linalg.hadamard(n).astype(float)
    changes = (np.diff(H, axis=1) != 0).sum(axis=1)
    return H[np.argsort(changes)]


def _inverse_perm(hd, nk, rep):
    src = np.empty(hd * nk * rep, dtype=np.int64)
    for n in range(nk):
        for r in range(rep):
            src[(n + nk * r) * hd:(n + nk * r + 1) * hd] = np.arange((r + rep * n) * hd,
                                                                     (r + rep * n + 1) * hd)
    return src


def _signs_after_transform(x, signs, perm=None):
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    p = orc._check_perm(perm)
    xp = orc.permute_tiled_to_grouped(x, *p) if p else x
    blocks = xp.reshape(xp.shape[:-1] + (K // 1024, 1024))
    out = (blocks @ orc.sylvester_hadamard(1024)) * orc.WHT_SCALE
    return out.reshape(x.shape) * np.asarray(signs, dtype=np.float64)


def _scale_index_by_word(w_bits, scales, K):
    s = np.asarray(scales, dtype=np.float64)
    pm = orc.weight_signs(w_bits, K).astype(np.float64)
    k = np.arange(K)
    return pm * s[:, np.minimum(k >> 5, s.shape[1] - 1)]


def _f16_truncating(v):
    a = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        b = a.astype(np.float16).view(np.uint16).copy()
    back = b.view(np.float16).astype(np.float64)
    over = np.abs(back) > np.abs(a)  # rounded away from zero: step back one
    b[over] -= 1
    return b


def _f16_decoded_as_bf16(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


MUTANTS = {
    "f16 rounding truncates": ("round_to_f16", _f16_truncating),
    "f16 bits decoded as bf16": ("f16_bits_to_float", _f16_decoded_as_bf16),
    "bit order MSB-first": ("weight_signs", _msb_first_signs),
    "bit 1 means -1": ("weight_signs", _inverted_convention),
    "sequency-ordered Walsh": ("sylvester_hadamard", _sequency_hadamard),
    "inverse permutation": ("head_source_index", _inverse_perm),
    "signs after transform": ("rotate", _signs_after_transform),
    "scale indexed by word": ("dequantize", _scale_index_by_word),
}


# Mistakes in the functions that set the parity bars (the normalizers) and in
# the row / entry forms the full-size parity tests use.
def _rotate_normalizer_per_row(x, signs, perm=None):
    x = np.asarray(x, dtype=np.float64)
    p = orc._check_perm(perm)
    xp = orc.permute_tiled_to_grouped(x, *p) if p else x
    a = np.abs(xp * np.asarray(signs, dtype=np.float64))
    return np.broadcast_to(a.sum(axis=-1, keepdims=True) * orc.WHT_SCALE, a.shape).copy()


def _rotate_normalizer_no_scale(x, signs, perm=None):
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    p = orc._check_perm(perm)
    xp = orc.permute_tiled_to_grouped(x, *p) if p else x
    a = np.abs(xp * np.asarray(signs, dtype=np.float64))
    blocks = a.reshape(a.shape[:-1] + (K // 1024, 1024))
    return np.broadcast_to(blocks.sum(axis=-1, keepdims=True), blocks.shape).reshape(x.shape).copy()


def _normalizer_signed_x(x_rot, w_bits, scales):
    X = np.asarray(x_rot, dtype=np.float64)
    return np.abs(X @ np.abs(orc.dequantize(w_bits, scales, X.shape[-1])).T)


def _gemv_rows_first(x_rot, w_bits, scales, rows):
    n = len(rows)
    return orc.gemv(x_rot, np.asarray(w_bits)[:n], np.asarray(scales)[:n])


def _normalizer_rows_sorted(x_rot, w_bits, scales, rows):
    rows = np.sort(np.asarray(rows, dtype=np.int64))
    return orc.normalizer(x_rot, np.asarray(w_bits)[rows], np.asarray(scales)[rows])


def _normalizer_entries_transposed(x_rot, w_bits, scales, ms, ns):
    X = np.asarray(x_rot, dtype=np.float64)
    W = orc.dequantize(np.asarray(w_bits)[ns], np.asarray(scales)[ns], X.shape[-1])
    return np.einsum("ik,ik->i", np.abs(X[np.asarray(ms)[::-1]]), np.abs(W))


def _embedding_rows_unscaled(w_bits, scales, K, rows):
    rows = np.asarray(rows, dtype=np.int64)
    return orc.weight_signs(np.asarray(w_bits)[rows], K).astype(np.float64)


MUTANTS.update({
    "rotate normalizer summed over the whole row": ("rotate_normalizer", _rotate_normalizer_per_row),
    "rotate normalizer without 1/32": ("rotate_normalizer", _rotate_normalizer_no_scale),
    "normalizer with signed x": ("normalizer", _normalizer_signed_x),
    "gemv_rows takes the first rows": ("gemv_rows", _gemv_rows_first),
    "normalizer_rows sorts the rows": ("normalizer_rows", _normalizer_rows_sorted),
    "normalizer_entries pairs the wrong rows": ("normalizer_entries", _normalizer_entries_transposed),
    "embedding_rows without scales": ("embedding_rows", _embedding_rows_unscaled),
})


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    assert _fails_some_pin(), f"no pin catches the mutant: {name}"


def test_mutant_dropped_normalization(monkeypatch):
    real = orc.rotate

    def unnormalized(x, signs, perm=None):
        return real(x, signs, perm) * 32.0

    monkeypatch.setattr(orc, "rotate", unnormalized)
    assert _fails_some_pin()


def test_mutant_dropped_scale(monkeypatch):
    def no_scale(w_bits, scales, K):
        return orc.weight_signs(w_bits, K).astype(np.float64)

    monkeypatch.setattr(orc, "dequantize", no_scale)
    assert _fails_some_pin()
