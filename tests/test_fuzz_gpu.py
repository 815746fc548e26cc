"""Property-based parity on the GPU: hypothesis draws shapes (ragged N, K from
128 up, permutations, both X layouts, stacked matrices, out-of-range token
ids) and every entry point is compared with the fp64 oracle under the same
bars as the fixed-shape tests.  Derandomized, so a failure reproduces."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle.pq1_oracle as orc
from gemm_hadamard_rotated_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-5
SETTINGS = dict(deadline=None, derandomize=True, print_blob=True,
                suppress_health_check=[HealthCheck.function_scoped_fixture,
                                       HealthCheck.too_slow])


@pytest.fixture(scope="module")
def pq(dev):
    from gemm_hadamard_rotated_amd import pq1
    pq1.load_library()
    return pq1


def f32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def words(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(dev)


def bf16(bits_u16, dev):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(dev).view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def check(got, ref, A, tol, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    worst = float(np.max(np.abs(got - ref) / np.maximum(A, 1e-300))) if got.size else 0.0
    assert worst <= tol, f"{what}: max |err|/A = {worst:.3e}"


def gemm_order_index(K):
    # stored position 8c + 2q + t of every 32-wide block holds offset 4c + q + 16t
    p = np.arange(K)
    pl = p % 32
    c, e = pl // 8, pl % 8
    return (p - pl) + 4 * c + e // 2 + 16 * (e % 2)


PERMS = {2048: [(64, 8, 4), (128, 4, 4), (32, 16, 4)], 3072: [(128, 8, 3), (64, 16, 3)],
         6144: [(128, 16, 3), (256, 8, 3)]}


@settings(max_examples=30, **SETTINGS)
@given(K=st.sampled_from([1024, 2048, 3072, 5120, 6144]), M=st.integers(1, 5),
       use_perm=st.booleans(), seed=st.integers(0, 2**31 - 1), data=st.data())
def test_fuzz_rotate(pq, dev, K, M, use_perm, seed, data):
    perm = data.draw(st.sampled_from(PERMS[K])) if use_perm and K in PERMS else None
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    s = wl.draw_signs(rng, K)
    got = host(pq.pq1_rotate(f32(x, dev), f32(s, dev), perm=perm))
    check(got, orc.rotate(x, s, perm), orc.rotate_normalizer(x, s, perm), TOL_F32,
          f"rotate M={M} K={K} perm={perm}")


@settings(max_examples=40, **SETTINGS)
@given(N=st.integers(1, 2500), kg=st.integers(1, 48), algo=st.sampled_from([1, 2]),
       seed=st.integers(0, 2**31 - 1))
def test_fuzz_gemv_canonical(pq, dev, N, kg, algo, seed):
    K = 128 * kg
    rng = np.random.default_rng(seed)
    bits, scales = wl.draw_bits(rng, N, K), wl.draw_scales(rng, N, K)
    xr = rng.standard_normal(K).astype(np.float32)
    y = host(pq.pq1_gemv_ex(f32(xr, dev), words(bits, dev), f32(scales, dev), algo=algo))
    check(y, orc.gemv(xr, bits, scales), orc.normalizer(xr, bits, scales), TOL_F32,
          f"gemv N={N} K={K} algo={algo}")


@settings(max_examples=40, **SETTINGS)
@given(N=st.integers(1, 3000), kb=st.integers(1, 6), fused=st.booleans(),
       scale_dtype=st.sampled_from(["f32", "f16"]), seed=st.integers(0, 2**31 - 1))
def test_fuzz_gemv_packed(pq, dev, N, kb, fused, scale_dtype, seed):
    K = 1024 * kb
    rng = np.random.default_rng(seed)
    bits, scales = wl.draw_bits(rng, N, K), wl.draw_scales(rng, N, K)
    x = rng.standard_normal(K).astype(np.float32)
    s = wl.draw_signs(rng, K)
    pw = pq.pq1_pack_weights(words(bits, dev), f32(scales, dev), scale_dtype=scale_dtype)
    if scale_dtype == "f16":  # the GEMV then uses the scales rounded to f16
        scales = orc.scales_as_f16(scales)
    xr = orc.rotate(x, s)
    if fused:
        y = host(pq.pq1_rotate_gemv_packed(f32(x, dev), f32(s, dev), pw))
    else:
        y = host(pq.pq1_gemv_packed(f32(xr.astype(np.float32), dev), pw))
        xr = xr.astype(np.float32)
    check(y, orc.gemv(xr, bits, scales), orc.normalizer(xr, bits, scales), TOL_F32,
          f"packed N={N} K={K} fused={fused} scales={scale_dtype}")


@settings(max_examples=40, **SETTINGS)
@given(M=st.integers(1, 200), N=st.integers(1, 700), kg=st.integers(1, 16),
       gemm_order=st.booleans(), seed=st.integers(0, 2**31 - 1))
def test_fuzz_gemm(pq, dev, M, N, kg, gemm_order, seed):
    K = 128 * kg
    rng = np.random.default_rng(seed)
    xb = wl.random_bf16_bits(rng, M, K)
    bits, scales = wl.draw_bits(rng, N, K), wl.draw_scales(rng, N, K)
    xin = np.ascontiguousarray(xb[:, gemm_order_index(K)]) if gemm_order else xb
    Y = host(pq.pq1_gemm(bf16(xin, dev), words(bits, dev), f32(scales, dev), gemm_order=gemm_order))
    X = orc.bf16_bits_to_float(xb)
    check(Y, orc.gemm(X, bits, scales), orc.normalizer(X, bits, scales), TOL_F32,
          f"gemm M={M} N={N} K={K} gemm_order={gemm_order}")


@settings(max_examples=16, **SETTINGS)
@given(M=st.integers(1, 64), N=st.integers(8193, 20000), kg=st.integers(1, 10),
       gemm_order=st.booleans(), seed=st.integers(0, 2**31 - 1))
def test_fuzz_gemm_short_prompt_wide(pq, dev, M, N, kg, gemm_order, seed):
    """Short prompts against wide weight matrices, where the plans put four or
    five column blocks in a workgroup (ragged last workgroup and block)."""
    K = 128 * kg
    rng = np.random.default_rng(seed)
    xb = wl.random_bf16_bits(rng, M, K)
    bits, scales = wl.draw_bits(rng, N, K), wl.draw_scales(rng, N, K)
    xin = np.ascontiguousarray(xb[:, gemm_order_index(K)]) if gemm_order else xb
    Y = host(pq.pq1_gemm(bf16(xin, dev), words(bits, dev), f32(scales, dev), gemm_order=gemm_order))
    X = orc.bf16_bits_to_float(xb)
    check(Y, orc.gemm(X, bits, scales), orc.normalizer(X, bits, scales), TOL_F32,
          f"short-prompt gemm M={M} N={N} K={K} gemm_order={gemm_order}")


@settings(max_examples=25, **SETTINGS)
@given(V=st.integers(1, 3000), kb=st.integers(1, 3), M=st.integers(1, 9),
       seed=st.integers(0, 2**31 - 1))
def test_fuzz_embed(pq, dev, V, kb, M, seed):
    K = 1024 * kb
    rng = np.random.default_rng(seed)
    bits, scales = wl.draw_bits(rng, V, K), wl.draw_scales(rng, V, K)
    s = wl.draw_signs(rng, K)
    toks = rng.integers(-3, V + 3, size=M).astype(np.int32)
    out = host(pq.pq1_embed(torch.from_numpy(toks).to(dev), words(bits, dev), f32(scales, dev),
                            f32(s, dev)))
    ok = (toks >= 0) & (toks < V)
    assert np.all(np.isnan(out[~ok]))
    if ok.any():
        z = orc.embedding_rows(bits, scales, K, toks[ok])
        check(out[ok], orc.inverse_rotate(z, s), orc.rotate_normalizer(z, np.ones(K)), TOL_F32,
              f"embed V={V} K={K}")


@settings(max_examples=25, **SETTINGS)
@given(ns=st.lists(st.integers(1, 400), min_size=1, max_size=4), kb=st.integers(1, 3),
       seed=st.integers(0, 2**31 - 1))
def test_fuzz_stacked_pack(pq, dev, ns, kb, seed):
    K = 1024 * kb
    rng = np.random.default_rng(seed)
    parts = [(wl.draw_bits(rng, n, K), wl.draw_scales(rng, n, K)) for n in ns]
    pw = pq.pq1_pack_weights_rows([(words(b, dev), f32(sc, dev)) for b, sc in parts])
    whole = pq.pq1_pack_weights(words(np.concatenate([b for b, _ in parts]), dev),
                                f32(np.concatenate([sc for _, sc in parts]), dev))
    assert torch.equal(pw.bits, whole.bits) and torch.equal(pw.scales, whole.scales)
