"""Property-based checks of the C ABI without a GPU: any combination of
pointers (null, misaligned, overlapping) and sizes (zero, negative, huge,
ragged) makes every entry point return one of its documented status codes --
and, with no device present, an argument set that passes validation stops at
the device check -- without crashing.  Skipped when a GPU is visible: there a
valid-looking set of made-up pointers would reach a kernel launch."""
import ctypes
import os

import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

from conftest import gpu_available

pytestmark = pytest.mark.skipif(gpu_available(), reason="needs a host without a visible GPU")

CODES = {1, 2, 3, 4, 5, 6, 8}
BASE = 1 << 36          # made-up device addresses, far apart unless chosen equal
P = ctypes.c_void_p
SETTINGS = dict(max_examples=300, deadline=None, derandomize=True,
                suppress_health_check=[HealthCheck.function_scoped_fixture])


@pytest.fixture(scope="module")
def lib():
    from gemm_hadamard_rotated_amd import build, pq1
    if not os.path.exists(pq1.LIB_PATH):
        build.build()
    return pq1.load_library()


ptr = st.one_of(st.just(None),
                st.builds(lambda k, off: BASE * k + off, st.integers(1, 8),
                          st.sampled_from([0, 0, 0, 2, 4, 8, 256])))
size = st.one_of(st.sampled_from([-1, 0, 1, 31, 32, 127, 128, 1000, 1024, 1152, 5120, 17408,
                                  (1 << 28), (1 << 31) - 1, 1 << 31, 1 << 40]),
                 st.integers(-5, 5000))


def _p(v):
    return P(v) if v is not None else None


@settings(**SETTINGS)
@given(x=ptr, s=ptr, out=ptr, M=size, K=size, dtype=st.integers(-1, 3))
def test_rotate_any_arguments(lib, x, s, out, M, K, dtype):
    assert lib.pq1_rotate(_p(x), _p(s), None, _p(out), dtype, M, K, None) in CODES


@settings(**SETTINGS)
@given(x=ptr, w=ptr, s=ptr, y=ptr, ws=ptr, N=size, K=size, algo=st.integers(-1, 4),
       wsb=st.sampled_from([0, 1024, 1 << 18, 1 << 30]))
def test_gemv_any_arguments(lib, x, w, s, y, ws, N, K, algo, wsb):
    assert lib.pq1_gemv_ex(_p(x), _p(w), _p(s), _p(y), N, K, algo, _p(ws), wsb, None) in CODES
    assert lib.pq1_gemv_packed(_p(x), _p(w), _p(s), _p(y), N, K, _p(ws), wsb, None) in CODES
    for sd in (-1, 0, 1, 2):
        assert lib.pq1_gemv_packed_ex(_p(x), _p(w), _p(s), sd, _p(y), N, K, _p(ws), wsb,
                                      None) in CODES


@settings(**SETTINGS)
@given(x=ptr, w=ptr, s=ptr, y=ptr, M=size, N=size, K=size, layout=st.integers(-1, 2))
def test_gemm_any_arguments(lib, x, w, s, y, M, N, K, layout):
    assert lib.pq1_gemm(_p(x), _p(w), _p(s), _p(y), M, N, K, None) in CODES
    assert lib.pq1_gemm_ex(_p(x), _p(w), _p(s), _p(y), M, N, K, layout, None) in CODES


@settings(**SETTINGS)
@given(w=ptr, s=ptr, pb=ptr, ps=ptr, N=size, K=size, total=size, row0=size)
def test_pack_rows_any_arguments(lib, w, s, pb, ps, N, K, total, row0):
    assert lib.pq1_pack_weights_rows(_p(w), _p(s), N, K, _p(pb), _p(ps), total, row0, None) in CODES
    for sd in (-1, 0, 1, 2):
        assert lib.pq1_pack_weights_ex(_p(w), _p(s), N, K, _p(pb), _p(ps), sd, total, row0,
                                       None) in CODES


@settings(**SETTINGS)
@given(tok=ptr, w=ptr, s=ptr, sg=ptr, out=ptr, M=size, V=size, K=size)
def test_embed_any_arguments(lib, tok, w, s, sg, out, M, V, K):
    assert lib.pq1_embed(_p(tok), M, _p(w), _p(s), _p(sg), _p(out), V, K, None) in CODES
