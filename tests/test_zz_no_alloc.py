"""The no-allocation decode step (pq1_rotate_gemv_packed_noalloc, called
through the C ABI) against the workspace version it varies: two calls in a
row on the library's own counter region, the second with a smaller input,
each within the fp32 bar of the workspace call's result on the same inputs
(both are also held to the oracle)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle.pq1_oracle as orc
from gemm_hadamard_rotated_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-5


@pytest.fixture(scope="module")
def pq(dev):
    from gemm_hadamard_rotated_amd import pq1
    pq1.load_library()
    return pq1


def _noalloc(pq, x, s, pw, perm, y, dev):
    lib = pq.load_library()
    with torch.cuda.device(dev):
        rc = lib.pq1_rotate_gemv_packed_noalloc(
            ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(s.data_ptr()), pq._perm(perm),
            ctypes.c_void_p(pw.bits.data_ptr()), ctypes.c_void_p(pw.scales.data_ptr()),
            pq.SCALE_DTYPES[pw.scale_dtype], ctypes.c_void_p(y.data_ptr()), pw.N, pw.K,
            ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert rc == 0, pq.pq1_status_str(rc)


@pytest.mark.parametrize("order", [("ffn_gate", "ssm_out"), ("ffn_down", "tiny")])
def test_noalloc_matches_workspace_call(pq, dev, order):
    for name in order:                      # the second input is the smaller one
        d = wl.make(name)
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
        bits = torch.from_numpy(d["bits"].view(np.int32)).to(dev)
        pw = pq.pq1_pack_weights(bits, f32(d["scales"]))
        x, s = f32(d["x"][0]), f32(d["signs"])
        y_ws = pq.pq1_rotate_gemv_packed(x, s, pw, perm=d["perm"])
        y_na = torch.full((d["N"],), float("nan"), dtype=torch.float32, device=dev)
        _noalloc(pq, x, s, pw, d["perm"], y_na, dev)
        torch.cuda.synchronize()
        xr = orc.rotate(d["x"][0], d["signs"], d["perm"])
        A = orc.normalizer(xr, d["bits"], d["scales"])
        ref = orc.gemv(xr, d["bits"], d["scales"])
        a, b = y_na.cpu().numpy().astype(np.float64), y_ws.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(a)), f"{name}: non-finite outputs"
        assert np.max(np.abs(a - b) / A) <= TOL_F32, f"{name}: no-alloc vs workspace call"
        assert np.max(np.abs(a - ref) / A) <= TOL_F32, f"{name}: no-alloc vs oracle"


def test_noalloc_f16_scales_and_binding(pq, dev):
    d = wl.make("ffn_gate")
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    bits = torch.from_numpy(d["bits"].view(np.int32)).to(dev)
    pw = pq.pq1_pack_weights(bits, f32(d["scales"]), scale_dtype="f16")
    x, s = f32(d["x"][0]), f32(d["signs"])
    y_ws = pq.pq1_rotate_gemv_packed(x, s, pw).cpu().numpy().astype(np.float64)
    y_na = pq.pq1_rotate_gemv_packed_noalloc(x, s, pw).cpu().numpy().astype(np.float64)
    s16 = orc.scales_as_f16(d["scales"])
    xr = orc.rotate(d["x"][0], d["signs"])
    A = orc.normalizer(xr, d["bits"], s16)
    assert np.max(np.abs(y_na - y_ws) / A) <= TOL_F32
    assert np.max(np.abs(y_na - orc.gemv(xr, d["bits"], s16)) / A) <= TOL_F32
