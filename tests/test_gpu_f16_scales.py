"""GPU parity of the f16-scale packed weight format against the fp64 oracle.

The format stores each 128-weight group's scale as an IEEE binary16 value
("Inside the One-Bit Engine": 640 bytes of sign bits and 80 bytes of f16
scales per 5120-wide row).  The repack rounds the fp32 scales to f16 (nearest,
ties to even); the oracle rounds the same fp32 values with its own routine.
Bars:
* the packed f16 scales: bit-identical to the oracle's rounding (an integer
  decision taken from the same fp32 input on both sides);
* GEMV results: the oracle's fp64 GEMV on the rounded scales, within
  2e-5 * A (A = sum_k |s_f16 w_k x_k|), as for fp32 scales;
* inputs on which every operation is exact (small integers, power-of-two
  scales, which f16 holds exactly): bit-exact, and equal to the fp32-scale
  path's result.
"""
import numpy as np
import pytest
import torch

import oracle.pq1_oracle as orc
from gemm_hadamard_rotated_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-5
DECODE = ["tiny", "ffn_gate", "ffn_down", "ssm_out"]


@pytest.fixture(scope="module")
def pq(dev):
    from gemm_hadamard_rotated_amd import pq1
    pq1.load_library()
    return pq1


def dev_f32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def dev_bits(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(dev)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def f16_bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_normalized(got, ref, A, tol, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: {np.sum(~np.isfinite(got))} non-finite outputs"
    ratio = np.abs(got - ref) / np.maximum(A, 1e-300)
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= tol, f"{what}: max |err|/A = {worst:.3e} > {tol:.0e}"


def packed_scale_rows(ps, N, K):
    """[row][group] view of a packed scale array ([band][group][lane])."""
    G = K // 128
    sc = ps.reshape(-1, G, 64)
    rows = np.arange(sc.shape[0] * 64)
    return sc[rows // 64, :, rows % 64], rows


SPECIAL = np.array([2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11),
                    65504.0, 65519.0, 65520.0, 1e6, 1e-9, 0.1, -0.3, 1.0 + 2.0 ** -11,
                    1.0 + 3 * 2.0 ** -11, 0.0, -0.0, 0.0125, 0.049], dtype=np.float32)


def test_pack_f16_rounding_and_layout(pq, dev):
    """Every packed scale is the oracle's f16 rounding of the source scale,
    bit for bit (ties, subnormals, overflow to infinity, signed zeros
    included); padding rows hold zeros; the bits are the fp32 layout's."""
    N, K = 130, 640
    rng = np.random.default_rng(160)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.draw_scales(rng, N, K)
    flat = scales.reshape(-1)
    flat[:SPECIAL.size] = SPECIAL
    flat[-SPECIAL.size:] = -SPECIAL
    pw = pq.pq1_pack_weights(dev_bits(bits, dev), dev_f32(scales, dev), scale_dtype="f16")
    assert pw.scale_dtype == "f16" and pw.scales.dtype == torch.float16
    assert pw.scales.numel() * 2 == pq.load_library().pq1_packed_scales_bytes_ex(N, K, 1)
    got, rows = packed_scale_rows(f16_bits(pw.scales), N, K)
    assert np.array_equal(got[rows < N], orc.round_to_f16(scales))
    assert not got[rows >= N].any()
    ref = pq.pq1_pack_weights(dev_bits(bits, dev), dev_f32(scales, dev))
    assert torch.equal(pw.bits, ref.bits)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", DECODE)
def test_f16_packed_matches_oracle(pq, dev, name, fused):
    d = wl.make(name)
    s16 = orc.scales_as_f16(d["scales"])
    pw = pq.pq1_pack_weights(dev_bits(d["bits"], dev), dev_f32(d["scales"], dev), scale_dtype="f16")
    xr = orc.rotate(d["x"][0], d["signs"], d["perm"])
    if fused:
        y = host(pq.pq1_rotate_gemv_packed(dev_f32(d["x"][0], dev), dev_f32(d["signs"], dev), pw,
                                           perm=d["perm"]))
    else:
        xr = xr.astype(np.float32)
        y = host(pq.pq1_gemv_packed(dev_f32(xr, dev), pw))
    assert_normalized(y, orc.gemv(xr, d["bits"], s16), orc.normalizer(xr, d["bits"], s16),
                      TOL_F32, f"f16 scales {name} fused={fused}")


@pytest.mark.parametrize("N,K", [(1000, 640), (77, 1152), (300, 17408), (1, 128), (4099, 3072),
                                 (65, 2048)])
def test_f16_exact_inputs_match_fp32_path(pq, dev, N, K):
    rng = np.random.default_rng(N * 11 + K)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.power_of_two_scales(rng, N, K)       # held exactly by f16
    assert np.array_equal(orc.scales_as_f16(scales), scales.astype(np.float64))
    xr = wl.integer_activation(rng, 1, K)[0]
    b, sc = dev_bits(bits, dev), dev_f32(scales, dev)
    p16, p32 = pq.pq1_pack_weights(b, sc, scale_dtype="f16"), pq.pq1_pack_weights(b, sc)
    y16 = host(pq.pq1_gemv_packed_ex(dev_f32(xr, dev), p16))
    assert np.array_equal(y16.astype(np.float64), orc.gemv(xr, bits, scales))
    assert np.array_equal(y16, host(pq.pq1_gemv_packed(dev_f32(xr, dev), p32)))
    if K % 1024 == 0:
        s = wl.draw_signs(rng, K)
        x = wl.integer_activation(rng, 1, K)[0]
        yf = host(pq.pq1_rotate_gemv_packed_ex(dev_f32(x, dev), dev_f32(s, dev), p16))
        assert np.array_equal(yf.astype(np.float64), orc.gemv(orc.rotate(x, s), bits, scales))


def test_f16_stacked_rows_and_gate_up(pq, dev):
    """ffn_gate + ffn_up packed one after the other with f16 scales: the same
    arrays as packing the concatenation, and one launch gives both outputs."""
    d = wl.make("gate_up")
    n = d["N"] // 2
    halves = [(dev_bits(d["bits"][:n], dev), dev_f32(d["scales"][:n], dev)),
              (dev_bits(d["bits"][n:], dev), dev_f32(d["scales"][n:], dev))]
    pw = pq.pq1_pack_weights_rows(halves, scale_dtype="f16")
    whole = pq.pq1_pack_weights(dev_bits(d["bits"], dev), dev_f32(d["scales"], dev),
                                scale_dtype="f16")
    assert torch.equal(pw.bits, whole.bits) and torch.equal(pw.scales, whole.scales)
    y = host(pq.pq1_rotate_gemv_packed(dev_f32(d["x"][0], dev), dev_f32(d["signs"], dev), pw))
    xr = orc.rotate(d["x"][0], d["signs"])
    s16 = orc.scales_as_f16(d["scales"])
    assert_normalized(y, orc.gemv(xr, d["bits"], s16), orc.normalizer(xr, d["bits"], s16),
                      TOL_F32, "gate + up, f16 scales")


def test_f16_pack_rows_leave_other_rows_alone(pq, dev):
    rng = np.random.default_rng(43)
    K, n1, n2 = 1024, 1000, 777
    b_bits, b_sc = wl.draw_bits(rng, n2, K), wl.draw_scales(rng, n2, K)
    lib = pq.load_library()
    nb, ns = lib.pq1_packed_bits_bytes(n1 + n2, K), lib.pq1_packed_scales_bytes_ex(n1 + n2, K, 1)
    pbits = torch.full((nb // 4,), 0x5A5A5A5A, dtype=torch.int32, device=dev)
    pscales = torch.full((ns // 2,), 7.0, dtype=torch.float16, device=dev)
    bb, bs = dev_bits(b_bits, dev), dev_f32(b_sc, dev)
    with torch.cuda.device(dev):
        rc = lib.pq1_pack_weights_ex(pq._ptr(bb), pq._ptr(bs), n2, K, pq._ptr(pbits),
                                     pq._ptr(pscales), 1, n1 + n2, n1, pq._stream(dev))
    assert rc == 0
    s_rows, rows = packed_scale_rows(f16_bits(pscales), n1 + n2, K)
    seven = np.float16(7.0).view(np.uint16)
    first, second, pad = rows < n1, (rows >= n1) & (rows < n1 + n2), rows >= n1 + n2
    assert np.all(s_rows[first] == seven)
    assert np.array_equal(s_rows[second], orc.round_to_f16(b_sc))
    assert np.all(s_rows[pad] == 0)


def test_f16_lm_head_sampled_and_graph_replay(pq, dev):
    """The output head with f16 scales at full size, eager and replayed from a
    graph, checked on sampled rows; a call of another shape in between."""
    d = wl.make("lm_head")
    N = d["N"]
    pw = pq.pq1_pack_weights(dev_bits(d["bits"], dev), dev_f32(d["scales"], dev), scale_dtype="f16")
    x, s = dev_f32(d["x"][0], dev), dev_f32(d["signs"], dev)
    rows = np.unique(np.concatenate([np.random.default_rng(8).integers(0, N, 2000),
                                     [0, 1, 63, 64, N - 65, N - 64, N - 1]]))
    xr = orc.rotate(d["x"][0], d["signs"])
    s16 = orc.scales_as_f16(d["scales"][rows])
    ref = orc.gemv(xr, d["bits"][rows], s16)
    A = orc.normalizer(xr, d["bits"][rows], s16)
    g8 = wl.make("ffn_gate")
    pg = pq.pq1_pack_weights(dev_bits(g8["bits"], dev), dev_f32(g8["scales"], dev), scale_dtype="f16")
    xg, sg = dev_f32(g8["x"][0], dev), dev_f32(g8["signs"], dev)
    xrg, sg16 = orc.rotate(g8["x"][0], g8["signs"]), orc.scales_as_f16(g8["scales"])
    refg, Ag = orc.gemv(xrg, g8["bits"], sg16), orc.normalizer(xrg, g8["bits"], sg16)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    out = torch.empty(N, dtype=torch.float32, device=dev)
    with torch.cuda.stream(side):
        pq.pq1_rotate_gemv_packed(x, s, pw, out=out)
    torch.cuda.synchronize()
    assert_normalized(host(out)[rows], ref, A, TOL_F32, "lm_head f16 eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        pq.pq1_rotate_gemv_packed(x, s, pw, out=out)
    for r in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        assert_normalized(host(out)[rows], ref, A, TOL_F32, f"lm_head f16 replay {r}")
        with torch.cuda.stream(side):
            yg = pq.pq1_rotate_gemv_packed(xg, sg, pg)
        assert_normalized(host(yg), refg, Ag, TOL_F32, f"ffn_gate f16 between replays {r}")


def test_f16_errors_on_device(pq, dev):
    """A scale dtype the library does not know is rejected before any launch."""
    lib = pq.load_library()
    d = wl.make("tiny")
    b, sc = dev_bits(d["bits"], dev), dev_f32(d["scales"], dev)
    pw = pq.pq1_pack_weights(b, sc, scale_dtype="f16")
    xr = dev_f32(np.zeros(d["K"], np.float32), dev)
    y = torch.empty(d["N"], dtype=torch.float32, device=dev)
    ws = pq.gemv_workspace(d["N"], d["K"], dev)
    with torch.cuda.device(dev):
        assert lib.pq1_gemv_packed_ex(pq._ptr(xr), pq._ptr(pw.bits), pq._ptr(pw.scales), 7,
                                      pq._ptr(y), d["N"], d["K"], pq._ptr(ws), ws.numel(),
                                      pq._stream(dev)) == 8
    with pytest.raises(pq.Pq1Error):
        pq.pq1_pack_weights(b, sc, scale_dtype="bf16")
