"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars (written here, from the method's arithmetic):
* fp32 results (rotate, gemv, fused rotate+gemv):
  max |y - y_ref| <= 2e-5 * A per output, A = sum_k |w_k x_k| (for the
  rotation A = (1/32) * sum over the 1024-block of |x|).
* bf16-MFMA prefill GEMM end to end (x' rounded to bf16 inside the path):
  <= 1e-2 * A against the oracle on the unrounded x'.
* The GEMM alone on bf16 inputs: products with +-1 are exact, so only the fp32
  accumulation rounds: <= 2e-5 * A.
* Inputs on which every operation is exact (small integers, power-of-two
  scales, one-hot vectors, all-ones / all-zeros bits): bit-exact.
* The bf16 output of the rotation equals the oracle's round-to-nearest-even
  of x' wherever x' is farther than the fp32 tolerance from a rounding tie.
"""
import numpy as np
import pytest
import torch

import oracle.pq1_oracle as orc
from gemm_hadamard_rotated_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-5
TOL_BF16 = 1e-2
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


def dev_bf16(bits_u16, dev):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(dev).view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def bf16_host_bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_normalized(got, ref, A, tol, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: {np.sum(~np.isfinite(got))} non-finite outputs"
    err = np.abs(got - ref)
    ratio = err / np.maximum(A, 1e-300)
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= tol, f"{what}: max |err|/A = {worst:.3e} > {tol:.0e}"
    return worst


def assert_rows_chunked(y, xr, bits, scales, tol, what, exact=False, chunk=8192):
    """Compare every output row of a GEMV (y [N]) or GEMM (y [M][N]) with the
    oracle, a block of weight rows at a time (the dense fp64 weights of a full
    output head would not fit in memory at once)."""
    y = np.asarray(y)
    N = bits.shape[0]
    worst = 0.0
    for n0 in range(0, N, chunk):
        b, sc = bits[n0:n0 + chunk], scales[n0:n0 + chunk]
        got = y[..., n0:n0 + chunk].astype(np.float64)
        ref = orc.gemm(xr, b, sc) if np.ndim(xr) == 2 else orc.gemv(xr, b, sc)
        if exact:
            bad = np.argwhere(got != ref)
            assert bad.size == 0, (f"{what}: {len(bad)} entries of rows {n0}.. differ, first at "
                                   f"{tuple(bad[0])}: {got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}")
            continue
        A = orc.normalizer(xr, b, sc)
        worst = max(worst, assert_normalized(got, ref, A, tol, f"{what} rows {n0}.."))
    return worst


# ----------------------------------------------------------------------------
# rotation
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name", DECODE + ["prefill"])
def test_rotate_fp32_matches_oracle(pq, dev, name):
    d = wl.make(name)
    x = d["x"] if name != "prefill" else d["x"][:64]
    xr = host(pq.pq1_rotate(dev_f32(x, dev), dev_f32(d["signs"], dev), perm=d["perm"]))
    ref = orc.rotate(x, d["signs"], d["perm"])
    A = orc.rotate_normalizer(x, d["signs"], d["perm"])
    assert_normalized(xr, ref, A, TOL_F32, f"rotate {name}")


def test_rotate_full_prefill_block(pq, dev):
    d = wl.make("prefill")
    xr = host(pq.pq1_rotate(dev_f32(d["x"], dev), dev_f32(d["signs"], dev)))
    ref = orc.rotate(d["x"], d["signs"])
    A = orc.rotate_normalizer(d["x"], d["signs"])
    assert_normalized(xr, ref, A, TOL_F32, "rotate prefill 1024x5120")


@pytest.mark.parametrize("K,perm", [(1024, None), (5120, None), (17408, None),
                                    (6144, (128, 16, 3)), (2048, (64, 8, 4))])
def test_rotate_integer_inputs_bit_exact(pq, dev, K, perm):
    rng = np.random.default_rng(K + 7)
    x = wl.integer_activation(rng, 3, K)
    s = wl.draw_signs(rng, K)
    got = host(pq.pq1_rotate(dev_f32(x, dev), dev_f32(s, dev), perm=perm))
    ref = orc.rotate(x, s, perm)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("M,K,perm", [(67, 2048, None), (66, 6144, (128, 16, 3)), (64, 1024, None),
                                      (63, 1024, None)])
def test_rotate_many_rows_bit_exact(pq, dev, M, K, perm):
    """Many rows, with and without the head permutation: on integer
    activations every output is exact, in fp32, in bf16 and in bf16 in the
    GEMM K order."""
    rng = np.random.default_rng(M * 13 + K)
    x = wl.integer_activation(rng, M, K)
    s = wl.draw_signs(rng, K)
    ref = orc.rotate(x, s, perm)
    got = host(pq.pq1_rotate(dev_f32(x, dev), dev_f32(s, dev), perm=perm))
    assert np.array_equal(got.astype(np.float64), ref)
    want = orc.bf16_bits_to_float(orc.round_to_bf16(ref))
    xb = bf16_host_bits(pq.pq1_rotate(dev_f32(x, dev), dev_f32(s, dev), perm=perm,
                                      out_dtype=torch.bfloat16))
    assert np.array_equal(orc.bf16_bits_to_float(xb), want)
    xg = bf16_host_bits(pq.pq1_rotate(dev_f32(x, dev), dev_f32(s, dev), perm=perm,
                                      out_dtype=torch.bfloat16, gemm_order=True))
    assert np.array_equal(orc.bf16_bits_to_float(xg), want[:, gemm_order_index(K)])


def test_rotate_one_hot_columns(pq, dev):
    # x = e_j (no signs): x' column j of H / 32, for every j of one block
    K = 1024
    X = np.eye(K, dtype=np.float32)
    got = host(pq.pq1_rotate(dev_f32(X, dev), dev_f32(np.ones(K), dev)))
    H = orc.sylvester_hadamard(K) / 32.0
    assert np.array_equal(got.astype(np.float64), H)


def test_rotate_bf16_output(pq, dev):
    d = wl.make("prefill")
    x = d["x"][:128]
    xb = bf16_host_bits(pq.pq1_rotate(dev_f32(x, dev), dev_f32(d["signs"], dev),
                                      out_dtype=torch.bfloat16))
    ref = orc.rotate(x, d["signs"])
    A = orc.rotate_normalizer(x, d["signs"])
    want = orc.round_to_bf16(ref)
    differ = xb != want
    # allowed only where the fp64 value is within the fp32 bar of a tie
    if differ.any():
        v = ref[differ]
        lo = orc.bf16_bits_to_float(np.minimum(xb[differ], want[differ]))
        hi = orc.bf16_bits_to_float(np.maximum(xb[differ], want[differ]))
        tie = (lo + hi) / 2
        near = np.abs(np.abs(v) - np.abs(tie)) <= TOL_F32 * A[differ]
        assert near.all(), f"{(~near).sum()} bf16 outputs differ away from a tie"
    # and the bf16 values are within half a bf16 ulp + fp32 bar of x'
    got = orc.bf16_bits_to_float(xb)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + TOL_F32 * A)


def test_rotate_sparse_integer_bf16_exact(pq, dev):
    rng = np.random.default_rng(3)
    x = wl.sparse_integer_activation(rng, 8, 5120)
    s = wl.draw_signs(rng, 5120)
    xb = bf16_host_bits(pq.pq1_rotate(dev_f32(x, dev), dev_f32(s, dev), out_dtype=torch.bfloat16))
    # compare values: a zero may come out as -0 (a zero input times a -1 sign)
    got = orc.bf16_bits_to_float(xb)
    want = orc.bf16_bits_to_float(orc.round_to_bf16(orc.rotate(x, s)))
    assert np.array_equal(got, want)


# ----------------------------------------------------------------------------
# GEMV
# ----------------------------------------------------------------------------
ALGOS = [1, 2]  # PQ1_GEMV_LUT, PQ1_GEMV_EXPAND


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("name", DECODE)
def test_gemv_matches_oracle(pq, dev, name, algo):
    d = wl.make(name)
    xr = orc.rotate(d["x"][0], d["signs"], d["perm"]).astype(np.float32)
    y = host(pq.pq1_gemv_ex(dev_f32(xr, dev), dev_bits(d["bits"], dev), dev_f32(d["scales"], dev),
                            algo=algo))
    ref = orc.gemv(xr, d["bits"], d["scales"])
    A = orc.normalizer(xr, d["bits"], d["scales"])
    w = assert_normalized(y, ref, A, TOL_F32, f"gemv {name} algo {algo}")
    print(f"  gemv {name} algo={algo}: max err/A = {w:.2e}", flush=True)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("N,K", [(1000, 640), (77, 1152), (300, 17408), (1, 128), (4099, 3072),
                                 (513, 384)])
def test_gemv_ragged_shapes(pq, dev, N, K, algo):
    d = wl.make_shape(N, K, seed=N * 31 + K)
    xr = d["x"][0]
    y = host(pq.pq1_gemv_ex(dev_f32(xr, dev), dev_bits(d["bits"], dev), dev_f32(d["scales"], dev),
                            algo=algo))
    ref = orc.gemv(xr, d["bits"], d["scales"])
    A = orc.normalizer(xr, d["bits"], d["scales"])
    assert_normalized(y, ref, A, TOL_F32, f"gemv {N}x{K} algo {algo}")


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("N,K", [(256, 1024), (17408, 5120), (5120, 17408), (5120, 6144),
                                 (1000, 640)])
def test_gemv_integer_inputs_bit_exact(pq, dev, N, K, algo):
    rng = np.random.default_rng(N + K)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.power_of_two_scales(rng, N, K)
    xr = wl.integer_activation(rng, 1, K)[0]
    y = host(pq.pq1_gemv_ex(dev_f32(xr, dev), dev_bits(bits, dev), dev_f32(scales, dev), algo=algo))
    assert np.array_equal(y.astype(np.float64), orc.gemv(xr, bits, scales))


@pytest.mark.parametrize("algo", ALGOS)
def test_gemv_one_hot_sweep(pq, dev, algo):
    # x' = e_k for every k of a 1024-wide row: y[n] = scale[n][k>>7] * (+-1)
    d = wl.make("tiny")
    bits = dev_bits(d["bits"], dev)
    sc = dev_f32(d["scales"], dev)
    W = orc.dequantize(d["bits"], d["scales"], 1024)
    e = torch.zeros(1024, dtype=torch.float32, device=dev)
    ys = []
    for k in range(1024):
        e.zero_()
        e[k] = 1.0
        ys.append(pq.pq1_gemv_ex(e, bits, sc, algo=algo).clone())
    Y = host(torch.stack(ys, 1))
    assert np.array_equal(Y.astype(np.float64), W)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("fill", [0xFFFFFFFF, 0])
def test_gemv_all_ones_all_zeros(pq, dev, algo, fill):
    N, K = 1000, 5120
    rng = np.random.default_rng(11)
    bits = np.full((N, K // 32), fill, dtype=np.uint32)
    scales = wl.draw_scales(rng, N, K)
    xr = rng.standard_normal(K).astype(np.float32)
    y = host(pq.pq1_gemv_ex(dev_f32(xr, dev), dev_bits(bits, dev), dev_f32(scales, dev), algo=algo))
    T = xr.astype(np.float64).reshape(-1, 128).sum(axis=1)
    ref = (1.0 if fill else -1.0) * (scales.astype(np.float64) @ T)
    A = orc.normalizer(xr, bits, scales)
    assert_normalized(y, ref, A, TOL_F32, "all-ones/zeros")


def test_gemv_deterministic_and_workspace_reuse(pq, dev):
    # shapes with different K-tilings alternate on one workspace; every result
    # must match the oracle and repeat bit for bit
    runs = []
    for name in ("ffn_down", "ssm_out", "tiny", "ffn_gate"):
        d = wl.make(name)
        xr = orc.rotate(d["x"][0], d["signs"], d["perm"]).astype(np.float32)
        args = (dev_f32(xr, dev), dev_bits(d["bits"], dev), dev_f32(d["scales"], dev))
        ref = orc.gemv(xr, d["bits"], d["scales"])
        A = orc.normalizer(xr, d["bits"], d["scales"])
        runs.append((name, args, ref, A))
    first = {}
    for rep in range(2):
        for name, args, ref, A in runs:
            for algo in ALGOS:
                y = pq.pq1_gemv_ex(*args, algo=algo).clone()
                assert_normalized(host(y), ref, A, TOL_F32, f"reuse {name} algo {algo}")
                if rep == 0:
                    first[(name, algo)] = y
                else:
                    assert torch.equal(first[(name, algo)], y)


def test_gemv_on_side_stream(pq, dev):
    d = wl.make("ffn_gate")
    xr = orc.rotate(d["x"][0], d["signs"]).astype(np.float32)
    args = (dev_f32(xr, dev), dev_bits(d["bits"], dev), dev_f32(d["scales"], dev))
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        y = pq.pq1_gemv(*args)
    torch.cuda.current_stream(dev).wait_stream(s)
    ref = orc.gemv(xr, d["bits"], d["scales"])
    A = orc.normalizer(xr, d["bits"], d["scales"])
    assert_normalized(host(y), ref, A, TOL_F32, "side stream")


# ----------------------------------------------------------------------------
# rotation -> GEMV, separate and fused
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name", DECODE)
def test_rotate_then_gemv_end_to_end(pq, dev, name):
    d = wl.make(name)
    xd = dev_f32(d["x"][0], dev)
    sd = dev_f32(d["signs"], dev)
    y = pq.pq1_gemv(pq.pq1_rotate(xd, sd, perm=d["perm"]), dev_bits(d["bits"], dev),
                    dev_f32(d["scales"], dev))
    xr_ref = orc.rotate(d["x"][0], d["signs"], d["perm"])
    ref = orc.gemv(xr_ref, d["bits"], d["scales"])
    A = orc.normalizer(xr_ref, d["bits"], d["scales"])
    assert_normalized(host(y), ref, A, TOL_F32, f"rotate->gemv {name}")


@pytest.mark.parametrize("name", DECODE)
def test_fused_rotate_gemv(pq, dev, name):
    d = wl.make(name)
    y = pq.pq1_rotate_gemv(dev_f32(d["x"][0], dev), dev_f32(d["signs"], dev),
                           dev_bits(d["bits"], dev), dev_f32(d["scales"], dev), perm=d["perm"])
    xr_ref = orc.rotate(d["x"][0], d["signs"], d["perm"])
    ref = orc.gemv(xr_ref, d["bits"], d["scales"])
    A = orc.normalizer(xr_ref, d["bits"], d["scales"])
    assert_normalized(host(y), ref, A, TOL_F32, f"fused {name}")


@pytest.mark.parametrize("N,K,perm", [(300, 2048, None), (1000, 6144, (128, 16, 3)),
                                      (5, 1024, None)])
def test_fused_integer_bit_exact(pq, dev, N, K, perm):
    rng = np.random.default_rng(N)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.power_of_two_scales(rng, N, K)
    x = wl.integer_activation(rng, 1, K)[0]
    s = wl.draw_signs(rng, K)
    y = host(pq.pq1_rotate_gemv(dev_f32(x, dev), dev_f32(s, dev), dev_bits(bits, dev),
                                dev_f32(scales, dev), perm=perm))
    assert np.array_equal(y.astype(np.float64), orc.gemv(orc.rotate(x, s, perm), bits, scales))


# ----------------------------------------------------------------------------
# packed (band-interleaved) weights
# ----------------------------------------------------------------------------
def packed_word(w):
    """A weight word as the packed layout stores it: rotated left by 2 bits
    (include/pq1.h, packed_bits)."""
    w = np.asarray(w, dtype=np.uint32)
    return ((w << np.uint32(2)) | (w >> np.uint32(30))).astype(np.uint32)


def test_pack_weights_layout(pq, dev):
    N, K = 130, 640
    d = wl.make_shape(N, K, seed=17)
    pw = pq.pq1_pack_weights(dev_bits(d["bits"], dev), dev_f32(d["scales"], dev))
    pb = host(pw.bits).view(np.uint32).reshape(-1, K // 128, 64, 4)
    ps = host(pw.scales).reshape(-1, K // 128, 64)
    nb = (N + 63) // 64
    assert pb.shape[0] == nb and ps.shape[0] == nb
    for b in range(nb):
        for l in range(64):
            n = 64 * b + l
            if n < N:
                assert np.array_equal(pb[b, :, l, :].reshape(-1), packed_word(d["bits"][n]))
                assert np.array_equal(ps[b, :, l], d["scales"][n])
            else:
                assert not pb[b, :, l, :].any() and not ps[b, :, l].any()


@pytest.mark.parametrize("name", DECODE)
def test_gemv_packed_matches_oracle(pq, dev, name):
    d = wl.make(name)
    xr = orc.rotate(d["x"][0], d["signs"], d["perm"]).astype(np.float32)
    pw = pq.pq1_pack_weights(dev_bits(d["bits"], dev), dev_f32(d["scales"], dev))
    y = host(pq.pq1_gemv_packed(dev_f32(xr, dev), pw))
    ref = orc.gemv(xr, d["bits"], d["scales"])
    A = orc.normalizer(xr, d["bits"], d["scales"])
    assert_normalized(y, ref, A, TOL_F32, f"packed gemv {name}")


@pytest.mark.parametrize("name", DECODE)
def test_fused_packed_matches_oracle(pq, dev, name):
    d = wl.make(name)
    pw = pq.pq1_pack_weights(dev_bits(d["bits"], dev), dev_f32(d["scales"], dev))
    y = host(pq.pq1_rotate_gemv_packed(dev_f32(d["x"][0], dev), dev_f32(d["signs"], dev), pw,
                                       perm=d["perm"]))
    xr_ref = orc.rotate(d["x"][0], d["signs"], d["perm"])
    ref = orc.gemv(xr_ref, d["bits"], d["scales"])
    A = orc.normalizer(xr_ref, d["bits"], d["scales"])
    assert_normalized(y, ref, A, TOL_F32, f"fused packed {name}")


@pytest.mark.parametrize("N,K", [(1000, 640), (77, 1152), (300, 17408), (1, 128), (4099, 3072),
                                 (513, 384), (65, 2048)])
def test_gemv_packed_ragged_and_exact(pq, dev, N, K):
    rng = np.random.default_rng(N * 7 + K)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.power_of_two_scales(rng, N, K)
    xr = wl.integer_activation(rng, 1, K)[0]
    pw = pq.pq1_pack_weights(dev_bits(bits, dev), dev_f32(scales, dev))
    y = host(pq.pq1_gemv_packed(dev_f32(xr, dev), pw))
    assert np.array_equal(y.astype(np.float64), orc.gemv(xr, bits, scales))
    if K % 1024 == 0:
        s = wl.draw_signs(rng, K)
        x = wl.integer_activation(rng, 1, K)[0]
        yf = host(pq.pq1_rotate_gemv_packed(dev_f32(x, dev), dev_f32(s, dev), pw))
        assert np.array_equal(yf.astype(np.float64), orc.gemv(orc.rotate(x, s), bits, scales))


@pytest.mark.parametrize("name", ["ffn_gate", "ffn_down", "ssm_out"])
def test_packed_graph_replay(pq, dev, name):
    """A graph holding ONE fused packed call, replayed several times with eager
    work in between, gives the eager result every time (the split-K bookkeeping
    depends on nothing the host passes per call); afterwards eager calls on the
    same workspace are still right and the canonical-layout counters are zero."""
    d = wl.make(name)
    pw = pq.pq1_pack_weights(dev_bits(d["bits"], dev), dev_f32(d["scales"], dev))
    x, s = dev_f32(d["x"][0], dev), dev_f32(d["signs"], dev)
    xr_ref = orc.rotate(d["x"][0], d["signs"], d["perm"])
    ref = orc.gemv(xr_ref, d["bits"], d["scales"])
    A = orc.normalizer(xr_ref, d["bits"], d["scales"])
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    out = torch.empty(d["N"], dtype=torch.float32, device=dev)
    with torch.cuda.stream(side):
        pq.pq1_rotate_gemv_packed(x, s, pw, perm=d["perm"], out=out)  # workspace for `side`
        ws = pq.gemv_workspace(d["N"], d["K"], dev)
    torch.cuda.synchronize()
    assert_normalized(host(out), ref, A, TOL_F32, f"{name} eager before capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        pq.pq1_rotate_gemv_packed(x, s, pw, perm=d["perm"], out=out)
    for r in range(5):
        out.fill_(float("nan"))  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        assert_normalized(host(out), ref, A, TOL_F32, f"{name} replay {r}")
    with torch.cuda.stream(side):
        for r in range(3):
            y = pq.pq1_rotate_gemv_packed(x, s, pw, perm=d["perm"])
            assert_normalized(host(y), ref, A, TOL_F32, f"{name} eager after replays {r}")
    counters = host(ws[:32768].view(torch.int32))
    assert not counters.any(), "canonical-layout arrival counters left non-zero"


def test_packed_calls_of_mixed_shapes_share_a_workspace(pq, dev):
    """Calls of different shapes (different split-K plans) interleaved on one
    stream and one workspace all stay right."""
    cases = []
    for name in ("ffn_gate", "ssm_out", "ffn_down"):
        d = wl.make(name)
        pw = pq.pq1_pack_weights(dev_bits(d["bits"], dev), dev_f32(d["scales"], dev))
        xr = orc.rotate(d["x"][0], d["signs"], d["perm"])
        cases.append((name, d, pw, dev_f32(xr.astype(np.float32), dev),
                      orc.gemv(xr.astype(np.float32), d["bits"], d["scales"]),
                      orc.normalizer(xr.astype(np.float32), d["bits"], d["scales"])))
    for it in range(3):
        for name, d, pw, xr, ref, A in (cases if it % 2 == 0 else cases[::-1]):
            y = host(pq.pq1_gemv_packed(xr, pw))
            assert_normalized(y, ref, A, TOL_F32, f"{name} call {it}")


# ----------------------------------------------------------------------------
# stacked matrices (ffn_gate + ffn_up), the output head, the embedding lookup
# ----------------------------------------------------------------------------
def test_pack_rows_equals_packing_the_concatenation(pq, dev):
    rng = np.random.default_rng(41)
    K = 1024
    a_bits, b_bits = wl.draw_bits(rng, 1000, K), wl.draw_bits(rng, 777, K)
    a_sc, b_sc = wl.draw_scales(rng, 1000, K), wl.draw_scales(rng, 777, K)
    stacked = pq.pq1_pack_weights_rows([(dev_bits(a_bits, dev), dev_f32(a_sc, dev)),
                                        (dev_bits(b_bits, dev), dev_f32(b_sc, dev))])
    whole = pq.pq1_pack_weights(dev_bits(np.concatenate([a_bits, b_bits]), dev),
                                dev_f32(np.concatenate([a_sc, b_sc]), dev))
    assert stacked.N == whole.N == 1777
    assert torch.equal(stacked.bits, whole.bits) and torch.equal(stacked.scales, whole.scales)


def test_pack_rows_leaves_other_rows_alone(pq, dev):
    # rows 960..1023 form one band shared by both matrices: packing the second
    # one must not touch the first one's entries (here: a sentinel)
    rng = np.random.default_rng(42)
    K, n1, n2 = 1024, 1000, 777
    b_bits, b_sc = wl.draw_bits(rng, n2, K), wl.draw_scales(rng, n2, K)
    lib = pq.load_library()
    nb, ns = lib.pq1_packed_bits_bytes(n1 + n2, K), lib.pq1_packed_scales_bytes(n1 + n2, K)
    pbits = torch.full((nb // 4,), 0x5A5A5A5A, dtype=torch.int32, device=dev)
    pscales = torch.full((ns // 4,), 7.0, dtype=torch.float32, device=dev)
    bb, bs = dev_bits(b_bits, dev), dev_f32(b_sc, dev)
    with torch.cuda.device(dev):
        rc = lib.pq1_pack_weights_rows(pq._ptr(bb), pq._ptr(bs), n2, K, pq._ptr(pbits),
                                       pq._ptr(pscales), n1 + n2, n1, pq._stream(dev))
    assert rc == 0
    G = K // 128
    words = host(pbits).view(np.uint32).reshape(-1, G, 64, 4)   # [band][group][lane][word]
    sc = host(pscales).reshape(-1, G, 64)
    rows = np.arange(words.shape[0] * 64)
    band, lane = rows // 64, rows % 64
    w_rows = words[band, :, lane, :]                            # [row][group][word]
    s_rows = sc[band, :, lane]
    first, second, pad = rows < n1, (rows >= n1) & (rows < n1 + n2), rows >= n1 + n2
    assert np.all(w_rows[first] == 0x5A5A5A5A) and np.all(s_rows[first] == 7.0)
    assert np.array_equal(w_rows[second].reshape(n2, -1), packed_word(b_bits))
    assert np.array_equal(s_rows[second], b_sc)
    assert np.all(w_rows[pad] == 0) and np.all(s_rows[pad] == 0.0)


def test_gate_up_in_one_launch(pq, dev):
    d = wl.make("gate_up")
    n = d["N"] // 2
    halves = [(dev_bits(d["bits"][:n], dev), dev_f32(d["scales"][:n], dev)),
              (dev_bits(d["bits"][n:], dev), dev_f32(d["scales"][n:], dev))]
    pw = pq.pq1_pack_weights_rows(halves)
    x, s = dev_f32(d["x"][0], dev), dev_f32(d["signs"], dev)
    y = host(pq.pq1_rotate_gemv_packed(x, s, pw))
    xr = orc.rotate(d["x"][0], d["signs"])
    ref = orc.gemv(xr, d["bits"], d["scales"])
    A = orc.normalizer(xr, d["bits"], d["scales"])
    assert_normalized(y, ref, A, TOL_F32, "gate + up stacked")
    # the same rows launched one matrix at a time
    for h, (b, sc) in enumerate(halves):
        yh = host(pq.pq1_rotate_gemv_packed(x, s, pq.pq1_pack_weights(b, sc)))
        assert_normalized(yh, ref[h * n:(h + 1) * n], A[h * n:(h + 1) * n], TOL_F32,
                          f"gate/up half {h} alone")


def test_lm_head_full_size(pq, dev):
    """Every one of the 248,320 output-head rows against the oracle."""
    d = wl.make("lm_head")
    pw = pq.pq1_pack_weights(dev_bits(d["bits"], dev), dev_f32(d["scales"], dev))
    y = host(pq.pq1_rotate_gemv_packed(dev_f32(d["x"][0], dev), dev_f32(d["signs"], dev), pw))
    xr = orc.rotate(d["x"][0], d["signs"])
    w = assert_rows_chunked(y, xr, d["bits"], d["scales"], TOL_F32, "lm_head", chunk=16384)
    print(f"  lm_head max err/A = {w:.2e}", flush=True)


def test_lm_head_integer_inputs_exact(pq, dev):
    """Every output-head row, bit-exact on inputs where every sum is exact."""
    rng = np.random.default_rng(77)
    N, K = 248320, 5120
    bits = wl.draw_bits(rng, N, K)
    scales = wl.power_of_two_scales(rng, N, K)
    xr = wl.integer_activation(rng, 1, K)[0]
    pw = pq.pq1_pack_weights(dev_bits(bits, dev), dev_f32(scales, dev))
    y = host(pq.pq1_gemv_packed(dev_f32(xr, dev), pw))
    assert_rows_chunked(y, xr, bits, scales, 0.0, "lm_head exact", exact=True, chunk=16384)


def test_lm_head_graph_replay_and_shared_workspace(pq, dev):
    """The output head's plan walks several band sets per workgroup; its
    split-K bookkeeping must survive graph replays and calls of another shape
    (ffn_gate) on the same workspace, checked on sampled rows."""
    d = wl.make("lm_head")
    g8 = wl.make("ffn_gate")
    pw = pq.pq1_pack_weights(dev_bits(d["bits"], dev), dev_f32(d["scales"], dev))
    pg = pq.pq1_pack_weights(dev_bits(g8["bits"], dev), dev_f32(g8["scales"], dev))
    x, s = dev_f32(d["x"][0], dev), dev_f32(d["signs"], dev)
    xg, sg = dev_f32(g8["x"][0], dev), dev_f32(g8["signs"], dev)
    rows = np.unique(np.concatenate([np.random.default_rng(6).integers(0, d["N"], 1500),
                                     [0, d["N"] - 1]]))
    xr = orc.rotate(d["x"][0], d["signs"])
    ref = orc.gemv_rows(xr, d["bits"], d["scales"], rows)
    A = orc.normalizer_rows(xr, d["bits"], d["scales"], rows)
    xrg = orc.rotate(g8["x"][0], g8["signs"])
    refg, Ag = orc.gemv(xrg, g8["bits"], g8["scales"]), orc.normalizer(xrg, g8["bits"], g8["scales"])
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    out = torch.empty(d["N"], dtype=torch.float32, device=dev)
    with torch.cuda.stream(side):
        pq.pq1_rotate_gemv_packed(x, s, pw, out=out)
    torch.cuda.synchronize()
    assert_normalized(host(out)[rows], ref, A, TOL_F32, "lm_head eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        pq.pq1_rotate_gemv_packed(x, s, pw, out=out)
    for r in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        assert_normalized(host(out)[rows], ref, A, TOL_F32, f"lm_head replay {r}")
        with torch.cuda.stream(side):  # another shape on the same workspace
            yg = pq.pq1_rotate_gemv_packed(xg, sg, pg)
        assert_normalized(host(yg), refg, Ag, TOL_F32, f"ffn_gate between replays {r}")


def test_embed_matches_oracle_full_table(pq, dev):
    d = wl.make_embedding(M=64)
    toks = d["tokens"].copy()
    toks[:3] = [0, d["V"] - 1, 12345]
    out = host(pq.pq1_embed(torch.from_numpy(toks).to(dev), dev_bits(d["bits"], dev),
                            dev_f32(d["scales"], dev), dev_f32(d["signs"], dev)))
    z = orc.embedding_rows(d["bits"], d["scales"], d["K"], toks)
    ref = orc.inverse_rotate(z, d["signs"])
    A = orc.rotate_normalizer(z, np.ones(d["K"]))
    assert_normalized(out, ref, A, TOL_F32, "embedding lookup")


def test_embed_exact_and_out_of_range_rows(pq, dev):
    rng = np.random.default_rng(8)
    V, K = 5000, 2048
    bits = wl.draw_bits(rng, V, K)
    scales = wl.power_of_two_scales(rng, V, K)
    signs = wl.draw_signs(rng, K)
    toks = np.array([7, -1, V, 4999, 0, 2 ** 31 - 1, 7], dtype=np.int32)
    out = host(pq.pq1_embed(torch.from_numpy(toks).to(dev), dev_bits(bits, dev),
                            dev_f32(scales, dev), dev_f32(signs, dev)))
    ok = (toks >= 0) & (toks < V)
    assert np.all(np.isnan(out[~ok]))
    ref = orc.inverse_rotate(orc.embedding_rows(bits, scales, K, toks[ok]), signs)
    assert np.array_equal(out[ok].astype(np.float64), ref)
    assert np.array_equal(out[0], out[6])


# ----------------------------------------------------------------------------
# GEMM (prefill)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K", [(128, 256, 1024), (100, 300, 640), (1, 17, 128),
                                   (257, 513, 5120), (64, 64, 2048)])
def test_gemm_integer_inputs_bit_exact(pq, dev, M, N, K):
    rng = np.random.default_rng(M * N + K)
    xb = wl.integer_bf16_bits(rng, M, K)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.power_of_two_scales(rng, N, K)
    Y = host(pq.pq1_gemm(dev_bf16(xb, dev), dev_bits(bits, dev), dev_f32(scales, dev)))
    X = orc.bf16_bits_to_float(xb)
    assert np.array_equal(Y.astype(np.float64), orc.gemm(X, bits, scales))


@pytest.mark.parametrize("M,N,K", [(128, 256, 1024), (200, 1000, 5120), (33, 96, 384)])
def test_gemm_random_bf16_inputs(pq, dev, M, N, K):
    rng = np.random.default_rng(M + N + K)
    xb = wl.random_bf16_bits(rng, M, K)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.draw_scales(rng, N, K)
    Y = host(pq.pq1_gemm(dev_bf16(xb, dev), dev_bits(bits, dev), dev_f32(scales, dev)))
    X = orc.bf16_bits_to_float(xb)
    ref = orc.gemm(X, bits, scales)
    A = orc.normalizer(X, bits, scales)
    assert_normalized(Y, ref, A, TOL_F32, f"gemm {M}x{N}x{K}")


def test_gemm_one_hot_rows(pq, dev):
    # X row m = e_{k(m)}: Y[m][n] = scale[n][k>>7] * (+-1)(n, k) for 256 positions k
    K, N = 1024, 300
    rng = np.random.default_rng(5)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.draw_scales(rng, N, K)
    ks = np.arange(0, K, 4)
    X = np.zeros((len(ks), K), dtype=np.float32)
    X[np.arange(len(ks)), ks] = 1.0
    xb = (X.view(np.uint32) >> 16).astype(np.uint16)
    Y = host(pq.pq1_gemm(dev_bf16(xb, dev), dev_bits(bits, dev), dev_f32(scales, dev)))
    W = orc.dequantize(bits, scales, K)
    assert np.array_equal(Y.astype(np.float64), W[:, ks].T)


def gemm_order_index(K):
    """Stored position -> natural K index of the GEMM operand order (the
    layout include/pq1.h documents for PQ1_BF16_GEMM)."""
    p = np.arange(K)
    pl = p % 32
    c, e = pl // 8, pl % 8
    return (p - pl) + 4 * c + e // 2 + 16 * (e % 2)


def test_rotate_gemm_order_output(pq, dev):
    d = wl.make("prefill", M=16)
    xb = bf16_host_bits(pq.pq1_rotate(dev_f32(d["x"], dev), dev_f32(d["signs"], dev),
                                      out_dtype=torch.bfloat16, gemm_order=True))
    xn = bf16_host_bits(pq.pq1_rotate(dev_f32(d["x"], dev), dev_f32(d["signs"], dev),
                                      out_dtype=torch.bfloat16))
    idx = gemm_order_index(d["K"])
    assert sorted(idx.tolist()) == list(range(d["K"]))
    assert np.array_equal(xb, xn[:, idx])


@pytest.mark.parametrize("M,N,K", [(128, 256, 1024), (100, 300, 640), (257, 513, 5120),
                                   (1, 17, 128)])
def test_gemm_gemm_order_bit_exact(pq, dev, M, N, K):
    rng = np.random.default_rng(M + 3 * N + K)
    xb = wl.integer_bf16_bits(rng, M, K)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.power_of_two_scales(rng, N, K)
    xg = np.ascontiguousarray(xb[:, gemm_order_index(K)])
    Y = host(pq.pq1_gemm(dev_bf16(xg, dev), dev_bits(bits, dev), dev_f32(scales, dev),
                         gemm_order=True))
    assert np.array_equal(Y.astype(np.float64), orc.gemm(orc.bf16_bits_to_float(xb), bits, scales))


@pytest.mark.parametrize("gemm_order", [False, True])
@pytest.mark.parametrize("M", [1, 2, 7, 8, 9, 15, 16, 17, 20, 31, 32, 33, 48, 63, 64, 65])
def test_gemm_small_m_bit_exact(pq, dev, M, gemm_order):
    """Short prompts (M <= 64 take the skinny kernel: 1-5 blocks of 16
    columns per workgroup, K split over its waves, 16 or 32 rows per wave;
    the 128-row tiles from 65 on): exact on integer activations and
    power-of-two scales, ragged N (300 = 18 x 16 + 12), both X layouts, both
    sides of every switch."""
    N, K = 300, 5120
    rng = np.random.default_rng(1000 + M)
    xb = wl.integer_bf16_bits(rng, M, K)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.power_of_two_scales(rng, N, K)
    xin = np.ascontiguousarray(xb[:, gemm_order_index(K)]) if gemm_order else xb
    Y = host(pq.pq1_gemm(dev_bf16(xin, dev), dev_bits(bits, dev), dev_f32(scales, dev),
                         gemm_order=gemm_order))
    assert np.array_equal(Y.astype(np.float64), orc.gemm(orc.bf16_bits_to_float(xb), bits, scales))


@pytest.mark.parametrize("M,N,K", [(5, 100, 128), (20, 33, 256), (9, 1000, 13056),
                                   (9, 1000, 20480), (9, 40, 26112), (9, 40, 26240),
                                   (18, 17, 1152), (40, 70, 640), (1, 17000, 1280),
                                   (16, 17000, 1280), (32, 17000, 1280), (64, 17000, 1280),
                                   (8, 16384, 640), (40, 1000, 13056), (40, 1000, 20480),
                                   (45, 17000, 1280), (40, 16384, 640), (64, 1000, 13056),
                                   (50, 16384, 640), (3, 1, 256), (64, 5, 128), (17, 15, 384)])
def test_gemm_skinny_edges_bit_exact(pq, dev, M, N, K):
    """Skinny-kernel edges: one K group (waves with no groups), fewer columns
    than a workgroup, K where the weights of the wider plans no longer fit the
    LDS limit (two blocks), where two no longer fit (one block), the largest
    K one block fits and the next K up (which takes the tiles), two row
    blocks of 32 with a ragged second one, and N wide enough for five column
    blocks per workgroup, with a last workgroup of three blocks whose last
    is half full and waves with an odd number of K groups (a re-read group
    folded with scale 0), N where four blocks balance best, 33-48 rows
    (three 16-row blocks per wave) with two blocks, one, five and four, and
    49-64 rows (four row blocks per wave) with two blocks, with four (whose
    partial blocks just fit the LDS) and with five (whose partial blocks
    are first added in pairs: 64 x 17000 above), and fewer than 16
    columns."""
    rng = np.random.default_rng(M * 7 + N + K)
    xb = wl.integer_bf16_bits(rng, M, K)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.power_of_two_scales(rng, N, K)
    ref = orc.gemm(orc.bf16_bits_to_float(xb), bits, scales)
    for gemm_order in (False, True):
        xin = np.ascontiguousarray(xb[:, gemm_order_index(K)]) if gemm_order else xb
        Y = host(pq.pq1_gemm(dev_bf16(xin, dev), dev_bits(bits, dev), dev_f32(scales, dev),
                             gemm_order=gemm_order))
        assert np.array_equal(Y.astype(np.float64), ref), f"{M}x{N}x{K} gemm_order={gemm_order}"


@pytest.mark.parametrize("M", [1, 16, 32, 48, 64])
def test_gemm_short_prompt_full_shape_bit_exact(pq, dev, M):
    """Short prompts against the prefill weights' full shape (N = 17408,
    K = 5120: the plans the bench times, five column blocks per workgroup on
    218 workgroups, 8 waves at 16 rows per wave, 4 at 32 and 48): every
    output exact on integer activations and power-of-two scales, both X
    layouts."""
    N, K = 17408, 5120
    rng = np.random.default_rng(4000 + M)
    xb = wl.integer_bf16_bits(rng, M, K)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.power_of_two_scales(rng, N, K)
    X = orc.bf16_bits_to_float(xb)
    ref = np.concatenate([orc.gemm(X, bits[c:c + 2048], scales[c:c + 2048])
                          for c in range(0, N, 2048)], axis=1)
    for gemm_order in (False, True):
        xin = np.ascontiguousarray(xb[:, gemm_order_index(K)]) if gemm_order else xb
        Y = host(pq.pq1_gemm(dev_bf16(xin, dev), dev_bits(bits, dev), dev_f32(scales, dev),
                             gemm_order=gemm_order))
        assert np.array_equal(Y.astype(np.float64), ref), f"M={M} gemm_order={gemm_order}"


@pytest.mark.parametrize("M,K", [(5, 640), (48, 1152), (20, 128)])
def test_gemm_small_m_random(pq, dev, M, K):
    N = 1000
    rng = np.random.default_rng(M * K)
    xb = wl.random_bf16_bits(rng, M, K)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.draw_scales(rng, N, K)
    for gemm_order in (False, True):
        xin = np.ascontiguousarray(xb[:, gemm_order_index(K)]) if gemm_order else xb
        Y = host(pq.pq1_gemm(dev_bf16(xin, dev), dev_bits(bits, dev), dev_f32(scales, dev),
                             gemm_order=gemm_order))
        X = orc.bf16_bits_to_float(xb)
        assert_normalized(Y, orc.gemm(X, bits, scales), orc.normalizer(X, bits, scales), TOL_F32,
                          f"small-M gemm {M}x{N}x{K} gemm_order={gemm_order}")


def test_gemm_small_m_full_width(pq, dev):
    d = wl.make("prefill", M=16)
    xb = pq.pq1_rotate(dev_f32(d["x"], dev), dev_f32(d["signs"], dev), out_dtype=torch.bfloat16,
                       gemm_order=True)
    Y = host(pq.pq1_gemm(xb, dev_bits(d["bits"], dev), dev_f32(d["scales"], dev), gemm_order=True))
    ns = np.unique(np.concatenate([np.random.default_rng(2).integers(0, d["N"], 600), [0, d["N"] - 1]]))
    xr = orc.rotate(d["x"], d["signs"])
    ms = np.repeat(np.arange(16), len(ns))
    nn = np.tile(ns, 16)
    got = Y[ms, nn]
    ref = orc.gemm_entries(xr, d["bits"], d["scales"], ms, nn)
    A = orc.normalizer_entries(xr, d["bits"], d["scales"], ms, nn)
    assert_normalized(got, ref, A, TOL_BF16, "small-M prefill, full width")


@pytest.mark.parametrize("gemm_order", [True, False])
def test_gemm_full_size_bit_exact(pq, dev, gemm_order):
    """The 1024 x 17408 x 5120 launch the prefill bench times, with X in the
    GEMM K order and row-major: every entry exact (small-integer activations,
    power-of-two scales).  On a 256-CU part the 1088 tiles leave 64 for a
    last round, which run as four 32-row pieces each, so both kinds of
    workgroup are covered."""
    M, N, K = 1024, 17408, 5120
    rng = np.random.default_rng(2024)
    xb = wl.integer_bf16_bits(rng, M, K)
    bits = wl.draw_bits(rng, N, K)
    scales = wl.power_of_two_scales(rng, N, K)
    xin = np.ascontiguousarray(xb[:, gemm_order_index(K)]) if gemm_order else xb
    Y = host(pq.pq1_gemm(dev_bf16(xin, dev), dev_bits(bits, dev), dev_f32(scales, dev),
                         gemm_order=gemm_order))
    assert_rows_chunked(Y, orc.bf16_bits_to_float(xb), bits, scales, 0.0,
                        f"prefill GEMM exact ({'GEMM' if gemm_order else 'row-major'} order)",
                        exact=True, chunk=4352)


def test_prefill_gemm_order_end_to_end(pq, dev):
    d = wl.make("prefill", M=64)
    xb = pq.pq1_rotate(dev_f32(d["x"], dev), dev_f32(d["signs"], dev), out_dtype=torch.bfloat16,
                       gemm_order=True)
    Y = host(pq.pq1_gemm(xb, dev_bits(d["bits"], dev), dev_f32(d["scales"], dev),
                         gemm_order=True))
    xr = orc.rotate(d["x"], d["signs"])
    ref = orc.gemm(xr, d["bits"], d["scales"])
    A = orc.normalizer(xr, d["bits"], d["scales"])
    assert_normalized(Y, ref, A, TOL_BF16, "prefill e2e gemm order")


def test_prefill_end_to_end_small(pq, dev):
    d = wl.make("prefill", M=96)
    xb = pq.pq1_rotate(dev_f32(d["x"], dev), dev_f32(d["signs"], dev), out_dtype=torch.bfloat16)
    Y = host(pq.pq1_gemm(xb, dev_bits(d["bits"], dev), dev_f32(d["scales"], dev)))
    xr = orc.rotate(d["x"], d["signs"])
    ref = orc.gemm(xr, d["bits"], d["scales"])
    A = orc.normalizer(xr, d["bits"], d["scales"])
    w = assert_normalized(Y, ref, A, TOL_BF16, "prefill e2e (96 rows)")
    print(f"  prefill e2e max err/A = {w:.2e}", flush=True)


@pytest.mark.parametrize("gemm_order", [False, True])
def test_prefill_full_size(pq, dev, gemm_order):
    """The whole prefill step (rotate to bf16, then the GEMM) at 1024 x 17408 x
    5120, every output against the oracle: within 1e-2 A of the product with
    the unrounded x', and within 2e-5 A of the product with x' rounded to bf16
    by the oracle (this separates the input rounding, which the method
    prescribes, from the fp32 accumulation)."""
    d = wl.make("prefill")
    xb = pq.pq1_rotate(dev_f32(d["x"], dev), dev_f32(d["signs"], dev), out_dtype=torch.bfloat16,
                       gemm_order=gemm_order)
    Y = host(pq.pq1_gemm(xb, dev_bits(d["bits"], dev), dev_f32(d["scales"], dev),
                         gemm_order=gemm_order))
    xr = orc.rotate(d["x"], d["signs"])
    w = assert_rows_chunked(Y, xr, d["bits"], d["scales"], TOL_BF16, "prefill vs unrounded x'",
                            chunk=4352)
    xr_b = orc.bf16_bits_to_float(orc.round_to_bf16(xr))
    wb = assert_rows_chunked(Y, xr_b, d["bits"], d["scales"], TOL_F32,
                             "prefill vs x' rounded to bf16", chunk=4352)
    print(f"  prefill max err/A: {w:.2e} (unrounded x'), {wb:.2e} (bf16 x')", flush=True)


# ----------------------------------------------------------------------------
# errors through the binding on a real device
# ----------------------------------------------------------------------------
def test_errors_on_device(pq, dev):
    x = torch.zeros(1025, dtype=torch.float32, device=dev)
    s = torch.ones(1024, dtype=torch.float32, device=dev)
    with pytest.raises(pq.Pq1Error) as e:
        pq.pq1_rotate(x[1:], s)  # 4-byte offset: misaligned
    assert e.value.code == 3
    w = torch.zeros((16, 32), dtype=torch.int32, device=dev)
    sc = torch.zeros((16, 8), dtype=torch.float32, device=dev)
    with pytest.raises(pq.Pq1Error) as e:
        pq.pq1_gemv(x[:1024], w, sc, out=sc.view(-1)[:16])
    assert e.value.code == 5


def test_binding_rejects_mismatched_sizes(pq, dev):
    """The library sees plain pointers and sizes; the binding refuses tensors
    whose element counts disagree with the sizes it passes (before any
    launch), so no kernel reads or writes past a tensor's end."""
    K, N, M = 1024, 64, 40
    f32 = dict(dtype=torch.float32, device=dev)
    x = torch.zeros(K, **f32)
    s = torch.ones(K, **f32)
    w = torch.zeros((N, K // 32), dtype=torch.int32, device=dev)
    sc = torch.ones((N, K // 128), **f32)
    cases = [
        ("rotate: short signs", lambda: pq.pq1_rotate(x, s[:512])),
        ("gemv: w_bits for another K", lambda: pq.pq1_gemv(x[:512], w, sc)),
        ("gemv: short scales", lambda: pq.pq1_gemv(x, w, torch.ones((N, 4), **f32))),
        ("gemv: short out", lambda: pq.pq1_gemv(x, w, sc, out=torch.empty(N - 1, **f32))),
        ("rotate_gemv: short signs", lambda: pq.pq1_rotate_gemv(x, s[:512], w, sc)),
        ("gemm: short out", lambda: pq.pq1_gemm(torch.zeros((M, K), dtype=torch.bfloat16, device=dev),
                                                w, sc, out=torch.empty((M, N - 1), **f32))),
        ("gemm: w_bits for another K", lambda: pq.pq1_gemm(
            torch.zeros((M, 2 * K), dtype=torch.bfloat16, device=dev), w, sc)),
        ("embed: short out", lambda: pq.pq1_embed(torch.zeros(3, dtype=torch.int32, device=dev),
                                                  w, sc, s, out=torch.empty((2, K), **f32))),
        ("pack: short scales", lambda: pq.pq1_pack_weights(w, torch.ones((N, 4), **f32))),
    ]
    pw = pq.pq1_pack_weights(w, sc)
    cases += [
        ("gemv_packed: x of another K", lambda: pq.pq1_gemv_packed(x[:512], pw)),
        ("gemv_packed: short out", lambda: pq.pq1_gemv_packed(x, pw, out=torch.empty(N - 1, **f32))),
        ("rotate_gemv_packed: short signs", lambda: pq.pq1_rotate_gemv_packed(x, s[:512], pw)),
        ("rotate_gemv_packed: x of another K", lambda: pq.pq1_rotate_gemv_packed(
            torch.zeros(2 * K, **f32), torch.ones(2 * K, **f32), pw)),
        ("gemv_packed: truncated packed bits", lambda: pq.pq1_gemv_packed(
            x, pq.PackedWeights(pw.bits[:16], pw.scales, N, K))),
    ]
    for what, call in cases:
        with pytest.raises(ValueError):
            call()
            pytest.fail(f"{what}: accepted")
    torch.cuda.synchronize()
