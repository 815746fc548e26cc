"""The packed-layout GEMV's split-K handshake reports trouble instead of
failing silently.

K chunk 0 of a row block zeroes the rows and advances a generation word per
(band, K chunk); the other chunks wait for it before they add their partial
sums.  Two failure paths are forced from the host, each with every kernel
ending normally:

* a workspace whose generation and seen words disagree (as after a wait that
  gave up, or a workspace that was never zero-filled): K chunk 0 notices at
  the launch, sets the band's rows to NaN, reports PQ1_SPLITK_OUT_OF_STEP and
  puts the pair back in step;
* K chunk 0 withholding its publish (the library's test flag): the other
  chunks' bounded waits expire, they add NaN and report
  PQ1_SPLITK_WAIT_GAVE_UP.

The binding turns either report into Pq1Error(PQ1_ERR_SPLITK), and the next
call is correct again.
"""
import numpy as np
import pytest
import torch

import oracle.pq1_oracle as orc
from gemm_hadamard_rotated_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-5
MAX_SLOTS = 28640  # generation words, then as many seen words, in the counter region
FLAG_OFFSET = 32768


@pytest.fixture(scope="module")
def pq(dev):
    from gemm_hadamard_rotated_amd import pq1
    pq1.load_library()
    return pq1


def _case(dev, N, K, seed):
    d = wl.make_shape(N, K, seed=seed)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    bits = torch.from_numpy(d["bits"].view(np.int32)).to(dev)
    xr = orc.rotate(d["x"][0], d["signs"])
    ref = orc.gemv(xr, d["bits"], d["scales"])
    A = orc.normalizer(xr, d["bits"], d["scales"])
    return d, f32(d["x"][0]), f32(d["signs"]), bits, f32(d["scales"]), ref, A


def _err(y, ref, A):
    return float(np.max(np.abs(y.astype(np.float64) - ref) / A))


def test_clean_calls_report_nothing(pq, dev):
    _, x, s, bits, sc, ref, A = _case(dev, 1000, 4096, 3)
    pw = pq.pq1_pack_weights(bits, sc)
    for _ in range(3):
        y = pq.pq1_rotate_gemv_packed(x, s, pw)
    pq.check_gemv_workspace(dev)  # raises on any status bit
    torch.cuda.synchronize()
    assert _err(y.cpu().numpy(), ref, A) <= TOL_F32


def test_out_of_step_pair_is_reported_and_repaired(pq, dev):
    N, K = 1000, 4096          # 16 bands of 64 rows, 4 K chunks of 1024
    _, x, s, bits, sc, ref, A = _case(dev, N, K, 4)
    pw = pq.pq1_pack_weights(bits, sc)
    y = pq.pq1_rotate_gemv_packed(x, s, pw)
    pq.check_gemv_workspace(dev)
    ws = pq.gemv_workspace(N, K, dev)
    words = ws[:pq.PQ1_GEMV_COUNTER_BYTES].view(torch.int32)
    nkt, band, chunk = K // 1024, 5, 2
    slot = band * nkt + chunk
    gen_i, seen_i = FLAG_OFFSET // 4 + slot, FLAG_OFFSET // 4 + MAX_SLOTS + slot
    torch.cuda.synchronize()
    gen, seen = int(words[gen_i]), int(words[seen_i])
    assert gen == seen, "the pair is in step after a clean call"
    words[seen_i] = seen + 5                    # as after an earlier expired wait
    torch.cuda.synchronize()
    y = pq.pq1_rotate_gemv_packed(x, s, pw).cpu().numpy()
    rows = np.arange(N)
    poisoned = (rows // 64) == band
    assert np.all(np.isnan(y[poisoned])), "the band's rows are NaN for this call"
    assert _err(y[~poisoned], ref[~poisoned], A[~poisoned]) <= TOL_F32
    with pytest.raises(pq.Pq1Error) as e:
        pq.check_gemv_workspace(dev)
    assert e.value.code == pq.PQ1_ERR_SPLITK and "out of step" in str(e.value)
    # the check zero-filled the counter region; now a pair with gen behind
    # seen: K chunk 0 alone puts it back in step (publishing seen + 1)
    torch.cuda.synchronize()
    assert int(words[gen_i]) == int(words[seen_i]) == 0
    words[seen_i] = 9
    words[gen_i] = 3
    torch.cuda.synchronize()
    pq.pq1_rotate_gemv_packed(x, s, pw)        # repairs (and poisons once)
    torch.cuda.synchronize()
    assert int(words[gen_i]) == int(words[seen_i]) == 10
    status = int(ws[pq.PQ1_GEMV_STATUS_OFFSET:pq.PQ1_GEMV_STATUS_OFFSET + 4].view(torch.int32))
    assert status == pq.PQ1_SPLITK_OUT_OF_STEP
    ws[pq.PQ1_GEMV_STATUS_OFFSET:pq.PQ1_GEMV_STATUS_OFFSET + 4].zero_()
    y = pq.pq1_rotate_gemv_packed(x, s, pw).cpu().numpy()
    pq.check_gemv_workspace(dev)
    assert _err(y, ref, A) <= TOL_F32


def test_expired_wait_is_reported(pq, dev):
    N, K = 256, 2048           # 4 bands, 2 K chunks: K chunk 1 waits for chunk 0
    _, x, s, bits, sc, ref, A = _case(dev, N, K, 5)
    pw = pq.pq1_pack_weights(bits, sc)
    y = pq.pq1_rotate_gemv_packed(x, s, pw)
    pq.check_gemv_workspace(dev)
    prev = pq.pq1_set_test_flags(pq.PQ1_TEST_WITHHOLD_PUBLISH)
    try:
        y = pq.pq1_rotate_gemv_packed(x, s, pw)
        torch.cuda.synchronize()                # every kernel ends (bounded waits)
    finally:
        pq.pq1_set_test_flags(prev)
    assert np.all(np.isnan(y.cpu().numpy())), "every row waited in vain: NaN"
    with pytest.raises(pq.Pq1Error) as e:
        pq.check_gemv_workspace(dev)           # also zero-fills the counter region
    assert e.value.code == pq.PQ1_ERR_SPLITK and "gave up" in str(e.value)
    y = pq.pq1_rotate_gemv_packed(x, s, pw).cpu().numpy()
    pq.check_gemv_workspace(dev)
    assert _err(y, ref, A) <= TOL_F32
