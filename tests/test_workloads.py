"""Checks of the seeded input generator against the pages' input statistics."""
import json
import os

import numpy as np
import pytest

from gemm_hadamard_rotated_amd import workloads as wl

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def test_config_shapes():
    c = wl.CONFIGS
    assert (c["tiny"].M, c["tiny"].K, c["tiny"].N) == (1, 1024, 256)
    assert (c["ffn_gate"].K, c["ffn_gate"].N) == (5120, 17408)
    assert (c["ffn_down"].K, c["ffn_down"].N) == (17408, 5120)
    assert (c["ssm_out"].K, c["ssm_out"].N, c["ssm_out"].perm) == (6144, 5120, (128, 16, 3))
    assert (c["prefill"].M, c["prefill"].K, c["prefill"].N) == (1024, 5120, 17408)
    widths = sorted({c[k].K for k in ("ffn_gate", "ffn_down", "ssm_out")})
    assert widths == FACTS["sign_widths"]["value"]
    # stacked gate + up: two ffn_gate-shaped matrices on one activation
    assert (c["gate_up"].K, c["gate_up"].N) == (c["ffn_gate"].K, 2 * c["ffn_gate"].N)
    # the output head and the embedding table: vocabulary x hidden
    vt = FACTS["vocab_table"]
    assert (c["lm_head"].N, c["lm_head"].K) == (vt["rows"], vt["width"])
    assert c["lm_head"].K == FACTS["output_head_convention"]["in_width"]
    assert (wl.EMBED_ROWS, wl.EMBED_WIDTH) == (vt["rows"], vt["width"])
    assert vt["rows"] * vt["width"] == vt["bits_per_table"]
    # 640 bytes of bits + 80 of f16 scales per row on the pages
    assert vt["rows"] * FACTS["row_bytes_f16_scales_5120"]["value"] == vt["bytes_f16_scales"]


def test_embedding_inputs_are_reproducible():
    a = wl.make_embedding(M=8, V=1000, K=2048)
    b = wl.make_embedding(M=8, V=1000, K=2048)
    for k in ("bits", "scales", "signs", "tokens"):
        assert np.array_equal(a[k], b[k])
    assert a["tokens"].dtype == np.int32 and a["tokens"].min() >= 0 and a["tokens"].max() < 1000
    assert a["bits"].shape == (1000, 64) and a["scales"].shape == (1000, 16)


def test_tiny_is_reproducible_and_sized():
    a = wl.make("tiny")
    b = wl.make("tiny")
    for k in ("bits", "scales", "signs", "x"):
        assert np.array_equal(a[k], b[k])
    assert a["bits"].shape == (256, 32) and a["bits"].dtype == np.uint32
    assert a["scales"].shape == (256, 8) and a["scales"].dtype == np.float32
    assert a["bits"].nbytes == 256 * 1024 // 8
    assert a["scales"].nbytes == 4 * 256 * 1024 // 128
    c = wl.make("tiny", seed=5)
    assert not np.array_equal(a["bits"], c["bits"])


def test_bit_statistics_match_fair_coins():
    d = wl.make("ffn_gate")
    bits = d["bits"][:2048]
    # popcount of each 128-weight group (4 words)
    pc = np.bitwise_count(bits).reshape(2048, -1, 4).sum(axis=2).ravel()
    var = pc.var()
    # Binomial(128, 1/2): mean 64, variance 32; 81920 groups -> sd(var) ~ 0.16
    assert abs(pc.mean() - 64.0) < 0.2
    assert abs(var - FACTS["popcount_variance_128"]["value"]) < 1.0


def test_scales_signs_ranges():
    d = wl.make("ssm_out")
    assert d["scales"].min() >= wl.SCALE_LO and d["scales"].max() <= wl.SCALE_HI
    assert set(np.unique(d["signs"])) == {-1.0, 1.0}
    assert abs(d["signs"].mean()) < 0.05
    assert d["x"].shape == (1, 6144)


def test_outlier_channels():
    d = wl.make("ffn_gate")
    big = np.abs(d["x"][0]) > 8.0
    # 8 channels scaled by 20 from N(0,1): most land above 8, normals never do
    assert 4 <= big.sum() <= 8


def test_swiglu_activation():
    d = wl.make("ffn_down")
    x = d["x"][0]
    assert x.shape == (17408,)
    # silu(a)*b has mean ~0 and heavier tails than a normal of the same sd
    assert abs(x.mean()) < 0.05
    kurt = ((x - x.mean()) ** 4).mean() / x.var() ** 2
    assert kurt > 4.0


def test_exact_generators():
    rng = np.random.default_rng(0)
    x = wl.integer_activation(rng, 2, 1024)
    assert np.all(x == np.round(x)) and np.abs(x).max() <= 8
    s = wl.power_of_two_scales(rng, 4, 1024)
    assert np.all(np.log2(s) == np.round(np.log2(s)))
    b = wl.integer_bf16_bits(rng, 2, 256)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    assert np.all(f == np.round(f)) and np.abs(f).max() <= 8


@pytest.mark.parametrize("name", ["tiny", "ssm_out"])
def test_make_prefill_rows_override(name):
    d = wl.make(name, M=3)
    assert d["x"].shape == (3, d["K"])
