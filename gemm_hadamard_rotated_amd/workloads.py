"""Seeded synthetic inputs for the rotated 1-bit GEMV/GEMM.

This module only draws random inputs; it holds none of the method's
arithmetic (no rotation, no unpacking, no products), so both the HIP path and
the CPU oracle can be fed from it without sharing any computation.

Shapes follow the widths the tested 27B model uses (hidden 5120, ssm-inner
6144, ffn 17408; Pulse ARCHITECTURE-SPEC metadata table and per-weight
convention table).  Distributions:

* weight bits: fair coin flips, packed LSB-first into uint32 words along K
  ("Inside the One-Bit Engine", station "The 27 billion sign bits pass every
  test for fair coin flips": per-128-group popcount variance is 32, the
  Binomial(128, 1/2) value);
* scales: fp32, uniform in [0.005, 0.05], one per 128 weights;
* signs: +-1 fp32, fair coin;
* activations: fp32 N(0, 1), with the per-config structure listed in
  ``CONFIGS``.

Draw order for every config: bits, scales, signs, activation.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

SCALE_LO, SCALE_HI = 0.005, 0.05


@dataclass(frozen=True)
class Config:
    name: str
    M: int
    K: int
    N: int
    seed: int
    perm: Optional[Tuple[int, int, int]]  # (hd, nk, rep) or None
    x_kind: str                           # "normal" | "outliers" | "swiglu"
    description: str


CONFIGS = {
    "tiny": Config("tiny", 1, 1024, 256, 1001, None, "normal",
                   "M=1 K=1024 N=256, one transform block"),
    "ffn_gate": Config("ffn_gate", 1, 5120, 17408, 1002, None, "outliers",
                       "decode ffn_gate: M=1 K=5120 N=17408, 8 outlier channels x20"),
    "ffn_down": Config("ffn_down", 1, 17408, 5120, 1003, None, "swiglu",
                       "decode ffn_down: M=1 K=17408 N=5120, x = silu(a)*b"),
    "ssm_out": Config("ssm_out", 1, 6144, 5120, 1004, (128, 16, 3), "normal",
                      "decode ssm_out: M=1 K=6144 N=5120, tiled->grouped heads"),
    "prefill": Config("prefill", 1024, 5120, 17408, 1005, None, "normal",
                      "prefill: M=1024 K=5120 N=17408, x' cast to bf16"),
    # ffn_gate and ffn_up take the same rotated activation; rows 0..17407 are
    # the gate matrix, rows 17408.. the up matrix, packed one after the other
    "gate_up": Config("gate_up", 1, 5120, 2 * 17408, 1006, None, "outliers",
                      "decode ffn_gate + ffn_up stacked: M=1 K=5120 N=2x17408"),
    # the output head: vocabulary 248,320 x hidden 5,120 ("Inside the One-Bit
    # Engine", station on the vocabulary binarized twice), signs + WHT
    "lm_head": Config("lm_head", 1, 5120, 248320, 1007, None, "normal",
                      "decode output head: M=1 K=5120 N=248320"),
}

# The token-embedding table: vocabulary x hidden, stored rotated (lookups use
# the inverse rotation).
EMBED_ROWS, EMBED_WIDTH, EMBED_SEED = 248320, 5120, 1008


def draw_bits(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """[N][K/32] uint32, every bit an independent fair coin."""
    return rng.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint32)


def draw_scales(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    return rng.uniform(SCALE_LO, SCALE_HI, size=(N, K // 128)).astype(np.float32)


def draw_signs(rng: np.random.Generator, K: int) -> np.ndarray:
    return (rng.integers(0, 2, size=K).astype(np.float32) * 2.0 - 1.0).astype(np.float32)


def draw_activation(rng: np.random.Generator, M: int, K: int, kind: str) -> np.ndarray:
    if kind == "normal":
        x = rng.standard_normal((M, K))
    elif kind == "outliers":
        x = rng.standard_normal((M, K))
        ch = rng.choice(K, size=8, replace=False)
        x[:, ch] *= 20.0
    elif kind == "swiglu":
        a = rng.standard_normal((M, K))
        b = rng.standard_normal((M, K))
        x = a / (1.0 + np.exp(-a)) * b
    else:
        raise ValueError(kind)
    return x.astype(np.float32)


def make(name: str, seed: Optional[int] = None, M: Optional[int] = None) -> dict:
    """Inputs of one named config: bits, scales, signs, x (and the shape).

    ``x`` is [M][K] (M=1 for the decode configs).  ``M`` may override the
    row count of the activation (used for small prefill parity cases).
    """
    c = CONFIGS[name]
    rng = np.random.default_rng(c.seed if seed is None else seed)
    Mx = c.M if M is None else M
    bits = draw_bits(rng, c.N, c.K)
    scales = draw_scales(rng, c.N, c.K)
    signs = draw_signs(rng, c.K)
    x = draw_activation(rng, Mx, c.K, c.x_kind)
    return dict(cfg=c, M=Mx, K=c.K, N=c.N, perm=c.perm,
                bits=bits, scales=scales, signs=signs, x=x)


def make_embedding(M: int = 1, seed: int = EMBED_SEED, V: int = EMBED_ROWS,
                   K: int = EMBED_WIDTH) -> dict:
    """An embedding table (bits, scales), the hidden-width signs and M token
    ids drawn uniformly from [0, V); draw order bits, scales, signs, tokens."""
    rng = np.random.default_rng(seed)
    bits = draw_bits(rng, V, K)
    scales = draw_scales(rng, V, K)
    signs = draw_signs(rng, K)
    tokens = rng.integers(0, V, size=M).astype(np.int32)
    return dict(M=M, K=K, V=V, bits=bits, scales=scales, signs=signs, tokens=tokens)


def make_shape(N: int, K: int, M: int = 1, seed: int = 0, x_kind: str = "normal") -> dict:
    """Inputs of an arbitrary shape with the standard distributions."""
    rng = np.random.default_rng(seed)
    bits = draw_bits(rng, N, K)
    scales = draw_scales(rng, N, K)
    signs = draw_signs(rng, K)
    x = draw_activation(rng, M, K, x_kind)
    return dict(M=M, K=K, N=N, bits=bits, scales=scales, signs=signs, x=x)


# ----------------------------------------------------------------------------
# Inputs on which every sum is exact in fp32 (bit-exact pins)
# ----------------------------------------------------------------------------
def integer_activation(rng: np.random.Generator, M: int, K: int, lo: int = -8, hi: int = 8):
    """Small integers: every +-1 combination of 1024 of them is exact in fp32."""
    return rng.integers(lo, hi + 1, size=(M, K)).astype(np.float32)


def power_of_two_scales(rng: np.random.Generator, N: int, K: int):
    """Scales 2^-7 .. 2^-4: products and sums with integers stay exact."""
    e = rng.integers(-7, -3, size=(N, K // 128))
    return np.ldexp(np.ones_like(e, dtype=np.float32), e).astype(np.float32)


def sparse_integer_activation(rng: np.random.Generator, M: int, K: int, nnz: int = 4):
    """A few small integer spikes per row: the rotated values need at most a
    few significant bits, so they are exact in bfloat16 as well."""
    x = np.zeros((M, K), dtype=np.float32)
    for m in range(M):
        pos = rng.choice(K, size=nnz, replace=False)
        x[m, pos] = rng.choice(np.array([-2.0, -1.0, 1.0, 2.0], dtype=np.float32), size=nnz)
    return x


def random_bf16_bits(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    """bfloat16 bit patterns of N(0,1) draws (top 16 bits of the fp32 draw)."""
    f = rng.standard_normal((M, K)).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def integer_bf16_bits(rng: np.random.Generator, M: int, K: int, lo: int = -8, hi: int = 8):
    """bfloat16 bit patterns of small integers (exactly representable)."""
    f = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
