"""Plain, slow, fp64 CPU oracle for the Hadamard-rotated 1-bit GEMV/GEMM.

TEST INFRASTRUCTURE ONLY -- used by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; the HIP library never calls it
and shares no code, constant table or helper with it.

Sources (cited by page title and section):

* "Inside the One-Bit Engine" (mentria.ai engine facts), station "A weight is
  one bit": a weight bit 1 means +1, bit 0 means -1, and 128 consecutive
  weights along K share one scale.  Stations "A token's embedding is 5,120
  numbers ..." and "A one-bit weight row cannot change its length": the
  weight of row ``n`` at input position ``k`` is bit ``k & 31`` of 32-bit word
  ``k >> 5`` of that row, and its scale is group ``k >> 7``.
* Pulse ARCHITECTURE-SPEC, Hadamard-fold notes ("Order" block): the activation
  is first head-permuted (tiled -> grouped, only when the repetition factor is
  above one), then multiplied element-wise by an explicit +-1 sign vector,
  then passed through a normalized Sylvester-Walsh-Hadamard transform with
  block 1024 and scale 1/32, and only then multiplied by W.  The same notes
  give the inverse order for the embedding table (transform first, then
  signs), the tiled [hd=128, nk=16, rep=3] -> grouped [hd, rep, nk]
  permutation of the ssm_out input, and the head-mapping table (grouped
  layout: key head = h / 3 blocks; tiled layout: key head = h % 16).
* Pulse ARCHITECTURE-SPEC, method notes: errors are scaled by the sum of the
  absolute values of the terms, not by the result.
* "Inside the One-Bit Engine", station "A token's embedding is 5,120 numbers
  ..." and the bits-per-weight table of station "Cutting a weight from 16 bits
  to 1.125 ...": the shipped format stores each group's scale as a 16-bit
  IEEE float (f16).  Scales given in fp32 are rounded to f16 to the nearest
  value, ties to even (IEEE 754 binary16, the default rounding); the product
  then uses the rounded value exactly.

Readings where the pages leave a step open:

* Sylvester order means the natural (not sequency) order,
  ``H[i][j] = (-1)^popcount(i & j)``; the transform is block-diagonal over
  contiguous 1024-element blocks of K, every block with the same matrix, and
  normalized by multiplying with 1/32.
* The permutation's axes are listed fastest-first: in the tiled layout head
  ``h = n + nk*r``, in the grouped layout head ``h' = r + rep*n``; the
  destination (grouped) head ``h'`` takes the source (tiled) head ``h`` with
  the same ``(n, r)``; each head is ``hd`` contiguous values.
* The sign vector is indexed in the post-permutation order.

All arithmetic is fp64 on the fp32 / uint32 input bytes.  Matrix products use
numpy's matmul as the library primitive; there is no blocking or reordering
beyond the definitions above.
"""
from __future__ import annotations

import numpy as np

WHT_BLOCK = 1024          # block length of the transform (Hadamard-fold notes)
WHT_SCALE = 1.0 / 32.0    # normalization: 1/sqrt(1024)
GROUP = 128               # weights per shared scale (station "A weight is one bit")
WORD_BITS = 32            # weights per packed 32-bit word

__all__ = [
    "WHT_BLOCK", "WHT_SCALE", "GROUP", "WORD_BITS",
    "sylvester_hadamard", "fwht_fp64", "head_source_index",
    "permute_tiled_to_grouped", "rotate", "rotate_normalizer",
    "inverse_rotate", "weight_signs", "dequantize", "gemv", "gemm",
    "gemv_rows", "gemm_entries", "normalizer", "normalizer_rows",
    "normalizer_entries", "round_to_bf16", "bf16_bits_to_float",
    "embedding_rows", "round_to_f16", "f16_bits_to_float", "scales_as_f16",
]


# ----------------------------------------------------------------------------
# Hadamard transform
# ----------------------------------------------------------------------------
def sylvester_hadamard(n: int = WHT_BLOCK) -> np.ndarray:
    """Dense Sylvester Hadamard matrix of order ``n`` (a power of two), fp64.

    Entry (i, j) is +1 when ``i & j`` has an even number of set bits and -1
    otherwise -- the natural-order Sylvester matrix named in the Pulse
    ARCHITECTURE-SPEC Hadamard-fold notes.  Unnormalized.
    """
    if n <= 0 or n & (n - 1):
        raise ValueError("order must be a power of two")
    idx = np.arange(n, dtype=np.uint64)
    parity = np.bitwise_count(np.bitwise_and.outer(idx, idx)) & 1
    return np.where(parity == 0, 1.0, -1.0)


def fwht_fp64(v: np.ndarray) -> np.ndarray:
    """Unnormalized fast Walsh-Hadamard transform along the last axis, fp64.

    The textbook radix-2 butterfly (a, b) -> (a + b, a - b) over strides
    1, 2, 4, ...; it equals multiplication by ``sylvester_hadamard``.  Kept as
    an independent second route to the same product so the two can be
    cross-checked.
    """
    a = np.array(v, dtype=np.float64, copy=True)
    n = a.shape[-1]
    if n <= 0 or n & (n - 1):
        raise ValueError("length must be a power of two")
    h = 1
    while h < n:
        a = a.reshape(a.shape[:-1] + (n // (2 * h), 2, h))
        lo = a[..., 0, :].copy()
        hi = a[..., 1, :].copy()
        a[..., 0, :] = lo + hi
        a[..., 1, :] = lo - hi
        a = a.reshape(a.shape[:-3] + (n,))
        h *= 2
    return a


# ----------------------------------------------------------------------------
# Head permutation (ssm_out input)
# ----------------------------------------------------------------------------
def head_source_index(hd: int, nk: int, rep: int) -> np.ndarray:
    """For each destination position of the grouped layout, its source position.

    Tiled layout [hd, nk, rep] (fastest axis first): head ``n + nk*r``.
    Grouped layout [hd, rep, nk]: head ``r + rep*n``.  Destination head
    ``r + rep*n`` copies source head ``n + nk*r``; within a head the ``hd``
    values keep their order.
    """
    if hd < 1 or nk < 1 or rep < 1:
        raise ValueError("hd, nk and rep must be positive")
    src = np.empty(hd * nk * rep, dtype=np.int64)
    for n in range(nk):
        for r in range(rep):
            dst_head = r + rep * n
            src_head = n + nk * r
            src[dst_head * hd:(dst_head + 1) * hd] = np.arange(
                src_head * hd, (src_head + 1) * hd)
    return src


def permute_tiled_to_grouped(x: np.ndarray, hd: int, nk: int, rep: int) -> np.ndarray:
    """Apply the tiled -> grouped head permutation along the last axis."""
    x = np.asarray(x)
    if x.shape[-1] != hd * nk * rep:
        raise ValueError("last axis must equal hd * nk * rep")
    return x[..., head_source_index(hd, nk, rep)]


# ----------------------------------------------------------------------------
# Activation rotation
# ----------------------------------------------------------------------------
def _check_perm(perm):
    if perm is None:
        return None
    hd, nk, rep = (int(v) for v in perm)
    if rep <= 1:
        return None
    return hd, nk, rep


def rotate(x: np.ndarray, signs: np.ndarray, perm=None) -> np.ndarray:
    """x' = WHT_1024(signs * P x), normalized by 1/32, fp64.

    Order from the Pulse ARCHITECTURE-SPEC "Order" block: optional tiled ->
    grouped permutation (only when rep > 1), element-wise signs, then the
    block-diagonal Sylvester transform with block 1024 and scale 1/32.  The
    transform is the dense matrix product with ``sylvester_hadamard(1024)``.
    ``x`` is [K] or [M][K]; K must be a multiple of 1024.
    """
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    K = x.shape[-1]
    if K % WHT_BLOCK:
        raise ValueError("K must be a multiple of 1024")
    if s.shape != (K,):
        raise ValueError("signs must have shape [K]")
    p = _check_perm(perm)
    xp = permute_tiled_to_grouped(x, *p) if p else x
    xs = xp * s
    blocks = xs.reshape(xs.shape[:-1] + (K // WHT_BLOCK, WHT_BLOCK))
    H = sylvester_hadamard(WHT_BLOCK)
    out = (blocks @ H) * WHT_SCALE       # H is symmetric
    return out.reshape(x.shape)


def rotate_normalizer(x: np.ndarray, signs: np.ndarray, perm=None) -> np.ndarray:
    """Per-output sum of |terms| of ``rotate``: (1/32) * sum over the block of |x|.

    Every output element of a block is a +-1 combination of all 1024 inputs of
    that block, so the sum of the absolute values of its terms is the same
    for the whole block.
    """
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    p = _check_perm(perm)
    xp = permute_tiled_to_grouped(x, *p) if p else x
    a = np.abs(xp * np.asarray(signs, dtype=np.float64))
    blocks = a.reshape(a.shape[:-1] + (K // WHT_BLOCK, WHT_BLOCK))
    per_block = blocks.sum(axis=-1, keepdims=True) * WHT_SCALE
    return np.broadcast_to(per_block, blocks.shape).reshape(x.shape).copy()


def inverse_rotate(z: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """h = signs * WHT_1024(z): the embedding-side order (transform, then signs).

    Pulse ARCHITECTURE-SPEC Hadamard-fold notes: the embedding table stores
    rotated rows, and the lookup restores the primal basis by applying the
    transform first and the signs second.  Normalized by 1/32 like ``rotate``.
    """
    z = np.asarray(z, dtype=np.float64)
    K = z.shape[-1]
    if K % WHT_BLOCK:
        raise ValueError("K must be a multiple of 1024")
    blocks = z.reshape(z.shape[:-1] + (K // WHT_BLOCK, WHT_BLOCK))
    H = sylvester_hadamard(WHT_BLOCK)
    t = ((blocks @ H) * WHT_SCALE).reshape(z.shape)
    return t * np.asarray(signs, dtype=np.float64)


# ----------------------------------------------------------------------------
# 1-bit weights
# ----------------------------------------------------------------------------
def weight_signs(w_bits: np.ndarray, K: int) -> np.ndarray:
    """Unpack [N][K/32] uint32 words to the [N][K] +-1 weight matrix (int8).

    Weight (n, k) is bit ``k & 31`` of word ``k >> 5`` of row ``n``; a set bit
    is +1 and a clear bit is -1.
    """
    words = np.asarray(w_bits, dtype=np.uint32)
    if K % WORD_BITS or words.ndim != 2 or words.shape[1] != K // WORD_BITS:
        raise ValueError("w_bits must be [N][K/32] with K a multiple of 32")
    k = np.arange(K)
    bits = (words[:, k >> 5] >> (k & 31).astype(np.uint32)) & np.uint32(1)
    return (bits.astype(np.int8) * 2 - 1).astype(np.int8)


def dequantize(w_bits: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """Dense fp64 weights W[n][k] = scale[n][k >> 7] * (+-1)."""
    s = np.asarray(scales, dtype=np.float64)
    pm = weight_signs(w_bits, K)
    if K % GROUP or s.shape != (pm.shape[0], K // GROUP):
        raise ValueError("scales must be [N][K/128]")
    return pm.astype(np.float64) * np.repeat(s, GROUP, axis=1)


def gemv(x_rot: np.ndarray, w_bits: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """y = W x' in fp64 for a [K] activation."""
    x = np.asarray(x_rot, dtype=np.float64)
    return dequantize(w_bits, scales, x.shape[-1]) @ x


def gemm(x_rot: np.ndarray, w_bits: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Y = X' W^T in fp64 for an [M][K] activation block."""
    X = np.asarray(x_rot, dtype=np.float64)
    return X @ dequantize(w_bits, scales, X.shape[-1]).T


def normalizer(x_rot: np.ndarray, w_bits: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """A = sum_k |W[n][k] * x'[k]| (per output; [M][N] for a matrix input)."""
    X = np.asarray(x_rot, dtype=np.float64)
    Wabs = np.abs(dequantize(w_bits, scales, X.shape[-1]))
    return np.abs(X) @ Wabs.T


def gemv_rows(x_rot, w_bits, scales, rows) -> np.ndarray:
    """``gemv`` restricted to the listed output rows."""
    rows = np.asarray(rows, dtype=np.int64)
    return gemv(x_rot, np.asarray(w_bits)[rows], np.asarray(scales)[rows])


def normalizer_rows(x_rot, w_bits, scales, rows) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    return normalizer(x_rot, np.asarray(w_bits)[rows], np.asarray(scales)[rows])


def gemm_entries(x_rot, w_bits, scales, ms, ns):
    """Y[m][n] for the listed (m, n) pairs of a [M][K] x' block."""
    X = np.asarray(x_rot, dtype=np.float64)
    ms = np.asarray(ms, dtype=np.int64)
    ns = np.asarray(ns, dtype=np.int64)
    W = dequantize(np.asarray(w_bits)[ns], np.asarray(scales)[ns], X.shape[-1])
    return np.einsum("ik,ik->i", X[ms], W)


def normalizer_entries(x_rot, w_bits, scales, ms, ns):
    X = np.asarray(x_rot, dtype=np.float64)
    ms = np.asarray(ms, dtype=np.int64)
    ns = np.asarray(ns, dtype=np.int64)
    W = dequantize(np.asarray(w_bits)[ns], np.asarray(scales)[ns], X.shape[-1])
    return np.einsum("ik,ik->i", np.abs(X[ms]), np.abs(W))


def embedding_rows(w_bits, scales, K, rows) -> np.ndarray:
    """Dequantized rows of a 1-bit table: each entry is +-scale of its group.

    "Inside the One-Bit Engine", station "A token's embedding is 5,120 numbers
    with at most 80 different values": one value per dimension, the group's
    scale with the sign of the bit.
    """
    rows = np.asarray(rows, dtype=np.int64)
    return dequantize(np.asarray(w_bits)[rows], np.asarray(scales)[rows], K)


# ----------------------------------------------------------------------------
# bf16 rounding (the prefill operand is x' rounded to bfloat16)
# ----------------------------------------------------------------------------
def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  bfloat16 keeps fp32's sign and 8-bit
    exponent and the top 7 explicit mantissa bits; the value is first rounded
    to fp32 and then to the bfloat16 grid.  NaN and infinities are not
    expected on this path and are not handled specially.
    """
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lower = u & np.uint64(0xFFFF)
    upper = u >> np.uint64(16)
    half = np.uint64(0x8000)
    round_up = (lower > half) | ((lower == half) & ((upper & np.uint64(1)) == 1))
    upper = upper + round_up.astype(np.uint64)
    return upper.astype(np.uint16)


def bf16_bits_to_float(b: np.ndarray) -> np.ndarray:
    """Exact fp64 value of bfloat16 bit patterns."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# f16 scales (the shipped Q1G128 format stores one 16-bit float per group)
# ----------------------------------------------------------------------------
def round_to_f16(v: np.ndarray) -> np.ndarray:
    """Round values to IEEE binary16, to nearest with ties to even; returns the
    uint16 bit patterns.  numpy's float16 conversion is the library primitive:
    it rounds once, from the exact value, with IEEE overflow to infinity and
    gradual underflow to subnormals."""
    with np.errstate(over="ignore"):  # overflow to infinity is the defined result
        return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_bits_to_float(b: np.ndarray) -> np.ndarray:
    """Exact fp64 value of binary16 bit patterns."""
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def scales_as_f16(scales: np.ndarray) -> np.ndarray:
    """The scales a Q1G128 matrix with f16 scale slots holds (fp64 values)."""
    return f16_bits_to_float(round_to_f16(scales))
