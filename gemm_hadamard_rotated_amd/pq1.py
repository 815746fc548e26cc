"""Thin Python binding of libpq1 (include/pq1.h), same names as the C calls.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libpq1.so.  PyTorch provides device memory and the stream (the
current torch stream of the tensors' device).  There is no CPU fallback:
if the library is missing or the tensors are not on a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PQ1_LIBRARY") or os.path.join(_HERE, "libpq1.so")

PQ1_OK = 0
PQ1_F32, PQ1_BF16, PQ1_BF16_GEMM = 0, 1, 2
PQ1_X_ROW_MAJOR, PQ1_X_GEMM_ORDER = 0, 1
PQ1_GEMV_AUTO, PQ1_GEMV_LUT, PQ1_GEMV_EXPAND = 0, 1, 2
PQ1_GEMV_COUNTER_BYTES = 262144  # split-K bookkeeping at the start of a GEMV workspace
PQ1_GEMV_STATUS_OFFSET = 261888  # the status word inside it
PQ1_SPLITK_WAIT_GAVE_UP, PQ1_SPLITK_OUT_OF_STEP = 1, 2
PQ1_TEST_WITHHOLD_PUBLISH = 1
PQ1_ERR_SPLITK = 9
STATUS_NAMES = {0: "PQ1_OK", 1: "PQ1_ERR_NULL", 2: "PQ1_ERR_SHAPE", 3: "PQ1_ERR_ALIGN",
                4: "PQ1_ERR_PERM", 5: "PQ1_ERR_ALIAS", 6: "PQ1_ERR_DEVICE",
                7: "PQ1_ERR_LAUNCH", 8: "PQ1_ERR_ARG", 9: "PQ1_ERR_SPLITK"}

# every symbol include/pq1.h declares
EXPORTS = ("pq1_rotate", "pq1_gemv_workspace_bytes", "pq1_gemv", "pq1_gemv_ex",
           "pq1_rotate_gemv", "pq1_packed_bits_bytes", "pq1_packed_scales_bytes",
           "pq1_packed_scales_bytes_ex", "pq1_pack_weights", "pq1_pack_weights_rows",
           "pq1_pack_weights_ex", "pq1_embed", "pq1_gemv_packed", "pq1_rotate_gemv_packed",
           "pq1_gemv_packed_ex", "pq1_rotate_gemv_packed_ex", "pq1_gemm", "pq1_gemm_ex",
           "pq1_status_str", "pq1_abi_version", "pq1_last_hip_error", "pq1_set_test_flags",
           "pq1_rotate_gemv_packed_noalloc")


class Pq1Error(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(code, code)} ({msg})")
        self.code = code


class Pq1Perm(ctypes.Structure):
    _fields_ = [("hd", ctypes.c_int32), ("nk", ctypes.c_int32), ("rep", ctypes.c_int32)]


_lib = None
_lib_lock = threading.Lock()


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpq1.so (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m gemm_hadamard_rotated_amd.build`")
        lib = ctypes.CDLL(path)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        PP = ctypes.POINTER(Pq1Perm)
        sig = {
            "pq1_rotate": (I32, [P, P, PP, P, I32, I64, I64, P]),
            "pq1_gemv_workspace_bytes": (SZ, [I64, I64]),
            "pq1_gemv": (I32, [P, P, P, P, I64, I64, P, SZ, P]),
            "pq1_gemv_ex": (I32, [P, P, P, P, I64, I64, I32, P, SZ, P]),
            "pq1_rotate_gemv": (I32, [P, P, PP, P, P, P, I64, I64, P, SZ, P]),
            "pq1_packed_bits_bytes": (SZ, [I64, I64]),
            "pq1_packed_scales_bytes": (SZ, [I64, I64]),
            "pq1_packed_scales_bytes_ex": (SZ, [I64, I64, I32]),
            "pq1_pack_weights": (I32, [P, P, I64, I64, P, P, P]),
            "pq1_pack_weights_rows": (I32, [P, P, I64, I64, P, P, I64, I64, P]),
            "pq1_pack_weights_ex": (I32, [P, P, I64, I64, P, P, I32, I64, I64, P]),
            "pq1_embed": (I32, [P, I64, P, P, P, P, I64, I64, P]),
            "pq1_gemv_packed": (I32, [P, P, P, P, I64, I64, P, SZ, P]),
            "pq1_rotate_gemv_packed": (I32, [P, P, PP, P, P, P, I64, I64, P, SZ, P]),
            "pq1_gemv_packed_ex": (I32, [P, P, P, I32, P, I64, I64, P, SZ, P]),
            "pq1_rotate_gemv_packed_ex": (I32, [P, P, PP, P, P, I32, P, I64, I64, P, SZ, P]),
            "pq1_gemm": (I32, [P, P, P, P, I64, I64, I64, P]),
            "pq1_gemm_ex": (I32, [P, P, P, P, I64, I64, I64, I32, P]),
            "pq1_set_test_flags": (ctypes.c_uint32, [ctypes.c_uint32]),
            "pq1_rotate_gemv_packed_noalloc": (I32, [P, P, PP, P, P, I32, P, I64, I64, P]),
            "pq1_status_str": (ctypes.c_char_p, [I32]),
            "pq1_abi_version": (I32, []),
            "pq1_last_hip_error": (I32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _check(code: int, where: str):
    if code != PQ1_OK:
        lib = load_library()
        raise Pq1Error(code, where, lib.pq1_status_str(code).decode()
                       + f"; hip error {lib.pq1_last_hip_error()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtypes: Sequence[torch.dtype], dev=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (no CPU path exists)")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# The library takes plain pointers and sizes, so it cannot see a tensor that
# is smaller than the sizes say; these checks keep a mismatched tensor from
# reaching a kernel that would read or write past its end.
def _need_numel(t: torch.Tensor, name: str, n: int):
    if t.numel() != n:
        raise ValueError(f"{name} has {t.numel()} elements, expected {n}")


def _need_weights(w_bits: torch.Tensor, scales: torch.Tensor, K: int, what: str) -> int:
    """w_bits [N][K/32] words and scales [N][K/128] for an activation of
    width K; returns N.  (A K the library rejects is left to it.)"""
    if w_bits.dim() != 2:
        raise ValueError(f"{what}: w_bits must be 2-D, [N][K/32] words")
    N = int(w_bits.shape[0])
    if w_bits.shape[1] * 32 != K:
        raise ValueError(f"{what}: w_bits has {w_bits.shape[1]} words per row, "
                         f"an activation of width {K} needs {K / 32:g}")
    if K % 128 == 0:
        _need_numel(scales, "scales", N * (K // 128))
    return N


def _perm(perm):
    if perm is None:
        return None
    hd, nk, rep = (int(v) for v in perm)
    return ctypes.byref(Pq1Perm(hd, nk, rep))


_WORD_DTYPES = (torch.int32, torch.uint32)

# ----------------------------------------------------------------------------
# GEMV workspace, one per (device, stream), grown on demand.  A new workspace
# is zero-filled; every call leaves its counter region in a state the next call
# accepts, so calls of any shapes ordered on the stream can share it
# (include/pq1.h).
# ----------------------------------------------------------------------------
_ws = {}
_ws_retired = []  # replaced workspaces, kept alive for graphs that captured them
_ws_lock = threading.Lock()


def check_gemv_workspace(device: Optional[torch.device] = None) -> None:
    """Raise Pq1Error(PQ1_ERR_SPLITK) if a packed-layout GEMV on the current
    stream's workspace reported trouble in the workspace's status word since
    the last check (a split-K wait that gave up, or bookkeeping found out of
    step; the affected outputs are NaN).  Waits for the stream.  On an error
    the counter region is zero-filled, so the next call starts in step."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    with _ws_lock:
        ws = _ws.get(key)
    if ws is None:
        return
    word = ws[PQ1_GEMV_STATUS_OFFSET:PQ1_GEMV_STATUS_OFFSET + 4].view(torch.int32)
    status = int(word.item())
    if status:
        ws[:PQ1_GEMV_COUNTER_BYTES].zero_()
        parts = []
        if status & PQ1_SPLITK_WAIT_GAVE_UP:
            parts.append("a split-K wait gave up")
        if status & PQ1_SPLITK_OUT_OF_STEP:
            parts.append("split-K bookkeeping was out of step")
        raise Pq1Error(PQ1_ERR_SPLITK, "GEMV workspace",
                       " and ".join(parts) + "; the affected outputs are NaN")


def pq1_set_test_flags(flags: int) -> int:
    """Failure-handling tests only (include/pq1.h); returns the previous flags."""
    return int(load_library().pq1_set_test_flags(int(flags)))


def gemv_workspace(N: int, K: int, device: torch.device) -> torch.Tensor:
    lib = load_library()
    need = int(lib.pq1_gemv_workspace_bytes(int(N), int(K)))
    if need == 0:
        raise Pq1Error(2, "pq1_gemv_workspace_bytes", "invalid shape")
    stream = torch.cuda.current_stream(device).cuda_stream
    key = (device.index, stream)
    with _ws_lock:
        ws = _ws.get(key)
        if ws is None or ws.numel() < need:
            if ws is not None:
                # a graph captured earlier may still hold the old buffer's address
                _ws_retired.append(ws)
            ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=device)
            _ws[key] = ws
        return ws


# ----------------------------------------------------------------------------
# Calls
# ----------------------------------------------------------------------------
def pq1_rotate(x: torch.Tensor, signs: torch.Tensor, perm=None,
               out_dtype: torch.dtype = torch.float32,
               out: Optional[torch.Tensor] = None, gemm_order: bool = False) -> torch.Tensor:
    """x_rot = WHT_1024(signs * P x) / 32 per row of x ([K] or [M][K] fp32).

    With out_dtype=torch.bfloat16 and gemm_order=True the result is stored in
    the K order of pq1_gemm's operand (PQ1_BF16_GEMM)."""
    _need(x, "x", (torch.float32,))
    dev = x.device
    _need(signs, "signs", (torch.float32,), dev)
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    _need_numel(signs, "signs", K)
    code = {torch.float32: PQ1_F32, torch.bfloat16: PQ1_BF16}.get(out_dtype)
    if code is None:
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    if gemm_order:
        if code != PQ1_BF16:
            raise ValueError("gemm_order needs out_dtype=torch.bfloat16")
        code = PQ1_BF16_GEMM
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype, device=dev)
    else:
        _need(out, "out", (out_dtype,), dev)
        if out.shape != x.shape:
            raise ValueError("out must have the shape of x")
    lib = load_library()
    with torch.cuda.device(dev):
        _check(lib.pq1_rotate(_ptr(x), _ptr(signs), _perm(perm), _ptr(out), code, M, K,
                              _stream(dev)), "pq1_rotate")
    return out


def pq1_gemv_ex(x_rot: torch.Tensor, w_bits: torch.Tensor, scales: torch.Tensor,
                algo: int = PQ1_GEMV_AUTO, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = W x_rot for one [K] fp32 activation; W from packed bits and scales."""
    _need(x_rot, "x_rot", (torch.float32,))
    dev = x_rot.device
    _need(w_bits, "w_bits", _WORD_DTYPES, dev)
    _need(scales, "scales", (torch.float32,), dev)
    K = x_rot.numel()
    N = _need_weights(w_bits, scales, K, "pq1_gemv_ex")
    if out is None:
        out = torch.empty(N, dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), dev)
        _need_numel(out, "out", N)
    lib = load_library()
    with torch.cuda.device(dev):
        ws = gemv_workspace(N, K, dev) if K >= 128 and K % 128 == 0 and N >= 1 else None
        _check(lib.pq1_gemv_ex(_ptr(x_rot), _ptr(w_bits), _ptr(scales), _ptr(out), N, K,
                               int(algo), _ptr(ws), 0 if ws is None else ws.numel(),
                               _stream(dev)), "pq1_gemv_ex")
    return out


def pq1_gemv(x_rot, w_bits, scales, out=None) -> torch.Tensor:
    return pq1_gemv_ex(x_rot, w_bits, scales, PQ1_GEMV_AUTO, out)


def pq1_rotate_gemv(x: torch.Tensor, signs: torch.Tensor, w_bits: torch.Tensor,
                    scales: torch.Tensor, perm=None,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = W WHT_1024(signs * P x) / 32 in one launch, for one [K] activation."""
    _need(x, "x", (torch.float32,))
    dev = x.device
    _need(signs, "signs", (torch.float32,), dev)
    _need(w_bits, "w_bits", _WORD_DTYPES, dev)
    _need(scales, "scales", (torch.float32,), dev)
    K = x.numel()
    N = _need_weights(w_bits, scales, K, "pq1_rotate_gemv")
    _need_numel(signs, "signs", K)
    if out is None:
        out = torch.empty(N, dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), dev)
        _need_numel(out, "out", N)
    lib = load_library()
    with torch.cuda.device(dev):
        ws = gemv_workspace(N, K, dev) if K >= 128 and K % 128 == 0 and N >= 1 else None
        _check(lib.pq1_rotate_gemv(_ptr(x), _ptr(signs), _perm(perm), _ptr(w_bits),
                                   _ptr(scales), _ptr(out), N, K, _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(dev)),
               "pq1_rotate_gemv")
    return out


# pq1_scale_dtype: storage type of the packed scales
SCALE_DTYPES = {"f32": 0, "f16": 1}
_SCALE_TORCH = {"f32": torch.float32, "f16": torch.float16}


def _scale_code(scale_dtype: str) -> int:
    if scale_dtype not in SCALE_DTYPES:
        raise Pq1Error(8, "scale_dtype", f"unknown scale dtype {scale_dtype!r} (f32 or f16)")
    return SCALE_DTYPES[scale_dtype]


class PackedWeights:
    """Band-interleaved copy of a 1-bit weight matrix (see pq1_pack_weights);
    scale_dtype is the storage type of its scales ("f32" or "f16")."""

    def __init__(self, bits: torch.Tensor, scales: torch.Tensor, N: int, K: int,
                 scale_dtype: str = "f32"):
        self.bits, self.scales, self.N, self.K = bits, scales, int(N), int(K)
        self.scale_dtype = scale_dtype

    @property
    def device(self):
        return self.bits.device


def _need_packed(pw: PackedWeights, dev):
    """The packed arrays are on `dev` and as large as the library says a
    packed matrix of pw.N x pw.K is."""
    if not isinstance(pw, PackedWeights):
        raise TypeError("pw must be a PackedWeights (pq1_pack_weights)")
    lib = load_library()
    nb = int(lib.pq1_packed_bits_bytes(pw.N, pw.K))
    ns = int(lib.pq1_packed_scales_bytes_ex(pw.N, pw.K, _scale_code(pw.scale_dtype)))
    for t, name, need in ((pw.bits, "packed bits", nb), (pw.scales, "packed scales", ns)):
        if t.device != dev:
            raise ValueError(f"{name} are on {t.device}, expected {dev}")
        if not t.is_contiguous() or t.numel() * t.element_size() < need:
            raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, need {need}")


def _alloc_packed(N: int, K: int, scale_dtype: str, dev, what: str) -> PackedWeights:
    lib = load_library()
    nb = int(lib.pq1_packed_bits_bytes(N, K))
    ns = int(lib.pq1_packed_scales_bytes_ex(N, K, _scale_code(scale_dtype)))
    if nb == 0 or ns == 0:
        raise Pq1Error(2, what, "invalid shape")
    dt = _SCALE_TORCH[scale_dtype]
    pbits = torch.empty(nb // 4, dtype=torch.int32, device=dev)
    pscales = torch.empty(ns // dt.itemsize, dtype=dt, device=dev)
    return PackedWeights(pbits, pscales, N, K, scale_dtype)


def _check_parts(parts, dev, what):
    if not parts:
        raise Pq1Error(2, what, "no matrices")
    KW = parts[0][0].shape[1]
    for w_bits, scales in parts:
        _need(w_bits, "w_bits", _WORD_DTYPES, dev)
        _need(scales, "scales", (torch.float32,), dev)
        if w_bits.dim() != 2 or w_bits.shape[1] != KW:
            raise Pq1Error(2, what, "all matrices must have the same K")
        _need_weights(w_bits, scales, KW * 32, what)
    return KW * 32, sum(w.shape[0] for w, _ in parts)


def pq1_pack_weights(w_bits: torch.Tensor, scales: torch.Tensor,
                     scale_dtype: str = "f32") -> PackedWeights:
    """Repack [N][K/32] words + [N][K/128] scales into the packed layout
    (scales stored as fp32, or rounded to f16 through pq1_pack_weights_ex)."""
    if scale_dtype != "f32":
        return pq1_pack_weights_ex(w_bits, scales, scale_dtype)
    _need(w_bits, "w_bits", _WORD_DTYPES)
    dev = w_bits.device
    _need(scales, "scales", (torch.float32,), dev)
    N, KW = w_bits.shape
    K = KW * 32
    _need_weights(w_bits, scales, K, "pq1_pack_weights")
    pw = _alloc_packed(N, K, "f32", dev, "pq1_pack_weights")
    lib = load_library()
    with torch.cuda.device(dev):
        _check(lib.pq1_pack_weights(_ptr(w_bits), _ptr(scales), N, K, _ptr(pw.bits),
                                    _ptr(pw.scales), _stream(dev)), "pq1_pack_weights")
    return pw


def pq1_pack_weights_ex(w_bits: torch.Tensor, scales: torch.Tensor, scale_dtype: str = "f16",
                        into: Optional[PackedWeights] = None, row0: int = 0) -> PackedWeights:
    """Repack one matrix with the given scale storage.  Without `into` a new
    packed matrix of N rows is made; with it, the rows go to rows row0 ..
    row0+N-1 of `into` (same K and scale_dtype), which is returned."""
    _need(w_bits, "w_bits", _WORD_DTYPES)
    dev = w_bits.device
    _need(scales, "scales", (torch.float32,), dev)
    code = _scale_code(scale_dtype)
    N, KW = w_bits.shape
    K = KW * 32
    _need_weights(w_bits, scales, K, "pq1_pack_weights_ex")
    if into is None:
        into = _alloc_packed(N, K, scale_dtype, dev, "pq1_pack_weights_ex")
        row0 = 0
    elif into.K != K or into.scale_dtype != scale_dtype or into.device != dev:
        raise Pq1Error(2, "pq1_pack_weights_ex", "target has another K, scale dtype or device")
    lib = load_library()
    with torch.cuda.device(dev):
        _check(lib.pq1_pack_weights_ex(_ptr(w_bits), _ptr(scales), N, K, _ptr(into.bits),
                                       _ptr(into.scales), code, into.N, row0, _stream(dev)),
               "pq1_pack_weights_ex")
    return into


def pq1_pack_weights_rows(parts, dev=None, scale_dtype: str = "f32") -> PackedWeights:
    """Pack several matrices with the same K, given as [(w_bits, scales), ...],
    one after another into one packed matrix (pq1_pack_weights_rows per part,
    or pq1_pack_weights_ex for f16 scales): one GEMV launch then yields their
    outputs one after another."""
    parts = list(parts)
    dev = parts[0][0].device if (dev is None and parts) else dev
    K, n_total = _check_parts(parts, dev, "pq1_pack_weights_rows")
    pw = _alloc_packed(n_total, K, scale_dtype, dev, "pq1_pack_weights_rows")
    lib = load_library()
    row0 = 0
    with torch.cuda.device(dev):
        for w_bits, scales in parts:
            n = w_bits.shape[0]
            if scale_dtype == "f32":
                _check(lib.pq1_pack_weights_rows(_ptr(w_bits), _ptr(scales), n, K, _ptr(pw.bits),
                                                 _ptr(pw.scales), n_total, row0, _stream(dev)),
                       "pq1_pack_weights_rows")
            else:
                pq1_pack_weights_ex(w_bits, scales, scale_dtype, into=pw, row0=row0)
            row0 += n
    return pw


def pq1_embed(tokens: torch.Tensor, w_bits: torch.Tensor, scales: torch.Tensor,
              signs: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rows tokens[m] of a 1-bit table, with the inverse rotation:
    out[m] = signs * WHT_1024(dequantized row) / 32 (fp32 [M][K])."""
    _need(tokens, "tokens", (torch.int32,))
    dev = tokens.device
    _need(w_bits, "w_bits", _WORD_DTYPES, dev)
    _need(scales, "scales", (torch.float32,), dev)
    _need(signs, "signs", (torch.float32,), dev)
    V, KW = w_bits.shape
    K = KW * 32
    M = tokens.numel()
    _need_weights(w_bits, scales, K, "pq1_embed")
    _need_numel(signs, "signs", K)
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), dev)
        _need_numel(out, "out", M * K)
    lib = load_library()
    with torch.cuda.device(dev):
        _check(lib.pq1_embed(_ptr(tokens), M, _ptr(w_bits), _ptr(scales), _ptr(signs), _ptr(out),
                             V, K, _stream(dev)), "pq1_embed")
    return out


def pq1_gemv_packed(x_rot: torch.Tensor, pw: PackedWeights,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = W x_rot with W given as PackedWeights (f16 scales: pq1_gemv_packed_ex)."""
    if pw.scale_dtype != "f32":
        return pq1_gemv_packed_ex(x_rot, pw, out)
    _need(x_rot, "x_rot", (torch.float32,))
    dev = x_rot.device
    _need_packed(pw, dev)
    _need_numel(x_rot, "x_rot", pw.K)
    if out is None:
        out = torch.empty(pw.N, dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), dev)
        _need_numel(out, "out", pw.N)
    lib = load_library()
    with torch.cuda.device(dev):
        ws = gemv_workspace(pw.N, pw.K, dev)
        _check(lib.pq1_gemv_packed(_ptr(x_rot), _ptr(pw.bits), _ptr(pw.scales), _ptr(out),
                                   pw.N, x_rot.numel(), _ptr(ws), ws.numel(), _stream(dev)),
               "pq1_gemv_packed")
    return out


def pq1_rotate_gemv_packed(x: torch.Tensor, signs: torch.Tensor, pw: PackedWeights, perm=None,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = W WHT_1024(signs * P x) / 32 in one launch, W given as PackedWeights
    (f16 scales: pq1_rotate_gemv_packed_ex)."""
    if pw.scale_dtype != "f32":
        return pq1_rotate_gemv_packed_ex(x, signs, pw, perm, out)
    _need(x, "x", (torch.float32,))
    dev = x.device
    _need(signs, "signs", (torch.float32,), dev)
    _need_packed(pw, dev)
    _need_numel(x, "x", pw.K)
    _need_numel(signs, "signs", pw.K)
    if out is None:
        out = torch.empty(pw.N, dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), dev)
        _need_numel(out, "out", pw.N)
    lib = load_library()
    with torch.cuda.device(dev):
        ws = gemv_workspace(pw.N, pw.K, dev)
        _check(lib.pq1_rotate_gemv_packed(_ptr(x), _ptr(signs), _perm(perm), _ptr(pw.bits),
                                          _ptr(pw.scales), _ptr(out), pw.N, x.numel(), _ptr(ws),
                                          ws.numel(), _stream(dev)), "pq1_rotate_gemv_packed")
    return out


def pq1_gemv_packed_ex(x_rot: torch.Tensor, pw: PackedWeights,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """pq1_gemv_packed for packed weights of either scale storage type."""
    _need(x_rot, "x_rot", (torch.float32,))
    dev = x_rot.device
    _need_packed(pw, dev)
    _need_numel(x_rot, "x_rot", pw.K)
    if out is None:
        out = torch.empty(pw.N, dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), dev)
        _need_numel(out, "out", pw.N)
    lib = load_library()
    with torch.cuda.device(dev):
        ws = gemv_workspace(pw.N, pw.K, dev)
        _check(lib.pq1_gemv_packed_ex(_ptr(x_rot), _ptr(pw.bits), _ptr(pw.scales),
                                      _scale_code(pw.scale_dtype), _ptr(out), pw.N, x_rot.numel(),
                                      _ptr(ws), ws.numel(), _stream(dev)), "pq1_gemv_packed_ex")
    return out


def pq1_rotate_gemv_packed_ex(x: torch.Tensor, signs: torch.Tensor, pw: PackedWeights, perm=None,
                              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """pq1_rotate_gemv_packed for packed weights of either scale storage type."""
    _need(x, "x", (torch.float32,))
    dev = x.device
    _need(signs, "signs", (torch.float32,), dev)
    _need_packed(pw, dev)
    _need_numel(x, "x", pw.K)
    _need_numel(signs, "signs", pw.K)
    if out is None:
        out = torch.empty(pw.N, dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), dev)
        _need_numel(out, "out", pw.N)
    lib = load_library()
    with torch.cuda.device(dev):
        ws = gemv_workspace(pw.N, pw.K, dev)
        _check(lib.pq1_rotate_gemv_packed_ex(_ptr(x), _ptr(signs), _perm(perm), _ptr(pw.bits),
                                             _ptr(pw.scales), _scale_code(pw.scale_dtype),
                                             _ptr(out), pw.N, x.numel(), _ptr(ws), ws.numel(),
                                             _stream(dev)), "pq1_rotate_gemv_packed_ex")
    return out


def pq1_rotate_gemv_packed_noalloc(x: torch.Tensor, signs: torch.Tensor, pw: PackedWeights,
                                   perm=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """pq1_rotate_gemv_packed_ex with the library's own counter region: no
    workspace.  With `out` given the call allocates nothing (include/pq1.h)."""
    _need(x, "x", (torch.float32,))
    dev = x.device
    _need(signs, "signs", (torch.float32,), dev)
    _need_packed(pw, dev)
    _need_numel(x, "x", pw.K)
    _need_numel(signs, "signs", pw.K)
    if out is None:
        out = torch.empty(pw.N, dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), dev)
        _need_numel(out, "out", pw.N)
    lib = load_library()
    with torch.cuda.device(dev):
        _check(lib.pq1_rotate_gemv_packed_noalloc(_ptr(x), _ptr(signs), _perm(perm), _ptr(pw.bits),
                                                  _ptr(pw.scales), _scale_code(pw.scale_dtype),
                                                  _ptr(out), pw.N, x.numel(), _stream(dev)),
               "pq1_rotate_gemv_packed_noalloc")
    return out


def pq1_gemm_ex(x_rot_bf16: torch.Tensor, w_bits: torch.Tensor, scales: torch.Tensor,
                out: Optional[torch.Tensor] = None, gemm_order: bool = False) -> torch.Tensor:
    """Y = X W^T for a [M][K] bf16 activation block; fp32 [M][N] result.

    gemm_order=True: X is in the GEMM K order (pq1_rotate(..., gemm_order=True),
    x_layout PQ1_X_GEMM_ORDER); else row-major (PQ1_X_ROW_MAJOR)."""
    _need(x_rot_bf16, "x_rot_bf16", (torch.bfloat16, torch.int16, torch.uint16))
    dev = x_rot_bf16.device
    _need(w_bits, "w_bits", _WORD_DTYPES, dev)
    _need(scales, "scales", (torch.float32,), dev)
    if x_rot_bf16.dim() != 2:
        raise ValueError("x_rot_bf16 must be 2-D, [M][K]")
    M, K = x_rot_bf16.shape
    N = _need_weights(w_bits, scales, K, "pq1_gemm")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), dev)
        _need_numel(out, "out", M * N)
    lib = load_library()
    with torch.cuda.device(dev):
        if gemm_order:
            code = lib.pq1_gemm_ex(_ptr(x_rot_bf16), _ptr(w_bits), _ptr(scales), _ptr(out), M, N,
                                   K, PQ1_X_GEMM_ORDER, _stream(dev))
        else:
            code = lib.pq1_gemm(_ptr(x_rot_bf16), _ptr(w_bits), _ptr(scales), _ptr(out), M, N, K,
                                _stream(dev))
        _check(code, "pq1_gemm_ex" if gemm_order else "pq1_gemm")
    return out


def pq1_gemm(x_rot_bf16: torch.Tensor, w_bits: torch.Tensor, scales: torch.Tensor,
             out: Optional[torch.Tensor] = None, gemm_order: bool = False) -> torch.Tensor:
    """Y = X W^T for a row-major [M][K] bf16 activation block (pq1_gemm);
    gemm_order=True forwards to pq1_gemm_ex with X in the GEMM K order."""
    return pq1_gemm_ex(x_rot_bf16, w_bits, scales, out, gemm_order)


def pq1_status_str(code: int) -> str:
    return load_library().pq1_status_str(int(code)).decode()


def pq1_abi_version() -> int:
    return int(load_library().pq1_abi_version())


def pq1_gemv_workspace_bytes(N: int, K: int) -> int:
    return int(load_library().pq1_gemv_workspace_bytes(int(N), int(K)))
