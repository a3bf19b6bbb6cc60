"""CPU oracle for the MXFP4 -> MXFP8 / 128x128 FP8 weight-quantization path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product imports this package: only the
test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
load it.  It wraps ``mxq_oracle.c`` (plain C, exact integer arithmetic on dyadic
rationals) through ctypes and numpy, and shares no code with the HIP library.

Functions work on numpy arrays of raw bits: bf16 as uint16, fp32 as uint32,
FP8 payloads and E8M0 codes as uint8.  Row ranges can be spread over threads;
ctypes drops the GIL for the duration of each C call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxq_oracle.c")
_LIB = os.path.join(_HERE, "libmxq_oracle.so")

BF16, FP32 = 0, 1
E4M3, E5M2 = 0, 1
ROW_1X32, TILE_128X128, COL_32X1 = 0, 1, 2

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (host only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB)
            i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
            L.orc_fake_quantize_mxfp4.argtypes = [vp, i64, vp, i64, i64, i64, i32, i64, i64]
            L.orc_mxfp4_to_mxfp8_row.argtypes = [vp, i64, i64, i64, i32, vp, vp, i64, i64, i64]
            L.orc_mxfp4_to_fp8_block128.argtypes = [vp, i64, i64, i64, i32, vp, vp, i64, i64, i64]
            L.orc_mxfp4_to_mxfp8_col.argtypes = [vp, i64, i64, i64, i32, vp, vp, i64, i64, i64]
            L.orc_export_mxfp8.argtypes = [vp, i64, i64, i64, vp]
            L.orc_dequantize.argtypes = [vp, vp, i64, i64, i64, i32, i32, vp, i64, i32, i64, i64]
            L.orc_quantize_mxfp4.argtypes = [vp, i64, i64, i64, i32, vp, vp, i64, i64, i64]
            L.orc_dequantize_mxfp4.argtypes = [vp, vp, i64, i64, i64, vp, i64, i32, i64, i64]
            L.orc_mxfp4_packed_to_mxfp8_row.argtypes = [vp, vp, i64, i64, i64, vp, vp, i64, i64, i64]
            L.orc_mxfp4_packed_to_fp8_block128.argtypes = [vp, vp, i64, i64, i64, vp, vp, i64, i64, i64]
            for name in ("orc_quantize_mxfp4", "orc_dequantize_mxfp4", "orc_mxfp4_packed_to_mxfp8_row",
                         "orc_mxfp4_packed_to_fp8_block128"):
                getattr(L, name).restype = ctypes.c_int
            L.orc_scale_exponent_bits.argtypes = [ctypes.c_uint32, i32]
            L.orc_e2m1_code_bits.argtypes = [ctypes.c_uint32, i32, i32]
            L.orc_round_to_format.argtypes = [i32, ctypes.c_uint64, i32, i32, ctypes.POINTER(i32)]
            L.orc_round_to_format.restype = ctypes.c_uint32
            L.orc_unpack.argtypes = [ctypes.c_uint32, i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_uint64),
                                     ctypes.POINTER(i32), ctypes.POINTER(i32)]
            for name in ("orc_fake_quantize_mxfp4", "orc_mxfp4_to_mxfp8_row", "orc_mxfp4_to_fp8_block128",
                         "orc_mxfp4_to_mxfp8_col", "orc_export_mxfp8", "orc_dequantize", "orc_scale_exponent_bits", "orc_e2m1_code_bits"):
                getattr(L, name).restype = ctypes.c_int
            _lib = L
    return _lib


def _dtype_of(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.uint32:
        return FP32
    raise TypeError("oracle inputs are raw bits: uint16 for bf16, uint32 for fp32")


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _bands(rows: int, threads: int, align: int = 1):
    """Split [0, rows) into up to `threads` bands whose starts are multiples of align."""
    units = (rows + align - 1) // align
    threads = max(1, min(threads, units))
    out, start = [], 0
    for t in range(threads):
        n = units // threads + (1 if t < units % threads else 0)
        end = min(rows, (start // align + n) * align)
        if end > start:
            out.append((start, end))
        start = end
    return out


def _run(fn, rows: int, threads: int, align: int = 1):
    bands = _bands(rows, threads, align)
    if len(bands) <= 1:
        for r0, r1 in bands:
            rc = fn(r0, r1)
            if rc:
                raise ValueError(f"oracle rejected its arguments (status {rc})")
        return
    with ThreadPoolExecutor(len(bands)) as ex:
        for rc in ex.map(lambda b: fn(*b), bands):
            if rc:
                raise ValueError(f"oracle rejected its arguments (status {rc})")


def _as2d(x: np.ndarray) -> np.ndarray:
    if x.ndim == 1:
        x = x.reshape(1, -1)
    if x.ndim != 2 or (x.shape[1] > 1 and x.strides[1] != x.itemsize):
        raise ValueError("expected a 2-D array with a contiguous last dimension")
    if x.shape[0] > 1 and (x.strides[0] % x.itemsize or x.strides[0] // x.itemsize < x.shape[1]):
        raise ValueError("rows must not overlap")
    return x


def _ld(x: np.ndarray) -> int:
    """Row stride in elements (a single row has none: use its length)."""
    return x.strides[0] // x.itemsize if x.shape[0] > 1 else x.shape[1]


def fake_quantize_mxfp4(x: np.ndarray, threads: int = 1) -> np.ndarray:
    """MXFP4 projection of a [rows, K] bf16/fp32 bit array; same dtype out."""
    x = _as2d(x)
    rows, K = x.shape
    ld = _ld(x)
    y = np.empty((rows, K), dtype=x.dtype)
    L = lib()
    _run(lambda r0, r1: L.orc_fake_quantize_mxfp4(_ptr(x), ld, _ptr(y), K, rows, K, _dtype_of(x), r0, r1), rows, threads)
    return y


def mxfp4_to_mxfp8_row(x: np.ndarray, scale_ld: int | None = None, threads: int = 1, fill: int = 0):
    """Direct MXFP8 rowwise lift: (payload uint8 [rows, K], scale uint8 [rows, scale_ld]).
    Padding columns keep `fill` (the oracle never writes them)."""
    x = _as2d(x)
    rows, K = x.shape
    ld = _ld(x)
    nb = (K + 31) // 32
    scale_ld = nb if scale_ld is None else scale_ld
    data = np.empty((rows, K), dtype=np.uint8)
    scale = np.full((rows, scale_ld), fill, dtype=np.uint8)
    L = lib()
    _run(lambda r0, r1: L.orc_mxfp4_to_mxfp8_row(_ptr(x), ld, rows, K, _dtype_of(x), _ptr(data), _ptr(scale),
                                                 scale_ld, r0, r1), rows, threads)
    return data, scale


def mxfp4_to_fp8_block128(x: np.ndarray, tile_ld: int | None = None, threads: int = 1):
    """Direct 128x128 blockwise FP8: (payload uint8 [rows, K], tile codes uint8 [ceil(rows/128), tile_ld])."""
    x = _as2d(x)
    rows, K = x.shape
    ld = _ld(x)
    ntc = (K + 127) // 128
    tile_ld = ntc if tile_ld is None else tile_ld
    data = np.empty((rows, K), dtype=np.uint8)
    codes = np.zeros(((rows + 127) // 128, tile_ld), dtype=np.uint8)
    L = lib()
    _run(lambda r0, r1: L.orc_mxfp4_to_fp8_block128(_ptr(x), ld, rows, K, _dtype_of(x), _ptr(data), _ptr(codes),
                                                    tile_ld, r0, r1), rows, threads, align=128)
    return data, codes


def mxfp4_to_mxfp8_col(x: np.ndarray, scale_ld: int | None = None, threads: int = 1, fill: int = 0):
    """MXFP8 columnwise (32x1 blocks) from the decomposition: (payload uint8 [rows, K],
    codes uint8 [ceil(rows/32), scale_ld]).  Padding columns keep `fill`."""
    x = _as2d(x)
    rows, K = x.shape
    ld = _ld(x)
    scale_ld = K if scale_ld is None else scale_ld
    data = np.empty((rows, K), dtype=np.uint8)
    scale = np.full(((rows + 31) // 32, scale_ld), fill, dtype=np.uint8)
    L = lib()
    _run(lambda r0, r1: L.orc_mxfp4_to_mxfp8_col(_ptr(x), ld, rows, K, _dtype_of(x), _ptr(data), _ptr(scale),
                                                 scale_ld, r0, r1), rows, threads, align=32)
    return data, scale


def export_mxfp8(scale_storage: np.ndarray, K: int) -> np.ndarray:
    """Unpadded E8M0 scales (rows, ceil(K/32)) from padded storage (rows, scale_ld)."""
    s = _as2d(np.ascontiguousarray(scale_storage, dtype=np.uint8))
    rows, scale_ld = s.shape
    out = np.empty((rows, (K + 31) // 32), dtype=np.uint8)
    rc = lib().orc_export_mxfp8(_ptr(s), rows, K, scale_ld, _ptr(out))
    if rc:
        raise ValueError(f"oracle rejected its arguments (status {rc})")
    return out


def dequantize(data: np.ndarray, scale: np.ndarray, layout: int = ROW_1X32, fp8: int = E4M3,
               out_dtype: int = BF16, threads: int = 1) -> np.ndarray:
    """Decode FP8 payload bytes with E8M0 codes to bf16 (uint16) or fp32 (uint32) bits."""
    data = _as2d(np.ascontiguousarray(data, dtype=np.uint8))
    scale = _as2d(np.ascontiguousarray(scale, dtype=np.uint8))
    rows, K = data.shape
    out = np.empty((rows, K), dtype=np.uint16 if out_dtype == BF16 else np.uint32)
    L = lib()
    _run(lambda r0, r1: L.orc_dequantize(_ptr(data), _ptr(scale), scale.shape[1], rows, K, fp8, layout, _ptr(out), K,
                                         out_dtype, r0, r1), rows, threads)
    return out


# ---- packed MXFP4 (deployment format) --------------------------------------------------

def quantize_mxfp4(x: np.ndarray, scale_ld: int | None = None, threads: int = 1, fill: int = 0):
    """Packed MXFP4: (nibble pairs uint8 [rows, ceil(K/2)], E8M0 codes uint8 [rows, scale_ld])."""
    x = _as2d(x)
    rows, K = x.shape
    ld = _ld(x)
    nb = (K + 31) // 32
    scale_ld = nb if scale_ld is None else scale_ld
    packed = np.empty((rows, (K + 1) // 2), dtype=np.uint8)
    scale = np.full((rows, scale_ld), fill, dtype=np.uint8)
    L = lib()
    _run(lambda r0, r1: L.orc_quantize_mxfp4(_ptr(x), ld, rows, K, _dtype_of(x), _ptr(packed), _ptr(scale), scale_ld,
                                             r0, r1), rows, threads)
    return packed, scale


def dequantize_mxfp4(packed: np.ndarray, scale: np.ndarray, K: int, out_dtype: int = BF16, threads: int = 1):
    packed = _as2d(np.ascontiguousarray(packed, dtype=np.uint8))
    scale = _as2d(np.ascontiguousarray(scale, dtype=np.uint8))
    rows = packed.shape[0]
    out = np.empty((rows, K), dtype=np.uint16 if out_dtype == BF16 else np.uint32)
    L = lib()
    _run(lambda r0, r1: L.orc_dequantize_mxfp4(_ptr(packed), _ptr(scale), scale.shape[1], rows, K, _ptr(out), K,
                                               out_dtype, r0, r1), rows, threads)
    return out


def mxfp4_packed_to_mxfp8_row(packed: np.ndarray, scale: np.ndarray, K: int, scale_out_ld: int | None = None,
                              threads: int = 1, fill: int = 0):
    packed = _as2d(np.ascontiguousarray(packed, dtype=np.uint8))
    scale = _as2d(np.ascontiguousarray(scale, dtype=np.uint8))
    rows = packed.shape[0]
    nb = (K + 31) // 32
    scale_out_ld = nb if scale_out_ld is None else scale_out_ld
    data = np.empty((rows, K), dtype=np.uint8)
    scale_out = np.full((rows, scale_out_ld), fill, dtype=np.uint8)
    L = lib()
    _run(lambda r0, r1: L.orc_mxfp4_packed_to_mxfp8_row(_ptr(packed), _ptr(scale), scale.shape[1], rows, K,
                                                        _ptr(data), _ptr(scale_out), scale_out_ld, r0, r1),
         rows, threads)
    return data, scale_out


def mxfp4_packed_to_fp8_block128(packed: np.ndarray, scale: np.ndarray, K: int, threads: int = 1):
    packed = _as2d(np.ascontiguousarray(packed, dtype=np.uint8))
    scale = _as2d(np.ascontiguousarray(scale, dtype=np.uint8))
    rows = packed.shape[0]
    data = np.empty((rows, K), dtype=np.uint8)
    codes = np.zeros(((rows + 127) // 128, (K + 127) // 128), dtype=np.uint8)
    L = lib()
    _run(lambda r0, r1: L.orc_mxfp4_packed_to_fp8_block128(_ptr(packed), _ptr(scale), scale.shape[1], rows, K,
                                                           _ptr(data), _ptr(codes), codes.shape[1], r0, r1),
         rows, threads, align=128)
    return data, codes


# ---- element-level helpers for the pins ------------------------------------------------

def scale_exponent_bits(amax_bits: int, dtype: int = BF16) -> int:
    return lib().orc_scale_exponent_bits(amax_bits, dtype)


def e2m1_code_bits(x_bits: int, e: int, dtype: int = BF16) -> int:
    return lib().orc_e2m1_code_bits(x_bits, dtype, e)


FMT_BF16, FMT_FP32, FMT_E4M3, FMT_E5M2 = 0, 1, 2, 3


def round_to_format(neg: int, M: int, k: int, fmt: int):
    """(bits, inexact, overflow) of nearest-even rounding of (-1)^neg * M * 2^k."""
    flags = ctypes.c_int(0)
    bits = lib().orc_round_to_format(neg, M, k, fmt, ctypes.byref(flags))
    return bits, bool(flags.value & 1), bool(flags.value & 2)


def unpack(bits: int, fmt: int):
    """(neg, M, k, cls) with value (-1)^neg * M * 2^k; cls 0 finite, 1 inf, 2 nan."""
    neg, k, cls = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    M = ctypes.c_uint64()
    lib().orc_unpack(bits, fmt, ctypes.byref(neg), ctypes.byref(M), ctypes.byref(k), ctypes.byref(cls))
    return neg.value, M.value, k.value, cls.value
