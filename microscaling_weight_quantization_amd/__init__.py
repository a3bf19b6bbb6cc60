"""Python binding of the gfx950 block-scaled weight-quantization library (libmxq.so).

The ``mxq_*`` functions carry the names of the C entry points in
``include/mxq.h`` and only marshal arguments: tensors become device pointers,
row strides and sizes, and the call is enqueued on torch's current stream.
Every step of the computation runs in the HIP kernels of ``csrc/mxq.hip``;
there is no fallback of any kind, and a missing library raises.

PyTorch is used for device memory and streams only.  A [rows, K] operand is a
tensor whose last dimension is contiguous; leading dimensions of a contiguous
tensor are flattened into rows.

Sources (page title, section): "[PyTorch] MXFP4 weight QAT on MXFP8 and FP8
block-scaling recipes" -- Description, Test results, Known limitations; and
"MXFP8TensorStorage.export_components()" -- Description.
"""
from __future__ import annotations

import ctypes
import functools
import os
import threading
from typing import NamedTuple, Optional

import torch

from . import build as _build

MXQ_BF16, MXQ_FP32, MXQ_FP16 = 0, 1, 2
MXQ_E4M3, MXQ_E5M2 = 0, 1
MXQ_SCALE_ROW_1X32, MXQ_SCALE_TILE_128X128, MXQ_SCALE_COL_32X1 = 0, 1, 2
MXQ_OK, MXQ_ERR_NULL, MXQ_ERR_SHAPE, MXQ_ERR_DTYPE, MXQ_ERR_NO_ROWWISE_DATA, MXQ_ERR_ALIAS, MXQ_ERR_HIP = range(7)

ENTRY_POINTS = ("mxq_status_string", "mxq_fake_quantize_mxfp4", "mxq_mxfp4_to_mxfp8_row",
                "mxq_mxfp4_to_fp8_block128", "mxq_export_mxfp8", "mxq_dequantize",
                "mxq_fake_quantize_mxfp4_with_mxfp8_row", "mxq_mxfp4_to_mxfp8_row_guarded",
                "mxq_mxfp4_to_fp8_block128_guarded", "mxq_quantize_mxfp4", "mxq_dequantize_mxfp4",
                "mxq_mxfp4_packed_to_mxfp8_row", "mxq_mxfp4_packed_to_fp8_block128", "mxq_mxfp4_to_mxfp8_col",
                "mxq_mxfp4_to_mxfp8_row_col", "mxq_mxfp4_to_mxfp8_col_guarded", "mxq_mxfp4_to_mxfp8_row_col_guarded",
                "mxq_mxfp4_to_mxfp8_row_grouped", "mxq_fake_quantize_mxfp4_grouped",
                "mxq_mxfp4_to_fp8_block128_grouped", "mxq_dequantize_grouped", "mxq_quantize_mxfp4_grouped")

_libs = {}
_lock = threading.Lock()


class _RowGroup(ctypes.Structure):
    """mxq_row_group of include/mxq.h."""
    _fields_ = [("x", ctypes.c_void_p), ("ld_x", ctypes.c_int64), ("rows", ctypes.c_int64), ("K", ctypes.c_int64),
                ("data", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("scale_ld", ctypes.c_int64)]


class _ProjGroup(ctypes.Structure):
    """mxq_proj_group of include/mxq.h."""
    _fields_ = [("x", ctypes.c_void_p), ("ld_x", ctypes.c_int64), ("y", ctypes.c_void_p), ("ld_y", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("K", ctypes.c_int64)]


class _Block128Group(ctypes.Structure):
    """mxq_block128_group of include/mxq.h."""
    _fields_ = [("x", ctypes.c_void_p), ("ld_x", ctypes.c_int64), ("rows", ctypes.c_int64), ("K", ctypes.c_int64),
                ("data", ctypes.c_void_p), ("tile_code", ctypes.c_void_p), ("tile_ld", ctypes.c_int64)]


class _DequantGroup(ctypes.Structure):
    """mxq_dequant_group of include/mxq.h."""
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("scale_ld", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("K", ctypes.c_int64), ("out", ctypes.c_void_p), ("ld_out", ctypes.c_int64)]


class _Mxfp4Group(ctypes.Structure):
    """mxq_mxfp4_group of include/mxq.h."""
    _fields_ = [("x", ctypes.c_void_p), ("ld_x", ctypes.c_int64), ("rows", ctypes.c_int64), ("K", ctypes.c_int64),
                ("packed", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("scale_ld", ctypes.c_int64)]


class MxqError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"mxq status {status}: {text}")
        self.status = status


def load(name: str = "libmxq.so") -> ctypes.CDLL:
    """Load a built variant of the library (build it first: ``__graft_entry__.build()``)."""
    with _lock:
        if name in _libs:
            return _libs[name]
        path = _build.library_path(name)
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} is not built; run __graft_entry__.build() "
                                    "(python -m microscaling_weight_quantization_amd.build)")
        L = ctypes.CDLL(path)
        i64, vp, i32, u8p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
        L.mxq_status_string.argtypes = [i32]
        L.mxq_status_string.restype = ctypes.c_char_p
        L.mxq_fake_quantize_mxfp4.argtypes = [vp, i64, vp, i64, i64, i64, i32, vp]
        L.mxq_mxfp4_to_mxfp8_row.argtypes = [vp, i64, i64, i64, i32, u8p, u8p, i64, vp]
        L.mxq_mxfp4_to_fp8_block128.argtypes = [vp, i64, i64, i64, i32, u8p, u8p, i64, vp]
        L.mxq_export_mxfp8.argtypes = [u8p, u8p, i64, i64, i64, u8p, vp]
        L.mxq_dequantize.argtypes = [u8p, u8p, i64, i64, i64, i32, i32, vp, i64, i32, vp]
        L.mxq_fake_quantize_mxfp4_with_mxfp8_row.argtypes = [vp, i64, vp, i64, i64, i64, i32, u8p, u8p, i64, vp]
        L.mxq_mxfp4_to_mxfp8_row_guarded.argtypes = [vp, i64, i64, i64, i32, u8p, u8p, i64, vp, vp]
        L.mxq_mxfp4_to_fp8_block128_guarded.argtypes = [vp, i64, i64, i64, i32, u8p, u8p, i64, vp, vp]
        L.mxq_quantize_mxfp4.argtypes = [vp, i64, i64, i64, i32, u8p, u8p, i64, vp]
        L.mxq_dequantize_mxfp4.argtypes = [u8p, u8p, i64, i64, i64, vp, i64, i32, vp]
        L.mxq_mxfp4_packed_to_mxfp8_row.argtypes = [u8p, u8p, i64, i64, i64, u8p, u8p, i64, vp]
        L.mxq_mxfp4_packed_to_fp8_block128.argtypes = [u8p, u8p, i64, i64, i64, u8p, u8p, i64, vp]
        L.mxq_mxfp4_to_mxfp8_col.argtypes = [vp, i64, i64, i64, i32, u8p, u8p, i64, vp]
        L.mxq_mxfp4_to_mxfp8_row_col.argtypes = [vp, i64, i64, i64, i32, u8p, u8p, i64, u8p, u8p, i64, vp]
        L.mxq_mxfp4_to_mxfp8_col_guarded.argtypes = [vp, i64, i64, i64, i32, u8p, u8p, i64, vp, vp]
        L.mxq_mxfp4_to_mxfp8_row_col_guarded.argtypes = [vp, i64, i64, i64, i32, u8p, u8p, i64, u8p, u8p, i64, vp, vp]
        L.mxq_mxfp4_to_mxfp8_row_grouped.argtypes = [ctypes.POINTER(_RowGroup), i64, i32, vp]
        L.mxq_fake_quantize_mxfp4_grouped.argtypes = [ctypes.POINTER(_ProjGroup), i64, i32, vp]
        L.mxq_mxfp4_to_fp8_block128_grouped.argtypes = [ctypes.POINTER(_Block128Group), i64, i32, vp]
        L.mxq_dequantize_grouped.argtypes = [ctypes.POINTER(_DequantGroup), i64, i32, i32, i32, vp]
        L.mxq_quantize_mxfp4_grouped.argtypes = [ctypes.POINTER(_Mxfp4Group), i64, i32, vp]
        for n in ENTRY_POINTS[1:]:
            getattr(L, n).restype = i32
        _libs[name] = L
        return L


def _device_operands(fn):
    """Every tensor argument of an entry point must be a device tensor, all on one
    device: the library takes raw device pointers, and a host pointer or one
    from another GPU would reach a kernel as an invalid address."""
    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        dev = -2                                            # get_device(): -1 for a host tensor
        for t in (*args, *kwargs.values()):
            if isinstance(t, torch.Tensor):
                d = t.get_device()
                if d < 0 or not t.is_cuda:
                    raise ValueError(f"{fn.__name__}: operands must be device tensors, got one on {t.device}")
                if dev == -2:
                    dev = d
                elif d != dev:
                    raise ValueError(f"{fn.__name__}: operands on cuda:{dev} and cuda:{d}; all must be on one device")
        return fn(*args, **kwargs)
    return wrapper


def _check(L, rc: int):
    if rc != MXQ_OK:
        raise MxqError(rc, L.mxq_status_string(rc).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MXQ_BF16
    if t.dtype == torch.float32:
        return MXQ_FP32
    if t.dtype == torch.float16:
        return MXQ_FP16
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or fp32 expected")


def _matrix(t: torch.Tensor):
    """(pointer, rows, K, row stride in elements) of a tensor with a contiguous last dim."""
    if t.dim() == 0:
        raise ValueError("a matrix needs at least one dimension")
    if t.dim() == 1:
        t = t.view(1, -1)
    if t.dim() > 2:
        if not t.is_contiguous():
            raise ValueError("leading dimensions can only be flattened for a contiguous tensor")
        t = t.view(-1, t.shape[-1])
    rows, K = t.shape
    if K > 1 and t.stride(1) != 1:
        raise ValueError("the last dimension must be contiguous")
    ld = t.stride(0) if rows > 1 else K
    return t.data_ptr(), rows, K, ld


def _operand(t: torch.Tensor, rows: int, cols: int, what: str, contiguous: bool = False, byte: bool = False):
    """(pointer, row stride) of an operand the call reads or writes as a
    [rows, cols] matrix.  Raises ValueError, before anything is launched, when
    the tensor is smaller than that region (the C entry points only see a
    pointer and a stride, so a short buffer would be accessed out of bounds),
    when `contiguous` is set and its rows are not packed (payloads have row
    stride cols), or when `byte` is set and its elements are not bytes."""
    if byte and t.element_size() != 1:
        raise ValueError(f"{what} holds bytes (uint8), got {t.dtype}")
    p, trows, tcols, ld = _matrix(t)
    if rows * cols == 0:
        return p, max(ld, cols)
    if trows < rows or tcols < cols:
        raise ValueError(f"{what} must cover [{rows}, {cols}], got [{trows}, {tcols}]")
    if contiguous and ld != cols:
        raise ValueError(f"{what} must be a contiguous [{rows}, {cols}] tensor (row stride {cols}), got row stride {ld}")
    return p, ld


def _flag(t: torch.Tensor) -> int:
    if t.dtype != torch.int32 or not t.is_cuda or t.numel() < 1:
        raise ValueError("the no-op flag is a device int32 tensor")
    return t.data_ptr()


# torch's current stream as a raw handle.  The internal accessor returns the
# handle directly (a tenth of the time of building a Stream object); the public
# call is the fallback where a torch build lacks it.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor):
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(t.get_device()))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


# ---- the C entry points, one to one ---------------------------------------------------

def _nb(K: int) -> int:
    return (K + 31) // 32


def _scale_for(x: torch.Tensor, rows: int, cols: int, ld: Optional[int]) -> torch.Tensor:
    """A zeroed code array [rows, ld or cols] on x's device (padding stays 0)."""
    return torch.zeros((rows, ld or cols), dtype=torch.uint8, device=x.device)


def _payload_for(x: torch.Tensor, rows: int, K: int, data: Optional[torch.Tensor], what: str = "payload"):
    if data is None:
        data = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    pd, _ = _operand(data, rows, K, what, contiguous=True, byte=True)
    return data, pd


@_device_operands
def mxq_fake_quantize_mxfp4(x: torch.Tensor, y: Optional[torch.Tensor] = None, lib: str = "libmxq.so") -> torch.Tensor:
    """MXFP4 projection of x (bf16 / fp32) into y (same dtype; y may be x)."""
    L = load(lib)
    dt = _dtype_code(x)
    if y is None:
        y = torch.empty_like(x, memory_format=torch.contiguous_format)
    if y.dtype != x.dtype or y.shape != x.shape:
        raise ValueError("y must have x's dtype and shape")
    px, rows, K, ldx = _matrix(x)
    py, ldy = _operand(y, rows, K, "y")
    _check(L, L.mxq_fake_quantize_mxfp4(px, ldx, py, ldy, rows, K, dt, _stream(x)))
    return y


@_device_operands
def mxq_mxfp4_to_mxfp8_row(x: torch.Tensor, data: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None,
                           scale_ld: Optional[int] = None, lib: str = "libmxq.so",
                           noop: Optional[torch.Tensor] = None):
    """Direct MXFP8 rowwise lift -> (payload uint8 [rows, K], E8M0 codes uint8 [rows, scale_ld]).
    With `noop` (an int32 device tensor) this is mxq_mxfp4_to_mxfp8_row_guarded."""
    L = load(lib)
    dt = _dtype_code(x)
    px, rows, K, ldx = _matrix(x)
    scale = _scale_for(x, rows, _nb(K), scale_ld) if scale is None else scale
    data, pd = _payload_for(x, rows, K, data)
    ps, ld_s = _operand(scale, rows, _nb(K), "scale", byte=True)
    if noop is None:
        _check(L, L.mxq_mxfp4_to_mxfp8_row(px, ldx, rows, K, dt, pd, ps, ld_s, _stream(x)))
    else:
        _check(L, L.mxq_mxfp4_to_mxfp8_row_guarded(px, ldx, rows, K, dt, pd, ps, ld_s, _flag(noop), _stream(x)))
    return data, scale


@_device_operands
def mxq_mxfp4_to_fp8_block128(x: torch.Tensor, data: Optional[torch.Tensor] = None,
                              tile_code: Optional[torch.Tensor] = None, lib: str = "libmxq.so",
                              noop: Optional[torch.Tensor] = None):
    """Direct 128x128 blockwise FP8 -> (payload uint8 [rows, K], tile codes uint8 [ceil(rows/128), tile_ld]).
    With `noop` (an int32 device tensor) this is mxq_mxfp4_to_fp8_block128_guarded."""
    L = load(lib)
    dt = _dtype_code(x)
    px, rows, K, ldx = _matrix(x)
    ntr, ntc = (rows + 127) // 128, (K + 127) // 128
    tile_code = _scale_for(x, ntr, ntc, None) if tile_code is None else tile_code
    data, pd = _payload_for(x, rows, K, data)
    pt, ldt = _operand(tile_code, ntr, ntc, "tile_code", byte=True)
    if noop is None:
        _check(L, L.mxq_mxfp4_to_fp8_block128(px, ldx, rows, K, dt, pd, pt, ldt, _stream(x)))
    else:
        _check(L, L.mxq_mxfp4_to_fp8_block128_guarded(px, ldx, rows, K, dt, pd, pt, ldt, _flag(noop), _stream(x)))
    return data, tile_code


@_device_operands
def mxq_mxfp4_to_mxfp8_col(x: torch.Tensor, data: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None,
                           scale_ld: Optional[int] = None, lib: str = "libmxq.so",
                           noop: Optional[torch.Tensor] = None):
    """MXFP8 columnwise (32x1 blocks) from the decomposition ->
    (payload uint8 [rows, K], E8M0 codes uint8 [ceil(rows/32), scale_ld]).
    With `noop` (an int32 device tensor) this is mxq_mxfp4_to_mxfp8_col_guarded."""
    L = load(lib)
    dt = _dtype_code(x)
    px, rows, K, ldx = _matrix(x)
    bands = (rows + 31) // 32
    scale = _scale_for(x, bands, K, scale_ld) if scale is None else scale
    data, pd = _payload_for(x, rows, K, data)
    ps, ld_s = _operand(scale, bands, K, "scale", byte=True)
    if noop is None:
        _check(L, L.mxq_mxfp4_to_mxfp8_col(px, ldx, rows, K, dt, pd, ps, ld_s, _stream(x)))
    else:
        _check(L, L.mxq_mxfp4_to_mxfp8_col_guarded(px, ldx, rows, K, dt, pd, ps, ld_s, _flag(noop), _stream(x)))
    return data, scale


@_device_operands
def mxq_mxfp4_to_mxfp8_row_col(x: torch.Tensor, row_data: Optional[torch.Tensor] = None,
                               row_scale: Optional[torch.Tensor] = None, col_data: Optional[torch.Tensor] = None,
                               col_scale: Optional[torch.Tensor] = None, row_scale_ld: Optional[int] = None,
                               col_scale_ld: Optional[int] = None, lib: str = "libmxq.so",
                               noop: Optional[torch.Tensor] = None):
    """Row lift and columnwise conversion from one read of x ->
    (row payload, row codes [rows, row_scale_ld], column payload, column codes [ceil(rows/32), col_scale_ld]).
    With `noop` (an int32 device tensor) this is mxq_mxfp4_to_mxfp8_row_col_guarded."""
    L = load(lib)
    dt = _dtype_code(x)
    px, rows, K, ldx = _matrix(x)
    bands = (rows + 31) // 32
    row_scale = _scale_for(x, rows, _nb(K), row_scale_ld) if row_scale is None else row_scale
    col_scale = _scale_for(x, bands, K, col_scale_ld) if col_scale is None else col_scale
    row_data, prd = _payload_for(x, rows, K, row_data, "row payload")
    col_data, pcd = _payload_for(x, rows, K, col_data, "column payload")
    prs, ld_rs = _operand(row_scale, rows, _nb(K), "row_scale", byte=True)
    pcs, ld_cs = _operand(col_scale, bands, K, "col_scale", byte=True)
    if noop is None:
        _check(L, L.mxq_mxfp4_to_mxfp8_row_col(px, ldx, rows, K, dt, prd, prs, ld_rs, pcd, pcs, ld_cs, _stream(x)))
    else:
        _check(L, L.mxq_mxfp4_to_mxfp8_row_col_guarded(px, ldx, rows, K, dt, prd, prs, ld_rs, pcd, pcs, ld_cs,
                                                       _flag(noop), _stream(x)))
    return row_data, row_scale, col_data, col_scale


@_device_operands
def mxq_fake_quantize_mxfp4_with_mxfp8_row(x: torch.Tensor, y: Optional[torch.Tensor] = None,
                                           data: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None,
                                           scale_ld: Optional[int] = None, lib: str = "libmxq.so"):
    """Projection and row lift from one read of x -> (y, payload, codes)."""
    L = load(lib)
    dt = _dtype_code(x)
    px, rows, K, ldx = _matrix(x)
    if y is None:
        y = torch.empty_like(x, memory_format=torch.contiguous_format)
    if y.dtype != x.dtype or y.shape != x.shape:
        raise ValueError("y must have x's dtype and shape")
    scale = _scale_for(x, rows, _nb(K), scale_ld) if scale is None else scale
    py, ldy = _operand(y, rows, K, "y")
    data, pd = _payload_for(x, rows, K, data)
    ps, ld_s = _operand(scale, rows, _nb(K), "scale", byte=True)
    _check(L, L.mxq_fake_quantize_mxfp4_with_mxfp8_row(px, ldx, py, ldy, rows, K, dt, pd, ps, ld_s, _stream(x)))
    return y, data, scale


@_device_operands
def mxq_export_mxfp8(data: Optional[torch.Tensor], scale_storage: Optional[torch.Tensor], K: int,
                     scale_out: Optional[torch.Tensor] = None, lib: str = "libmxq.so") -> torch.Tensor:
    """Compact [rows, ceil(K/32)] copy of padded E8M0 scale storage (rows, scale_ld)."""
    L = load(lib)
    if data is None or scale_storage is None:
        rc = L.mxq_export_mxfp8(None, None, 0, K, 0, None, None)
        _check(L, rc)
    ps, rows, _, ld_s = _matrix(scale_storage)
    nb = _nb(K)
    if scale_out is None:
        scale_out = torch.empty((rows, nb), dtype=torch.uint8, device=scale_storage.device)
    _operand(scale_storage, rows, nb, "scale_storage", byte=True)
    po, _ = _operand(scale_out, rows, nb, "scale_out", contiguous=True, byte=True)
    _check(L, L.mxq_export_mxfp8(data.data_ptr(), ps, rows, K, ld_s, po, _stream(scale_storage)))
    return scale_out


_SCALE_GRID = {MXQ_SCALE_ROW_1X32: lambda rows, K: (rows, _nb(K)),
               MXQ_SCALE_TILE_128X128: lambda rows, K: ((rows + 127) // 128, (K + 127) // 128),
               MXQ_SCALE_COL_32X1: lambda rows, K: ((rows + 31) // 32, K)}


@_device_operands
def mxq_dequantize(data: torch.Tensor, scale: torch.Tensor, layout: int = MXQ_SCALE_ROW_1X32, fmt: int = MXQ_E4M3,
                   out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                   lib: str = "libmxq.so") -> torch.Tensor:
    """Decode FP8 payload bytes with E8M0 codes into bf16 / fp32."""
    L = load(lib)
    _, rows, K, _ = _matrix(data)
    pd, _ = _operand(data, rows, K, "payload", contiguous=True, byte=True)
    if out is None:
        out = torch.empty((rows, K), dtype=out_dtype, device=data.device)
    srows, scols = _SCALE_GRID[layout](rows, K) if layout in _SCALE_GRID else (0, 0)   # the C call rejects others
    ps, lds = _operand(scale, srows, scols, "scale", byte=True)
    po, ldo = _operand(out, rows, K, "out")
    _check(L, L.mxq_dequantize(pd, ps, lds, rows, K, fmt, layout, po, ldo, _dtype_code(out), _stream(data)))
    return out


@_device_operands
def mxq_quantize_mxfp4(x: torch.Tensor, packed: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None,
                       scale_ld: Optional[int] = None, lib: str = "libmxq.so"):
    """Packed MXFP4 (deployment format) -> (nibble pairs uint8 [rows, ceil(K/2)], E8M0 codes)."""
    L = load(lib)
    dt = _dtype_code(x)
    px, rows, K, ldx = _matrix(x)
    pw = (K + 1) // 2
    if packed is None:
        packed = torch.empty((rows, pw), dtype=torch.uint8, device=x.device)
    scale = _scale_for(x, rows, _nb(K), scale_ld) if scale is None else scale
    pp, _ = _operand(packed, rows, pw, "packed", contiguous=True, byte=True)
    ps, ld_s = _operand(scale, rows, _nb(K), "scale", byte=True)
    _check(L, L.mxq_quantize_mxfp4(px, ldx, rows, K, dt, pp, ps, ld_s, _stream(x)))
    return packed, scale


def _packed_args(packed: torch.Tensor, scale: torch.Tensor, K: int):
    _, rows, _, _ = _matrix(packed)
    pp, _ = _operand(packed, rows, (K + 1) // 2, "packed", contiguous=True, byte=True)
    ps, ld_s = _operand(scale, rows, _nb(K), "scale", byte=True)
    return pp, ps, ld_s, rows


@_device_operands
def mxq_dequantize_mxfp4(packed: torch.Tensor, scale: torch.Tensor, K: int, out: Optional[torch.Tensor] = None,
                         out_dtype: torch.dtype = torch.bfloat16, lib: str = "libmxq.so") -> torch.Tensor:
    """Decode packed MXFP4 into bf16 / fp32 [rows, K]."""
    L = load(lib)
    pp, ps, ld_s, rows = _packed_args(packed, scale, K)
    if out is None:
        out = torch.empty((rows, K), dtype=out_dtype, device=packed.device)
    po, ldo = _operand(out, rows, K, "out")
    _check(L, L.mxq_dequantize_mxfp4(pp, ps, ld_s, rows, K, po, ldo, _dtype_code(out), _stream(packed)))
    return out


@_device_operands
def mxq_mxfp4_packed_to_mxfp8_row(packed: torch.Tensor, scale: torch.Tensor, K: int,
                                  data: Optional[torch.Tensor] = None, scale_out: Optional[torch.Tensor] = None,
                                  lib: str = "libmxq.so"):
    """Direct MXFP8 row lift from packed MXFP4 -> (payload uint8 [rows, K], codes)."""
    L = load(lib)
    pp, ps, ld_s, rows = _packed_args(packed, scale, K)
    data, pd = _payload_for(packed, rows, K, data)
    scale_out = _scale_for(packed, rows, _nb(K), None) if scale_out is None else scale_out
    po, ldo = _operand(scale_out, rows, _nb(K), "scale_out", byte=True)
    _check(L, L.mxq_mxfp4_packed_to_mxfp8_row(pp, ps, ld_s, rows, K, pd, po, ldo, _stream(packed)))
    return data, scale_out


@_device_operands
def mxq_mxfp4_packed_to_fp8_block128(packed: torch.Tensor, scale: torch.Tensor, K: int,
                                     data: Optional[torch.Tensor] = None, tile_code: Optional[torch.Tensor] = None,
                                     lib: str = "libmxq.so"):
    """Direct 128x128 blockwise FP8 from packed MXFP4 -> (payload uint8 [rows, K], tile codes)."""
    L = load(lib)
    pp, ps, ld_s, rows = _packed_args(packed, scale, K)
    ntr, ntc = (rows + 127) // 128, (K + 127) // 128
    data, pd = _payload_for(packed, rows, K, data)
    tile_code = _scale_for(packed, ntr, ntc, None) if tile_code is None else tile_code
    pt, ldt = _operand(tile_code, ntr, ntc, "tile_code", byte=True)
    _check(L, L.mxq_mxfp4_packed_to_fp8_block128(pp, ps, ld_s, rows, K, pd, pt, ldt, _stream(packed)))
    return data, tile_code


# ---- grouped calls ------------------------------------------------------------------------

class _Grouped:
    """A grouped entry point prepared once for a fixed list of weights and
    outputs: the descriptor table is built (and every operand checked) here,
    and each call enqueues the whole list on torch's current stream with one
    call into the library, for weights re-converted every training step.  The
    object keeps the tensors alive.

    Subclasses name the C function and its descriptor struct, the list
    arguments (the first is the per-weight input that sets rows and K),
    `_describe`, which fills in missing outputs for weight i, checks its
    operands and returns its descriptor, and `_extra_args`, the call's
    arguments between the table and the stream."""
    _fn: str
    _struct: type
    _lists: tuple

    def __init__(self, lists, lib: str):
        self._L = load(lib)
        lists = [list(l) if l is not None else None for l in lists]
        self.n = n = len(lists[0])
        lists = [[None] * n if l is None else l for l in lists]
        if any(len(l) != n for l in lists):
            raise ValueError(f"{self._fn}: {', '.join(self._lists[1:])} must have one entry per weight")
        self._tensors = lists
        self._first = None
        if n == 0:
            return
        for l in lists:
            for t in l:
                if t is not None and not (isinstance(t, torch.Tensor) and t.is_cuda):
                    raise ValueError(f"{self._fn}: operands must be device tensors on one device")
        dev = lists[0][0].device
        if any(t is not None and t.device != dev for l in lists for t in l):
            raise ValueError(f"{self._fn}: operands must be device tensors on one device")
        self._first = lists[0][0]
        self._table = (self._struct * n)(*[self._describe(i, dev) for i in range(n)])
        self._extra = self._extra_args()

    def _describe(self, i: int, dev):
        raise NotImplementedError

    def _extra_args(self):
        return (self._same_dtype(self._tensors[0], "weights"),)

    def _same_dtype(self, ts, what: str) -> int:
        if any(t.dtype != ts[0].dtype for t in ts):
            raise ValueError(f"all {what} of a group call must have one dtype")
        return _dtype_code(ts[0])

    def __call__(self):
        if self.n:
            _check(self._L, getattr(self._L, self._fn)(self._table, self.n, *self._extra, _stream(self._first)))
        return self._outputs()


class GroupedRowLift(_Grouped):
    """The grouped row lift (mxq_mxfp4_to_mxfp8_row_grouped); `datas` / `scales` are the outputs."""
    _fn, _struct, _lists = "mxq_mxfp4_to_mxfp8_row_grouped", _RowGroup, ("xs", "datas", "scales")

    def __init__(self, xs, datas=None, scales=None, scale_ld: Optional[int] = None, lib: str = "libmxq.so"):
        self._scale_ld = scale_ld
        super().__init__((xs, datas, scales), lib)

    def _describe(self, i, dev):
        xs, datas, scales = self._tensors
        px, rows, K, ldx = _matrix(xs[i])
        if scales[i] is None:
            scales[i] = _scale_for(xs[i], rows, _nb(K), self._scale_ld)
        datas[i], pd = _payload_for(xs[i], rows, K, datas[i])
        ps, ld_s = _operand(scales[i], rows, _nb(K), "scale", byte=True)
        return _RowGroup(px, ldx, rows, K, pd, ps, ld_s)

    def _outputs(self):
        return self._tensors[1], self._tensors[2]

    xs = property(lambda self: self._tensors[0])
    datas = property(lambda self: self._tensors[1])
    scales = property(lambda self: self._tensors[2])


class GroupedProjection(_Grouped):
    """The grouped MXFP4 projection (mxq_fake_quantize_mxfp4_grouped); an
    output may be its weight itself (in place); `ys` are the outputs."""
    _fn, _struct, _lists = "mxq_fake_quantize_mxfp4_grouped", _ProjGroup, ("xs", "ys")

    def __init__(self, xs, ys=None, lib: str = "libmxq.so"):
        super().__init__((xs, ys), lib)

    def _describe(self, i, dev):
        xs, ys = self._tensors
        if ys[i] is None:
            ys[i] = torch.empty_like(xs[i], memory_format=torch.contiguous_format)
        if ys[i].dtype != xs[i].dtype or ys[i].shape != xs[i].shape:
            raise ValueError("each output must have its weight's dtype and shape")
        px, rows, K, ldx = _matrix(xs[i])
        py, ldy = _operand(ys[i], rows, K, "y")
        return _ProjGroup(px, ldx, py, ldy, rows, K)

    def _outputs(self):
        return self._tensors[1]

    xs = property(lambda self: self._tensors[0])
    ys = property(lambda self: self._tensors[1])


class GroupedBlock128(_Grouped):
    """The grouped 128x128 fold (mxq_mxfp4_to_fp8_block128_grouped); `datas` / `tile_codes` are the outputs."""
    _fn, _struct, _lists = "mxq_mxfp4_to_fp8_block128_grouped", _Block128Group, ("xs", "datas", "tile_codes")

    def __init__(self, xs, datas=None, tile_codes=None, lib: str = "libmxq.so"):
        super().__init__((xs, datas, tile_codes), lib)

    def _describe(self, i, dev):
        xs, datas, tcs = self._tensors
        px, rows, K, ldx = _matrix(xs[i])
        ntr, ntc = (rows + 127) // 128, (K + 127) // 128
        if tcs[i] is None:
            tcs[i] = _scale_for(xs[i], ntr, ntc, None)
        datas[i], pd = _payload_for(xs[i], rows, K, datas[i])
        pt, ldt = _operand(tcs[i], ntr, ntc, "tile_code", byte=True)
        return _Block128Group(px, ldx, rows, K, pd, pt, ldt)

    def _outputs(self):
        return self._tensors[1], self._tensors[2]

    xs = property(lambda self: self._tensors[0])
    datas = property(lambda self: self._tensors[1])
    tile_codes = property(lambda self: self._tensors[2])


class GroupedDequantize(_Grouped):
    """The grouped decode (mxq_dequantize_grouped) of payloads with one format,
    scale layout and output dtype; `outs` are the outputs."""
    _fn, _struct, _lists = "mxq_dequantize_grouped", _DequantGroup, ("datas", "scales", "outs")

    def __init__(self, datas, scales, layout: int = MXQ_SCALE_ROW_1X32, fmt: int = MXQ_E4M3, outs=None,
                 out_dtype: torch.dtype = torch.bfloat16, lib: str = "libmxq.so"):
        self._layout, self._fmt, self._out_dtype = layout, fmt, out_dtype
        super().__init__((datas, scales, outs), lib)

    def _extra_args(self):
        return (self._fmt, self._layout, self._same_dtype(self._tensors[2], "outputs"))

    def _describe(self, i, dev):
        datas, scales, outs = self._tensors
        _, rows, K, _ = _matrix(datas[i])
        if outs[i] is None:
            outs[i] = torch.empty(tuple(datas[i].shape), dtype=self._out_dtype, device=dev)
        pd, _ = _operand(datas[i], rows, K, "payload", contiguous=True, byte=True)
        srows, scols = _SCALE_GRID[self._layout](rows, K) if self._layout in _SCALE_GRID else (0, 0)
        ps, lds = _operand(scales[i], srows, scols, "scale", byte=True)
        po, ldo = _operand(outs[i], rows, K, "out")
        return _DequantGroup(pd, ps, lds, rows, K, po, ldo)

    def _outputs(self):
        return self._tensors[2]

    datas = property(lambda self: self._tensors[0])
    outs = property(lambda self: self._tensors[2])


class GroupedQuantizeMxfp4(_Grouped):
    """The grouped packed MXFP4 encode (mxq_quantize_mxfp4_grouped); `packeds` / `scales` are the outputs."""
    _fn, _struct, _lists = "mxq_quantize_mxfp4_grouped", _Mxfp4Group, ("xs", "packeds", "scales")

    def __init__(self, xs, packeds=None, scales=None, scale_ld: Optional[int] = None, lib: str = "libmxq.so"):
        self._scale_ld = scale_ld
        super().__init__((xs, packeds, scales), lib)

    def _describe(self, i, dev):
        xs, packeds, scales = self._tensors
        px, rows, K, ldx = _matrix(xs[i])
        pw = (K + 1) // 2
        if packeds[i] is None:
            packeds[i] = torch.empty((rows, pw), dtype=torch.uint8, device=dev)
        if scales[i] is None:
            scales[i] = _scale_for(xs[i], rows, _nb(K), self._scale_ld)
        pp, _ = _operand(packeds[i], rows, pw, "packed", contiguous=True, byte=True)
        ps, ld_s = _operand(scales[i], rows, _nb(K), "scale", byte=True)
        return _Mxfp4Group(px, ldx, rows, K, pp, ps, ld_s)

    def _outputs(self):
        return self._tensors[1], self._tensors[2]

    xs = property(lambda self: self._tensors[0])
    packeds = property(lambda self: self._tensors[1])
    scales = property(lambda self: self._tensors[2])


@_device_operands
def mxq_mxfp4_to_mxfp8_row_grouped(xs, datas=None, scales=None, scale_ld: Optional[int] = None,
                                   lib: str = "libmxq.so"):
    """Direct MXFP8 rowwise lift of a list of weights of one dtype, in as few
    launches as possible -> (list of payloads, list of E8M0 codes); the same
    bytes as one mxq_mxfp4_to_mxfp8_row per weight.  `datas` / `scales`: lists
    of outputs (None entries, or None for the whole list, are allocated)."""
    return GroupedRowLift(xs, datas, scales, scale_ld, lib)()


@_device_operands
def mxq_fake_quantize_mxfp4_grouped(xs, ys=None, lib: str = "libmxq.so"):
    """MXFP4 projection of a list of weights of one dtype, in as few launches as
    possible -> list of outputs; the same bits as one mxq_fake_quantize_mxfp4 per
    weight (an entry of `ys` may be its weight, in place)."""
    return GroupedProjection(xs, ys, lib)()


@_device_operands
def mxq_mxfp4_to_fp8_block128_grouped(xs, datas=None, tile_codes=None, lib: str = "libmxq.so"):
    """Direct 128x128 blockwise FP8 of a list of weights of one dtype, in as few
    launches as possible -> (list of payloads, list of tile codes)."""
    return GroupedBlock128(xs, datas, tile_codes, lib)()


@_device_operands
def mxq_dequantize_grouped(datas, scales, layout: int = MXQ_SCALE_ROW_1X32, fmt: int = MXQ_E4M3, outs=None,
                           out_dtype: torch.dtype = torch.bfloat16, lib: str = "libmxq.so"):
    """Decode a list of FP8 payloads with their E8M0 codes (one format, scale
    layout and output dtype), in as few launches as possible -> list of outputs."""
    return GroupedDequantize(datas, scales, layout, fmt, outs, out_dtype, lib)()


@_device_operands
def mxq_quantize_mxfp4_grouped(xs, packeds=None, scales=None, scale_ld: Optional[int] = None,
                               lib: str = "libmxq.so"):
    """Packed MXFP4 (deployment format) of a list of weights of one dtype, in as
    few launches as possible -> (list of nibble pairs, list of E8M0 codes)."""
    return GroupedQuantizeMxfp4(xs, packeds, scales, scale_ld, lib)()


# ---- convenience layer ------------------------------------------------------------------

class MXFP8Components(NamedTuple):
    """FP8 values and unpadded E8M0 scales of an MXFP8 rowwise tensor."""
    data: torch.Tensor        # payload viewed as float8 with the tensor's shape
    scale_inv: torch.Tensor   # uint8 E8M0 codes, shape (*shape[:-1], ceil(K/32))


def export_components(data: Optional[torch.Tensor], scale_storage: Optional[torch.Tensor], shape,
                      fp8_dtype: torch.dtype = torch.float8_e4m3fn, lib: str = "libmxq.so") -> MXFP8Components:
    """Export values and scales in a storage-independent layout.  The values are
    always a view of `data`; the scales are a view when the storage has exactly
    ceil(K/32) columns and a copy (made by the library's kernel) when it is
    padded.  Missing row-scaled data raises ValueError."""
    if data is None or scale_storage is None:
        raise ValueError("tensor has no row-scaled data to export")
    shape = tuple(shape)
    K = shape[-1]
    nb = (K + 31) // 32
    values = data.view(fp8_dtype).view(shape)
    scale2d = scale_storage.view(-1, scale_storage.shape[-1]) if scale_storage.dim() != 2 else scale_storage
    if scale2d.shape[1] == nb:
        scale_inv = scale2d
    else:
        scale_inv = mxq_export_mxfp8(data, scale2d, K, lib=lib)
    return MXFP8Components(values, scale_inv.view(*shape[:-1], nb))


def fake_quantize_mxfp4(t: torch.Tensor, lib: str = "libmxq.so") -> torch.Tensor:
    if t.dtype == torch.float16:
        raise TypeError("fp16 is not supported: the MXFP4 grid exceeds fp16's range")
    return mxq_fake_quantize_mxfp4(t, lib=lib)
