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
        dev = None
        for t in list(args) + list(kwargs.values()):
            if isinstance(t, torch.Tensor):
                if not t.is_cuda:
                    raise ValueError(f"{fn.__name__}: operands must be device tensors, got one on {t.device}")
                if dev is None:
                    dev = t.device
                elif t.device != dev:
                    raise ValueError(f"{fn.__name__}: operands on {dev} and {t.device}; all must be on one device")
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


def _flag(t: torch.Tensor) -> int:
    if t.dtype != torch.int32 or not t.is_cuda or t.numel() < 1:
        raise ValueError("the no-op flag is a device int32 tensor")
    return t.data_ptr()


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


# ---- the C entry points, one to one ---------------------------------------------------

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
    py, _, _, ldy = _matrix(y)
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
    nb = (K + 31) // 32
    if scale is None:
        scale = torch.zeros((rows, scale_ld or nb), dtype=torch.uint8, device=x.device)
    if data is None:
        data = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    pd, _, _, ldd = _matrix(data)
    ps, _, sld, ld_s = _matrix(scale)
    if rows * K and (ldd != K or data.numel() != rows * K):
        raise ValueError("payload must be a contiguous [rows, K] uint8 tensor")
    if noop is None:
        _check(L, L.mxq_mxfp4_to_mxfp8_row(px, ldx, rows, K, dt, pd, ps, ld_s, _stream(x)))
    else:
        _check(L, L.mxq_mxfp4_to_mxfp8_row_guarded(px, ldx, rows, K, dt, pd, ps, ld_s, _flag(noop), _stream(x)))
    return data, scale


class GroupedRowLift:
    """The grouped row lift prepared once for a fixed list of weights and
    outputs: the descriptor table is built here, and each call enqueues the
    conversion on torch's current stream with one call into the library (for
    weights that are re-converted every training step).  The object keeps the
    tensors alive; `datas` / `scales` are the outputs."""

    def __init__(self, xs, datas=None, scales=None, scale_ld: Optional[int] = None, lib: str = "libmxq.so"):
        self._L = load(lib)
        xs = list(xs)
        n = len(xs)
        datas = [None] * n if datas is None else list(datas)
        scales = [None] * n if scales is None else list(scales)
        if len(datas) != n or len(scales) != n:
            raise ValueError("datas and scales must have one entry per weight")
        self.xs, self.n = xs, n
        if n == 0:
            self.datas, self.scales = [], []
            return
        dev, dtype = xs[0].device, xs[0].dtype
        for t in xs + datas + scales:
            if t is None:
                continue
            if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != dev:
                raise ValueError("mxq_mxfp4_to_mxfp8_row_grouped: operands must be device tensors on one device")
        if any(x.dtype != dtype for x in xs):
            raise ValueError("all weights of a group call must have one dtype")
        self._dt = _dtype_code(xs[0])
        self._table = (_RowGroup * n)()
        for i, x in enumerate(xs):
            px, rows, K, ldx = _matrix(x)
            nb = (K + 31) // 32
            if scales[i] is None:
                scales[i] = torch.zeros((rows, scale_ld or nb), dtype=torch.uint8, device=dev)
            if datas[i] is None:
                datas[i] = torch.empty((rows, K), dtype=torch.uint8, device=dev)
            pd, _, _, ldd = _matrix(datas[i])
            ps, _, _, ld_s = _matrix(scales[i])
            if rows * K and (ldd != K or datas[i].numel() != rows * K):
                raise ValueError("payload must be a contiguous [rows, K] uint8 tensor")
            self._table[i] = _RowGroup(px, ldx, rows, K, pd, ps, ld_s)
        self.datas, self.scales = datas, scales

    def __call__(self):
        if self.n:
            _check(self._L, self._L.mxq_mxfp4_to_mxfp8_row_grouped(self._table, self.n, self._dt,
                                                                    _stream(self.xs[0])))
        return self.datas, self.scales


class GroupedProjection:
    """The grouped MXFP4 projection prepared once for a fixed list of weights
    and outputs (an output may be its weight itself, in place); each call
    enqueues it on torch's current stream with one call into the library.  The
    object keeps the tensors alive; `ys` are the outputs."""

    def __init__(self, xs, ys=None, lib: str = "libmxq.so"):
        self._L = load(lib)
        xs = list(xs)
        n = len(xs)
        ys = [None] * n if ys is None else list(ys)
        if len(ys) != n:
            raise ValueError("ys must have one entry per weight")
        self.xs, self.n = xs, n
        if n == 0:
            self.ys = []
            return
        dev, dtype = xs[0].device, xs[0].dtype
        for t in xs + ys:
            if t is None:
                continue
            if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != dev:
                raise ValueError("mxq_fake_quantize_mxfp4_grouped: operands must be device tensors on one device")
        if any(x.dtype != dtype for x in xs):
            raise ValueError("all weights of a group call must have one dtype")
        self._dt = _dtype_code(xs[0])
        self._table = (_ProjGroup * n)()
        for i, x in enumerate(xs):
            if ys[i] is None:
                ys[i] = torch.empty_like(x, memory_format=torch.contiguous_format)
            if ys[i].dtype != x.dtype or ys[i].shape != x.shape:
                raise ValueError("each output must have its weight's dtype and shape")
            px, rows, K, ldx = _matrix(x)
            py, _, _, ldy = _matrix(ys[i])
            self._table[i] = _ProjGroup(px, ldx, py, ldy, rows, K)
        self.ys = ys

    def __call__(self):
        if self.n:
            _check(self._L, self._L.mxq_fake_quantize_mxfp4_grouped(self._table, self.n, self._dt, _stream(self.xs[0])))
        return self.ys


class GroupedBlock128:
    """The grouped 128x128 fold prepared once for a fixed list of weights and
    outputs; each call enqueues it on torch's current stream with one call into
    the library.  The object keeps the tensors alive; `datas` / `tile_codes`
    are the outputs."""

    def __init__(self, xs, datas=None, tile_codes=None, lib: str = "libmxq.so"):
        self._L = load(lib)
        xs = list(xs)
        n = len(xs)
        datas = [None] * n if datas is None else list(datas)
        tile_codes = [None] * n if tile_codes is None else list(tile_codes)
        if len(datas) != n or len(tile_codes) != n:
            raise ValueError("datas and tile_codes must have one entry per weight")
        self.xs, self.n = xs, n
        if n == 0:
            self.datas, self.tile_codes = [], []
            return
        dev, dtype = xs[0].device, xs[0].dtype
        for t in xs + datas + tile_codes:
            if t is None:
                continue
            if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != dev:
                raise ValueError("mxq_mxfp4_to_fp8_block128_grouped: operands must be device tensors on one device")
        if any(x.dtype != dtype for x in xs):
            raise ValueError("all weights of a group call must have one dtype")
        self._dt = _dtype_code(xs[0])
        self._table = (_Block128Group * n)()
        for i, x in enumerate(xs):
            px, rows, K, ldx = _matrix(x)
            if datas[i] is None:
                datas[i] = torch.empty((rows, K), dtype=torch.uint8, device=dev)
            if tile_codes[i] is None:
                tile_codes[i] = torch.zeros(((rows + 127) // 128, (K + 127) // 128), dtype=torch.uint8, device=dev)
            pd, _, _, ldd = _matrix(datas[i])
            pt, _, _, ldt = _matrix(tile_codes[i])
            if rows * K and (ldd != K or datas[i].numel() != rows * K):
                raise ValueError("payload must be a contiguous [rows, K] uint8 tensor")
            self._table[i] = _Block128Group(px, ldx, rows, K, pd, pt, ldt)
        self.datas, self.tile_codes = datas, tile_codes

    def __call__(self):
        if self.n:
            _check(self._L, self._L.mxq_mxfp4_to_fp8_block128_grouped(self._table, self.n, self._dt,
                                                                       _stream(self.xs[0])))
        return self.datas, self.tile_codes


class GroupedDequantize:
    """The grouped decode prepared once for a fixed list of payloads, codes and
    outputs of one payload format, scale layout and output dtype; each call
    enqueues it on torch's current stream with one call into the library.  The
    object keeps the tensors alive; `outs` are the outputs."""

    def __init__(self, datas, scales, layout: int = MXQ_SCALE_ROW_1X32, fmt: int = MXQ_E4M3, outs=None,
                 out_dtype: torch.dtype = torch.bfloat16, lib: str = "libmxq.so"):
        self._L = load(lib)
        datas, scales = list(datas), list(scales)
        n = len(datas)
        outs = [None] * n if outs is None else list(outs)
        if len(scales) != n or len(outs) != n:
            raise ValueError("scales and outs must have one entry per payload")
        self.datas, self.n = datas, n
        self._fmt, self._layout = fmt, layout
        if n == 0:
            self.outs = []
            return
        dev = datas[0].device
        for t in datas + scales + outs:
            if t is None:
                continue
            if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != dev:
                raise ValueError("mxq_dequantize_grouped: operands must be device tensors on one device")
        for i, d in enumerate(datas):
            if outs[i] is None:
                outs[i] = torch.empty(tuple(d.shape), dtype=out_dtype, device=dev)
        if any(o.dtype != outs[0].dtype for o in outs):
            raise ValueError("all outputs of a group call must have one dtype")
        self._dt = _dtype_code(outs[0])
        self._table = (_DequantGroup * n)()
        for i in range(n):
            pd, rows, K, ldd = _matrix(datas[i])
            if rows * K and ldd != K:
                raise ValueError("payload must be contiguous")
            ps, _, _, lds = _matrix(scales[i])
            po, _, _, ldo = _matrix(outs[i])
            self._table[i] = _DequantGroup(pd, ps, lds, rows, K, po, ldo)
        self.outs = outs

    def __call__(self):
        if self.n:
            _check(self._L, self._L.mxq_dequantize_grouped(self._table, self.n, self._fmt, self._layout, self._dt,
                                                            _stream(self.datas[0])))
        return self.outs


class GroupedQuantizeMxfp4:
    """The grouped packed MXFP4 encode prepared once for a fixed list of
    weights and outputs; each call enqueues it on torch's current stream with
    one call into the library.  The object keeps the tensors alive; `packeds` /
    `scales` are the outputs."""

    def __init__(self, xs, packeds=None, scales=None, scale_ld: Optional[int] = None, lib: str = "libmxq.so"):
        self._L = load(lib)
        xs = list(xs)
        n = len(xs)
        packeds = [None] * n if packeds is None else list(packeds)
        scales = [None] * n if scales is None else list(scales)
        if len(packeds) != n or len(scales) != n:
            raise ValueError("packeds and scales must have one entry per weight")
        self.xs, self.n = xs, n
        if n == 0:
            self.packeds, self.scales = [], []
            return
        dev, dtype = xs[0].device, xs[0].dtype
        for t in xs + packeds + scales:
            if t is None:
                continue
            if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != dev:
                raise ValueError("mxq_quantize_mxfp4_grouped: operands must be device tensors on one device")
        if any(x.dtype != dtype for x in xs):
            raise ValueError("all weights of a group call must have one dtype")
        self._dt = _dtype_code(xs[0])
        self._table = (_Mxfp4Group * n)()
        for i, x in enumerate(xs):
            px, rows, K, ldx = _matrix(x)
            nb, pw = (K + 31) // 32, (K + 1) // 2
            if packeds[i] is None:
                packeds[i] = torch.empty((rows, pw), dtype=torch.uint8, device=dev)
            if scales[i] is None:
                scales[i] = torch.zeros((rows, scale_ld or nb), dtype=torch.uint8, device=dev)
            pp, _, _, ldp = _matrix(packeds[i])
            ps, _, _, ld_s = _matrix(scales[i])
            if rows * K and (ldp != pw or packeds[i].numel() != rows * pw):
                raise ValueError("packed must be a contiguous [rows, ceil(K/2)] uint8 tensor")
            self._table[i] = _Mxfp4Group(px, ldx, rows, K, pp, ps, ld_s)
        self.packeds, self.scales = packeds, scales

    def __call__(self):
        if self.n:
            _check(self._L, self._L.mxq_quantize_mxfp4_grouped(self._table, self.n, self._dt, _stream(self.xs[0])))
        return self.packeds, self.scales


@_device_operands
def mxq_quantize_mxfp4_grouped(xs, packeds=None, scales=None, scale_ld: Optional[int] = None,
                               lib: str = "libmxq.so"):
    """Packed MXFP4 (deployment format) of a list of weights of one dtype, in as
    few launches as possible -> (list of nibble pairs, list of E8M0 codes); the
    same bytes as one mxq_quantize_mxfp4 per weight.  GroupedQuantizeMxfp4
    prepares the call once for repeated use."""
    return GroupedQuantizeMxfp4(xs, packeds, scales, scale_ld, lib)()


@_device_operands
def mxq_dequantize_grouped(datas, scales, layout: int = MXQ_SCALE_ROW_1X32, fmt: int = MXQ_E4M3, outs=None,
                           out_dtype: torch.dtype = torch.bfloat16, lib: str = "libmxq.so"):
    """Decode a list of FP8 payloads with their E8M0 codes (one format, scale
    layout and output dtype), in as few launches as possible -> list of
    outputs; the same bits as one mxq_dequantize per payload.  `outs`: list of
    outputs (None entries, or None for the whole list, are allocated).
    GroupedDequantize prepares the call once for repeated use."""
    return GroupedDequantize(datas, scales, layout, fmt, outs, out_dtype, lib)()


@_device_operands
def mxq_mxfp4_to_fp8_block128_grouped(xs, datas=None, tile_codes=None, lib: str = "libmxq.so"):
    """Direct 128x128 blockwise FP8 of a list of weights of one dtype, in as few
    launches as possible -> (list of payloads, list of tile codes); the same
    bytes as one mxq_mxfp4_to_fp8_block128 per weight.  GroupedBlock128
    prepares the call once for repeated use."""
    return GroupedBlock128(xs, datas, tile_codes, lib)()


@_device_operands
def mxq_fake_quantize_mxfp4_grouped(xs, ys=None, lib: str = "libmxq.so"):
    """MXFP4 projection of a list of weights of one dtype, in as few launches as
    possible -> list of outputs; the same bits as one mxq_fake_quantize_mxfp4 per
    weight.  `ys`: list of outputs (None entries, or None for the whole list,
    are allocated; an entry may be its weight, in place).  GroupedProjection
    prepares the call once for repeated use."""
    return GroupedProjection(xs, ys, lib)()


@_device_operands
def mxq_mxfp4_to_mxfp8_row_grouped(xs, datas=None, scales=None, scale_ld: Optional[int] = None,
                                   lib: str = "libmxq.so"):
    """Direct MXFP8 rowwise lift of a list of weights of one dtype, in as few
    launches as possible -> (list of payloads, list of E8M0 codes); the same
    bytes as one mxq_mxfp4_to_mxfp8_row per weight.  `datas` / `scales`: lists
    of outputs (None entries, or None for the whole list, are allocated).
    GroupedRowLift prepares the call once for repeated use."""
    return GroupedRowLift(xs, datas, scales, scale_ld, lib)()


@_device_operands
def mxq_mxfp4_to_fp8_block128(x: torch.Tensor, data: Optional[torch.Tensor] = None,
                              tile_code: Optional[torch.Tensor] = None, lib: str = "libmxq.so",
                              noop: Optional[torch.Tensor] = None):
    """Direct 128x128 blockwise FP8 -> (payload uint8 [rows, K], tile codes uint8 [ceil(rows/128), tile_ld]).
    With `noop` (an int32 device tensor) this is mxq_mxfp4_to_fp8_block128_guarded."""
    L = load(lib)
    dt = _dtype_code(x)
    px, rows, K, ldx = _matrix(x)
    if data is None:
        data = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    if tile_code is None:
        tile_code = torch.zeros(((rows + 127) // 128, (K + 127) // 128), dtype=torch.uint8, device=x.device)
    pd, _, _, ldd = _matrix(data)
    pt, trows, tcols, ldt = _matrix(tile_code)
    if rows * K and (ldd != K or data.numel() != rows * K):
        raise ValueError("payload must be a contiguous [rows, K] uint8 tensor")
    if noop is None:
        _check(L, L.mxq_mxfp4_to_fp8_block128(px, ldx, rows, K, dt, pd, pt, ldt, _stream(x)))
    else:
        _check(L, L.mxq_mxfp4_to_fp8_block128_guarded(px, ldx, rows, K, dt, pd, pt, ldt, _flag(noop), _stream(x)))
    return data, tile_code


def _payload_for(x: torch.Tensor, rows: int, K: int, data: Optional[torch.Tensor]):
    if data is None:
        data = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    pd, _, _, ldd = _matrix(data)
    if rows * K and (ldd != K or data.numel() != rows * K):
        raise ValueError("payload must be a contiguous [rows, K] uint8 tensor")
    return data, pd


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
    if scale is None:
        scale = torch.zeros(((rows + 31) // 32, scale_ld or K), dtype=torch.uint8, device=x.device)
    data, pd = _payload_for(x, rows, K, data)
    ps, _, _, ld_s = _matrix(scale)
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
    nb = (K + 31) // 32
    if row_scale is None:
        row_scale = torch.zeros((rows, row_scale_ld or nb), dtype=torch.uint8, device=x.device)
    if col_scale is None:
        col_scale = torch.zeros(((rows + 31) // 32, col_scale_ld or K), dtype=torch.uint8, device=x.device)
    row_data, prd = _payload_for(x, rows, K, row_data)
    col_data, pcd = _payload_for(x, rows, K, col_data)
    prs, _, _, ld_rs = _matrix(row_scale)
    pcs, _, _, ld_cs = _matrix(col_scale)
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
    nb = (K + 31) // 32
    if y is None:
        y = torch.empty_like(x, memory_format=torch.contiguous_format)
    if scale is None:
        scale = torch.zeros((rows, scale_ld or nb), dtype=torch.uint8, device=x.device)
    if data is None:
        data = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    py, _, _, ldy = _matrix(y)
    pd, _, _, ldd = _matrix(data)
    ps, _, _, ld_s = _matrix(scale)
    if rows * K and (ldd != K or data.numel() != rows * K):
        raise ValueError("payload must be a contiguous [rows, K] uint8 tensor")
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
    ps, rows, sld, ld_s = _matrix(scale_storage)
    nb = (K + 31) // 32
    if scale_out is None:
        scale_out = torch.empty((rows, nb), dtype=torch.uint8, device=scale_storage.device)
    po, _, _, _ = _matrix(scale_out)
    _check(L, L.mxq_export_mxfp8(data.data_ptr(), ps, rows, K, ld_s, po, _stream(scale_storage)))
    return scale_out


@_device_operands
def mxq_dequantize(data: torch.Tensor, scale: torch.Tensor, layout: int = MXQ_SCALE_ROW_1X32, fmt: int = MXQ_E4M3,
                   out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                   lib: str = "libmxq.so") -> torch.Tensor:
    """Decode FP8 payload bytes with E8M0 codes into bf16 / fp32."""
    L = load(lib)
    pd, rows, K, ldd = _matrix(data)
    if rows * K and ldd != K:
        raise ValueError("payload must be contiguous")
    ps, srows, scols, lds = _matrix(scale)
    if out is None:
        out = torch.empty((rows, K), dtype=out_dtype, device=data.device)
    po, _, _, ldo = _matrix(out)
    _check(L, L.mxq_dequantize(pd, ps, lds, rows, K, fmt, layout, po, ldo,
                               _dtype_code(out), _stream(data)))
    return out


@_device_operands
def mxq_quantize_mxfp4(x: torch.Tensor, packed: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None,
                       scale_ld: Optional[int] = None, lib: str = "libmxq.so"):
    """Packed MXFP4 (deployment format) -> (nibble pairs uint8 [rows, ceil(K/2)], E8M0 codes)."""
    L = load(lib)
    dt = _dtype_code(x)
    px, rows, K, ldx = _matrix(x)
    nb = (K + 31) // 32
    if packed is None:
        packed = torch.empty((rows, (K + 1) // 2), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.zeros((rows, scale_ld or nb), dtype=torch.uint8, device=x.device)
    pp, _, pw, ldp = _matrix(packed)
    ps, _, _, ld_s = _matrix(scale)
    if rows * K and (ldp != (K + 1) // 2 or pw != (K + 1) // 2):
        raise ValueError("packed must be a contiguous [rows, ceil(K/2)] uint8 tensor")
    _check(L, L.mxq_quantize_mxfp4(px, ldx, rows, K, dt, pp, ps, ld_s, _stream(x)))
    return packed, scale


def _packed_args(packed: torch.Tensor, scale: torch.Tensor, K: int):
    pp, rows, pw, ldp = _matrix(packed)
    if rows * K and (pw != (K + 1) // 2 or ldp != pw):
        raise ValueError("packed must be a contiguous [rows, ceil(K/2)] uint8 tensor")
    ps, _, _, ld_s = _matrix(scale)
    return pp, ps, ld_s, rows


@_device_operands
def mxq_dequantize_mxfp4(packed: torch.Tensor, scale: torch.Tensor, K: int, out: Optional[torch.Tensor] = None,
                         out_dtype: torch.dtype = torch.bfloat16, lib: str = "libmxq.so") -> torch.Tensor:
    """Decode packed MXFP4 into bf16 / fp32 [rows, K]."""
    L = load(lib)
    pp, ps, ld_s, rows = _packed_args(packed, scale, K)
    if out is None:
        out = torch.empty((rows, K), dtype=out_dtype, device=packed.device)
    po, _, _, ldo = _matrix(out)
    _check(L, L.mxq_dequantize_mxfp4(pp, ps, ld_s, rows, K, po, ldo, _dtype_code(out), _stream(packed)))
    return out


@_device_operands
def mxq_mxfp4_packed_to_mxfp8_row(packed: torch.Tensor, scale: torch.Tensor, K: int,
                                  data: Optional[torch.Tensor] = None, scale_out: Optional[torch.Tensor] = None,
                                  lib: str = "libmxq.so"):
    """Direct MXFP8 row lift from packed MXFP4 -> (payload uint8 [rows, K], codes)."""
    L = load(lib)
    pp, ps, ld_s, rows = _packed_args(packed, scale, K)
    if data is None:
        data = torch.empty((rows, K), dtype=torch.uint8, device=packed.device)
    if scale_out is None:
        scale_out = torch.zeros((rows, (K + 31) // 32), dtype=torch.uint8, device=packed.device)
    pd, _, _, _ = _matrix(data)
    po, _, _, ldo = _matrix(scale_out)
    _check(L, L.mxq_mxfp4_packed_to_mxfp8_row(pp, ps, ld_s, rows, K, pd, po, ldo, _stream(packed)))
    return data, scale_out


@_device_operands
def mxq_mxfp4_packed_to_fp8_block128(packed: torch.Tensor, scale: torch.Tensor, K: int,
                                     data: Optional[torch.Tensor] = None, tile_code: Optional[torch.Tensor] = None,
                                     lib: str = "libmxq.so"):
    """Direct 128x128 blockwise FP8 from packed MXFP4 -> (payload uint8 [rows, K], tile codes)."""
    L = load(lib)
    pp, ps, ld_s, rows = _packed_args(packed, scale, K)
    if data is None:
        data = torch.empty((rows, K), dtype=torch.uint8, device=packed.device)
    if tile_code is None:
        tile_code = torch.zeros(((rows + 127) // 128, (K + 127) // 128), dtype=torch.uint8, device=packed.device)
    pd, _, _, _ = _matrix(data)
    pt, _, _, ldt = _matrix(tile_code)
    _check(L, L.mxq_mxfp4_packed_to_fp8_block128(pp, ps, ld_s, rows, K, pd, pt, ldt, _stream(packed)))
    return data, tile_code


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
