"""The C-ABI library on the host (no GPU): it loads, exports every entry point
include/mxq.h declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import microscaling_weight_quantization_amd as mxq
from microscaling_weight_quantization_amd import build as B

HEADER = os.path.join(B.ROOT, "include", "mxq.h")


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(mxq_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if B.stale():
        B.build(["libmxq.so"])
    return mxq.load()


def test_header_declares_the_entry_points():
    assert declared() == sorted(mxq.ENTRY_POINTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s+(mxq_\w+)$", out, flags=re.M))
    assert set(declared()) <= exported
    for name in declared():
        assert hasattr(lib, name)


def test_header_compiles_as_c():
    src = f'#include "mxq.h"\nint main(void) {{ return (int)(mxq_status_string != 0) - 1; }}\n'
    r = subprocess.run(["gcc", "-fsyntax-only", "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I", os.path.dirname(HEADER),
                        "-I", "/opt/rocm/include", "-x", "c", "-"], input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings(lib):
    for code in range(7):
        assert lib.mxq_status_string(code)
    assert b"fp16" in lib.mxq_status_string(mxq.MXQ_ERR_DTYPE)
    assert lib.mxq_status_string(99) == b"unknown status"


def test_host_validation_without_a_gpu(lib):
    """Every one of these returns before anything is enqueued."""
    P = ctypes.c_void_p
    fake = P(0x100000)
    assert lib.mxq_fake_quantize_mxfp4(fake, 64, fake, 64, 4, 64, mxq.MXQ_FP16, None) == mxq.MXQ_ERR_DTYPE
    assert lib.mxq_fake_quantize_mxfp4(fake, 64, fake, 64, 4, 64, 7, None) == mxq.MXQ_ERR_DTYPE
    assert lib.mxq_fake_quantize_mxfp4(None, 64, fake, 64, 4, 64, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_NULL
    assert lib.mxq_fake_quantize_mxfp4(fake, 32, P(0x200000), 64, 4, 64, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_fake_quantize_mxfp4(fake, 64, fake, 64, -1, 64, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_fake_quantize_mxfp4(None, 0, None, 0, 0, 64, mxq.MXQ_BF16, None) == mxq.MXQ_OK   # empty
    assert lib.mxq_fake_quantize_mxfp4(None, 0, None, 0, 4, 0, mxq.MXQ_FP32, None) == mxq.MXQ_OK
    # partial overlap between x and y
    assert lib.mxq_fake_quantize_mxfp4(fake, 64, P(0x100002), 64, 4, 64, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_ALIAS
    # in place with a different stride is an overlap, not in-place
    assert lib.mxq_fake_quantize_mxfp4(fake, 64, fake, 128, 4, 64, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_ALIAS
    # row lift: scale storage too narrow, outputs overlapping
    assert lib.mxq_mxfp4_to_mxfp8_row(fake, 64, 4, 64, mxq.MXQ_BF16, P(0x200000), P(0x300000), 1, None) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_mxfp4_to_mxfp8_row(fake, 64, 4, 64, mxq.MXQ_BF16, P(0x200000), P(0x200010), 2, None) == mxq.MXQ_ERR_ALIAS
    assert lib.mxq_mxfp4_to_mxfp8_row(fake, 64, 4, 64, mxq.MXQ_BF16, P(0x100040), P(0x300000), 2, None) == mxq.MXQ_ERR_ALIAS
    # fused projection + row lift: y required, y must not overlap the payload
    assert lib.mxq_fake_quantize_mxfp4_with_mxfp8_row(fake, 64, None, 64, 4, 64, 0, P(0x200000), P(0x300000), 2, None) == mxq.MXQ_ERR_NULL
    assert lib.mxq_fake_quantize_mxfp4_with_mxfp8_row(fake, 64, P(0x200000), 64, 4, 64, 0, P(0x200010), P(0x300000), 2, None) == mxq.MXQ_ERR_ALIAS
    assert lib.mxq_fake_quantize_mxfp4_with_mxfp8_row(fake, 64, fake, 64, 4, 64, mxq.MXQ_FP16, P(0x200000), P(0x300000), 2, None) == mxq.MXQ_ERR_DTYPE
    # guarded variants need their flag
    assert lib.mxq_mxfp4_to_mxfp8_row_guarded(fake, 64, 4, 64, 0, P(0x200000), P(0x300000), 2, None, None) == mxq.MXQ_ERR_NULL
    assert lib.mxq_mxfp4_to_fp8_block128_guarded(fake, 256, 4, 256, 0, P(0x200000), P(0x300000), 2, None, None) == mxq.MXQ_ERR_NULL
    # block128: tile_ld too small
    assert lib.mxq_mxfp4_to_fp8_block128(fake, 256, 4, 256, mxq.MXQ_FP32, P(0x200000), P(0x300000), 1, None) == mxq.MXQ_ERR_SHAPE
    # export: no row-scaled data, the view case, bad stride
    assert lib.mxq_export_mxfp8(None, fake, 4, 64, 2, P(0x200000), None) == mxq.MXQ_ERR_NO_ROWWISE_DATA
    assert lib.mxq_export_mxfp8(fake, None, 4, 64, 2, P(0x200000), None) == mxq.MXQ_ERR_NO_ROWWISE_DATA
    assert lib.mxq_export_mxfp8(P(0x500000), fake, 4, 64, 2, fake, None) == mxq.MXQ_OK
    assert lib.mxq_export_mxfp8(P(0x500000), fake, 4, 64, 1, P(0x200000), None) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_export_mxfp8(P(0x500000), fake, 4, 64, 4, P(0x100001), None) == mxq.MXQ_ERR_ALIAS
    # dequantize: bad format / layout / dtype, narrow scale
    assert lib.mxq_dequantize(fake, P(0x200000), 2, 4, 64, 5, 0, P(0x300000), 64, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_DTYPE
    assert lib.mxq_dequantize(fake, P(0x200000), 2, 4, 64, 0, 9, P(0x300000), 64, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_DTYPE
    assert lib.mxq_dequantize(fake, P(0x200000), 2, 4, 64, 0, 0, P(0x300000), 64, mxq.MXQ_FP16, None) == mxq.MXQ_ERR_DTYPE
    assert lib.mxq_dequantize(fake, P(0x200000), 1, 4, 64, 0, 0, P(0x300000), 64, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_dequantize(fake, P(0x200000), 1, 4, 64, 0, 1, P(0x100010), 64, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_ALIAS
    # dequantize, 32x1 column layout: code rows must span K
    assert lib.mxq_dequantize(fake, P(0x200000), 63, 40, 64, 0, 2, P(0x300000), 64, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_dequantize(fake, P(0x200000), 64, 40, 64, 0, 3, P(0x300000), 64, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_DTYPE
    # columnwise: code rows narrower than K, overlaps, missing row outputs, fp16
    assert lib.mxq_mxfp4_to_mxfp8_col(fake, 64, 40, 64, 0, P(0x200000), P(0x300000), 63, None) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_mxfp4_to_mxfp8_col(fake, 64, 40, 64, 0, P(0x200000), P(0x200000 + 40 * 64 - 1), 64, None) == mxq.MXQ_ERR_ALIAS
    assert lib.mxq_mxfp4_to_mxfp8_col(fake, 64, 40, 64, 0, P(0x100010), P(0x300000), 64, None) == mxq.MXQ_ERR_ALIAS
    assert lib.mxq_mxfp4_to_mxfp8_col(fake, 64, 40, 64, mxq.MXQ_FP16, P(0x200000), P(0x300000), 64, None) == mxq.MXQ_ERR_DTYPE
    assert lib.mxq_mxfp4_to_mxfp8_col(None, 64, 40, 64, 0, P(0x200000), P(0x300000), 64, None) == mxq.MXQ_ERR_NULL
    assert lib.mxq_mxfp4_to_mxfp8_col(None, 64, 0, 64, 0, None, None, 64, None) == mxq.MXQ_OK
    assert lib.mxq_mxfp4_to_mxfp8_row_col(fake, 64, 40, 64, 0, None, P(0x400000), 2, P(0x200000), P(0x300000), 64,
                                          None) == mxq.MXQ_ERR_NULL
    assert lib.mxq_mxfp4_to_mxfp8_row_col(fake, 64, 40, 64, 0, P(0x200000), P(0x400000), 2, P(0x200000),
                                          P(0x300000), 64, None) == mxq.MXQ_ERR_ALIAS
    assert lib.mxq_mxfp4_to_mxfp8_row_col(fake, 64, 40, 64, 0, P(0x500000), P(0x400000), 1, P(0x200000),
                                          P(0x300000), 64, None) == mxq.MXQ_ERR_SHAPE
    # gated columnwise forms need their flag
    assert lib.mxq_mxfp4_to_mxfp8_col_guarded(fake, 64, 40, 64, 0, P(0x200000), P(0x300000), 64, None,
                                              None) == mxq.MXQ_ERR_NULL
    assert lib.mxq_mxfp4_to_mxfp8_row_col_guarded(fake, 64, 40, 64, 0, P(0x500000), P(0x400000), 2, P(0x200000),
                                                  P(0x300000), 64, None, None) == mxq.MXQ_ERR_NULL
    # packed MXFP4: narrow code storage, overlaps, odd shapes
    assert lib.mxq_quantize_mxfp4(fake, 64, 4, 64, 0, P(0x200000), P(0x300000), 1, None) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_quantize_mxfp4(fake, 64, 4, 64, 0, P(0x200000), P(0x200010), 2, None) == mxq.MXQ_ERR_ALIAS
    assert lib.mxq_dequantize_mxfp4(fake, P(0x200000), 1, 4, 64, P(0x300000), 64, 0, None) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_dequantize_mxfp4(fake, P(0x200000), 2, 4, 64, P(0x300000), 64, mxq.MXQ_FP16, None) == mxq.MXQ_ERR_DTYPE
    assert lib.mxq_mxfp4_packed_to_mxfp8_row(fake, P(0x200000), 2, 4, 64, P(0x300000), P(0x300000), 2,
                                             None) == mxq.MXQ_ERR_ALIAS
    assert lib.mxq_mxfp4_packed_to_fp8_block128(fake, P(0x200000), 2, 4, 64, P(0x300000), P(0x400000), 0,
                                                None) == mxq.MXQ_ERR_SHAPE
    # shapes too large for the launch grid are refused, not truncated (buffers
    # placed far apart so that no overlap is reported first)
    huge, far = 1 << 40, lambda k: P(1 << k)
    assert lib.mxq_fake_quantize_mxfp4(fake, 64, far(50), 64, huge, 64, 0, None) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_mxfp4_to_mxfp8_row(fake, 64, huge, 64, 0, far(50), far(52), 2, None) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_mxfp4_to_mxfp8_col(fake, 64, huge, 64, 0, far(50), far(52), 64, None) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_mxfp4_to_fp8_block128(fake, 1 << 10, huge, 1 << 10, 0, far(56), far(58), 8,
                                         None) == mxq.MXQ_ERR_SHAPE


def test_absurd_strides_are_rejected(lib):
    """A matrix whose byte span could not be an allocation (2^56 bytes or more,
    or past the end of the address space) is a shape error, found before any
    range arithmetic can overflow -- including the in-place projection, which
    has no alias check to trip over."""
    P = ctypes.c_void_p
    fake, far = P(0x100000), lambda k: P(1 << k)
    S = mxq.MXQ_ERR_SHAPE
    big = 1 << 62
    assert lib.mxq_fake_quantize_mxfp4(fake, big, fake, big, 4, 64, 0, None) == S           # in place
    assert lib.mxq_fake_quantize_mxfp4(fake, 64, far(50), big, 4, 64, 0, None) == S
    assert lib.mxq_mxfp4_to_mxfp8_row(fake, big, 4, 64, 0, far(50), far(52), 2, None) == S
    assert lib.mxq_mxfp4_to_mxfp8_row(fake, 64, 4, 64, 0, far(50), far(52), big, None) == S
    assert lib.mxq_fake_quantize_mxfp4_with_mxfp8_row(fake, 64, far(48), big, 4, 64, 0, far(50), far(52), 2,
                                                      None) == S
    assert lib.mxq_mxfp4_to_fp8_block128(fake, big, 4, 256, 0, far(50), far(52), 2, None) == S
    assert lib.mxq_mxfp4_to_mxfp8_col(fake, big, 40, 64, 0, far(50), far(52), 64, None) == S
    assert lib.mxq_mxfp4_to_mxfp8_row_col(fake, 64, 40, 64, 0, far(50), far(52), big, far(54), far(55), 64,
                                          None) == S
    assert lib.mxq_export_mxfp8(far(50), fake, 4, 64, 1 << 58, far(52), None) == S
    assert lib.mxq_dequantize(fake, far(50), 2, 4, 64, 0, 0, far(52), big, mxq.MXQ_BF16, None) == S
    assert lib.mxq_quantize_mxfp4(fake, 64, 4, 64, 0, far(50), far(52), big, None) == S
    assert lib.mxq_dequantize_mxfp4(fake, far(50), big, 4, 64, far(52), 64, 0, None) == S
    assert lib.mxq_mxfp4_packed_to_mxfp8_row(fake, far(50), big, 4, 64, far(52), far(54), 2, None) == S
    # (two tile rows, so the tile-code stride matters)
    assert lib.mxq_mxfp4_packed_to_fp8_block128(fake, far(50), 2, 256, 64, far(52), far(54), big, None) == S
    # a buffer running past the top of the address space
    top = P((1 << 64) - 4096)
    assert lib.mxq_fake_quantize_mxfp4(top, 64, top, 64, 64, 64, 0, None) == S
    assert lib.mxq_mxfp4_to_mxfp8_row(fake, 64, 4, 64, 0, P((1 << 64) - 128), far(52), 2, None) == S   # 256 B payload


def test_binding_raises_without_the_library(tmp_path, monkeypatch):
    monkeypatch.setattr(B, "library_path", lambda name="libmxq.so": str(tmp_path / name))
    with pytest.raises(FileNotFoundError):
        mxq.load("libmxq_missing.so")


def test_binding_rejects_host_tensors():
    """The binding passes raw pointers: a host tensor must be refused before any
    launch (it would reach a kernel as an invalid device address)."""
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    calls = [
        lambda: mxq.mxq_fake_quantize_mxfp4(x),
        lambda: mxq.mxq_mxfp4_to_mxfp8_row(x),
        lambda: mxq.mxq_mxfp4_to_fp8_block128(x),
        lambda: mxq.mxq_mxfp4_to_mxfp8_col(x),
        lambda: mxq.mxq_fake_quantize_mxfp4_with_mxfp8_row(x),
        lambda: mxq.mxq_quantize_mxfp4(x),
        lambda: mxq.mxq_export_mxfp8(torch.zeros(4, 64, dtype=torch.uint8), torch.zeros(4, 4, dtype=torch.uint8), 64),
        lambda: mxq.mxq_dequantize(torch.zeros(4, 64, dtype=torch.uint8), torch.zeros(4, 2, dtype=torch.uint8)),
        lambda: mxq.mxq_dequantize_mxfp4(torch.zeros(4, 32, dtype=torch.uint8), torch.zeros(4, 2, dtype=torch.uint8), 64),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="device tensors"):
            call()
    # every entry function carries the check
    names = [n for n in dir(mxq) if n.startswith("mxq_") and callable(getattr(mxq, n))]
    assert names and all(hasattr(getattr(mxq, n), "__wrapped__") for n in names)


def test_binding_operand_extent_checks():
    """Every operand whose extent the binding knows is checked against the
    region the C call touches before anything is launched (the C entry points
    see only a pointer and a stride): too few rows or columns, a single row
    standing in for several, a payload that is not packed row by row, and a
    payload or code array whose elements are not bytes all raise ValueError."""
    import torch
    op = mxq._operand
    codes = torch.zeros(100, 4, dtype=torch.uint8)
    assert op(codes, 100, 2, "scale")[1] == 4                        # padded storage: stride 4
    assert op(codes[:, :2], 100, 2, "scale")[1] == 4                 # a strided view that covers the region
    for bad, rows, cols in ((codes[:99], 100, 2), (codes[:, :1], 100, 2), (codes[:1], 100, 2),
                            (torch.zeros(1, 400, dtype=torch.uint8), 100, 2)):
        with pytest.raises(ValueError, match="must cover"):
            op(bad, rows, cols, "scale")
    data = torch.zeros(64, 128, dtype=torch.uint8)
    assert op(data, 64, 128, "payload", contiguous=True, byte=True)[1] == 128
    with pytest.raises(ValueError, match="contiguous"):
        op(data[:, :96], 64, 96, "payload", contiguous=True, byte=True)
    with pytest.raises(ValueError, match="bytes"):
        op(torch.zeros(64, 128, dtype=torch.bfloat16), 64, 128, "payload", contiguous=True, byte=True)
    assert op(torch.zeros(0, 4, dtype=torch.uint8), 0, 2, "scale")[1] == 4   # empty: nothing is touched


def test_grouped_row_lift_host_validation(lib):
    """The grouped row lift checks every group as the single call does, and
    refuses any output that overlaps another group's input or output -- all
    before anything is enqueued (fake addresses; no GPU is touched)."""
    G = mxq._RowGroup

    def grp(x, data, scale, rows=4, K=64, ld=64, sld=2):
        return G(x, ld, rows, K, data, scale, sld)

    def call(*groups, dt=mxq.MXQ_BF16, n=None):
        arr = (G * max(len(groups), 1))(*groups)
        return lib.mxq_mxfp4_to_mxfp8_row_grouped(arr, len(groups) if n is None else n, dt, None)

    # 4 x 64 bf16 weights take 512 bytes; payloads 256 bytes; codes 8 bytes
    a = grp(0x100000, 0x200000, 0x300000)
    b = grp(0x110000, 0x210000, 0x310000)
    assert call(a, b, n=-1) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_mxfp4_to_mxfp8_row_grouped(None, 2, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_NULL
    assert lib.mxq_mxfp4_to_mxfp8_row_grouped(None, 0, mxq.MXQ_BF16, None) == mxq.MXQ_OK
    assert call(a, b, dt=mxq.MXQ_FP16) == mxq.MXQ_ERR_DTYPE
    # a bad group anywhere in the list is reported
    assert call(a, grp(0x110000, 0x210000, 0x310000, K=-1)) == mxq.MXQ_ERR_SHAPE
    assert call(a, grp(None, 0x210000, 0x310000)) == mxq.MXQ_ERR_NULL
    assert call(a, grp(0x110000, 0x210000, 0x310000, sld=1)) == mxq.MXQ_ERR_SHAPE
    assert call(grp(0x100000, 0x100100, 0x300000), b) == mxq.MXQ_ERR_ALIAS          # within one group
    # across groups: an output over another group's input, over another output
    assert call(a, grp(0x110000, 0x100100, 0x310000)) == mxq.MXQ_ERR_ALIAS          # b's payload in a's weight
    assert call(a, grp(0x110000, 0x210000, 0x2000F0)) == mxq.MXQ_ERR_ALIAS          # b's codes in a's payload
    assert call(a, grp(0x110000, 0x200080, 0x310000)) == mxq.MXQ_ERR_ALIAS          # two payloads overlap
    assert call(a, grp(0x110000, 0x210000, 0x300004)) == mxq.MXQ_ERR_ALIAS          # two code arrays overlap
    assert call(grp(0x110000, 0x210000, 0x310000), grp(0x2100F0, 0x220000, 0x320000)) == mxq.MXQ_ERR_ALIAS  # an input over an output
    # empty groups only: nothing to do
    assert call(grp(None, None, None, rows=0), grp(None, None, None, K=0)) == mxq.MXQ_OK


def test_grouped_projection_host_validation(lib):
    """The grouped projection checks every weight as the single call does (in
    place allowed), and refuses an output over another weight's input or output,
    before anything is enqueued (fake addresses; no GPU is touched)."""
    G = mxq._ProjGroup

    def grp(x, y, rows=4, K=64, ldx=64, ldy=64):
        return G(x, ldx, y, ldy, rows, K)

    def call(*groups, dt=mxq.MXQ_BF16, n=None):
        arr = (G * max(len(groups), 1))(*groups)
        return lib.mxq_fake_quantize_mxfp4_grouped(arr, len(groups) if n is None else n, dt, None)

    a = grp(0x100000, 0x200000)                    # 4 x 64 bf16: 512 bytes each
    b = grp(0x110000, 0x210000)
    assert call(a, b, n=-1) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_fake_quantize_mxfp4_grouped(None, 1, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_NULL
    assert call(a, b, dt=mxq.MXQ_FP16) == mxq.MXQ_ERR_DTYPE
    assert call(a, grp(0x110000, None)) == mxq.MXQ_ERR_NULL
    assert call(a, grp(0x110000, 0x210000, ldx=32)) == mxq.MXQ_ERR_SHAPE
    assert call(a, grp(0x110000, 0x110002)) == mxq.MXQ_ERR_ALIAS                 # partial overlap in one weight
    assert call(a, grp(0x110000, 0x110000, ldx=64, ldy=128)) == mxq.MXQ_ERR_ALIAS  # in place needs equal strides
    assert call(a, grp(0x110000, 0x100100)) == mxq.MXQ_ERR_ALIAS                 # b's output over a's weight
    assert call(a, grp(0x110000, 0x200100)) == mxq.MXQ_ERR_ALIAS                 # two outputs overlap
    assert call(grp(0x100000, 0x100000), grp(0x100100, 0x210000)) == mxq.MXQ_ERR_ALIAS  # a weight inside an in-place one
    assert call(grp(None, None, rows=0), grp(None, None, K=0)) == mxq.MXQ_OK


def test_grouped_fold_host_validation(lib):
    """The grouped fold checks every weight as the single call does and refuses
    outputs over other weights' ranges, before anything is enqueued."""
    G = mxq._Block128Group

    def grp(x, data, tc, rows=4, K=256, ld=256, tld=2):
        return G(x, ld, rows, K, data, tc, tld)

    def call(*groups, dt=mxq.MXQ_BF16, n=None):
        arr = (G * max(len(groups), 1))(*groups)
        return lib.mxq_mxfp4_to_fp8_block128_grouped(arr, len(groups) if n is None else n, dt, None)

    a = grp(0x100000, 0x200000, 0x300000)          # 4 x 256 bf16: 2 KiB; payload 1 KiB; 2 tile codes
    b = grp(0x110000, 0x210000, 0x310000)
    assert call(a, b, n=-1) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_mxfp4_to_fp8_block128_grouped(None, 1, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_NULL
    assert call(a, b, dt=mxq.MXQ_FP16) == mxq.MXQ_ERR_DTYPE
    assert call(a, grp(0x110000, 0x210000, None)) == mxq.MXQ_ERR_NULL
    assert call(a, grp(0x110000, 0x210000, 0x310000, tld=1)) == mxq.MXQ_ERR_SHAPE
    assert call(a, grp(0x110000, 0x100400, 0x310000)) == mxq.MXQ_ERR_ALIAS      # b's payload in a's weight
    assert call(a, grp(0x110000, 0x210000, 0x200010)) == mxq.MXQ_ERR_ALIAS      # b's codes in a's payload
    assert call(a, grp(0x110000, 0x210000, 0x300001)) == mxq.MXQ_ERR_ALIAS      # code arrays overlap
    assert call(grp(None, None, None, rows=0), grp(None, None, None, K=0)) == mxq.MXQ_OK


def test_grouped_decode_host_validation(lib):
    """The grouped decode checks the call's format, layout and output dtype,
    every payload as the single call does, and refuses outputs over other
    payloads' ranges, before anything is enqueued."""
    G = mxq._DequantGroup

    def grp(data, scale, out, rows=4, K=256, sld=8, ldo=256):
        return G(data, scale, sld, rows, K, out, ldo)

    def call(*groups, fmt=mxq.MXQ_E4M3, lay=mxq.MXQ_SCALE_ROW_1X32, dt=mxq.MXQ_BF16, n=None):
        arr = (G * max(len(groups), 1))(*groups)
        return lib.mxq_dequantize_grouped(arr, len(groups) if n is None else n, fmt, lay, dt, None)

    a = grp(0x100000, 0x200000, 0x300000)          # 4 x 256 payload: 1 KiB; 4 x 8 codes; bf16 out 2 KiB
    b = grp(0x110000, 0x210000, 0x310000)
    assert call(a, b, n=-1) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_dequantize_grouped(None, 1, mxq.MXQ_E4M3, mxq.MXQ_SCALE_ROW_1X32, mxq.MXQ_BF16,
                                      None) == mxq.MXQ_ERR_NULL
    assert call(a, b, dt=mxq.MXQ_FP16) == mxq.MXQ_ERR_DTYPE
    assert call(a, b, fmt=7) == mxq.MXQ_ERR_DTYPE
    assert call(a, b, lay=9) == mxq.MXQ_ERR_DTYPE
    assert call(a, grp(0x110000, None, 0x310000)) == mxq.MXQ_ERR_NULL
    assert call(a, grp(0x110000, 0x210000, 0x310000, sld=7)) == mxq.MXQ_ERR_SHAPE
    assert call(a, grp(0x110000, 0x210000, 0x310000, ldo=255)) == mxq.MXQ_ERR_SHAPE
    assert call(a, b, lay=mxq.MXQ_SCALE_COL_32X1) == mxq.MXQ_ERR_SHAPE    # the column layout needs sld >= K
    assert call(a, grp(0x110000, 0x210000, 0x100000)) == mxq.MXQ_ERR_ALIAS  # b's output over a's payload
    assert call(a, grp(0x110000, 0x210000, 0x1FFF00)) == mxq.MXQ_ERR_ALIAS  # b's output over a's codes
    assert call(a, grp(0x110000, 0x210000, 0x300010)) == mxq.MXQ_ERR_ALIAS  # outputs overlap
    assert call(grp(0x100000, 0x200000, 0x100100)) == mxq.MXQ_ERR_ALIAS     # a single payload's own overlap
    assert call(grp(None, None, None, rows=0), grp(None, None, None, K=0)) == mxq.MXQ_OK


def test_grouped_mxfp4_encode_host_validation(lib):
    """The grouped packed encode checks every weight as the single call does
    and refuses outputs over other weights' ranges, before anything is
    enqueued."""
    G = mxq._Mxfp4Group

    def grp(x, packed, scale, rows=4, K=256, ld=256, sld=8):
        return G(x, ld, rows, K, packed, scale, sld)

    def call(*groups, dt=mxq.MXQ_BF16, n=None):
        arr = (G * max(len(groups), 1))(*groups)
        return lib.mxq_quantize_mxfp4_grouped(arr, len(groups) if n is None else n, dt, None)

    a = grp(0x100000, 0x200000, 0x300000)          # 4 x 256 bf16: 2 KiB; packed 512 B; 4 x 8 codes
    b = grp(0x110000, 0x210000, 0x310000)
    assert call(a, b, n=-1) == mxq.MXQ_ERR_SHAPE
    assert lib.mxq_quantize_mxfp4_grouped(None, 1, mxq.MXQ_BF16, None) == mxq.MXQ_ERR_NULL
    assert call(a, b, dt=mxq.MXQ_FP16) == mxq.MXQ_ERR_DTYPE
    assert call(a, grp(0x110000, None, 0x310000)) == mxq.MXQ_ERR_NULL
    assert call(a, grp(0x110000, 0x210000, 0x310000, sld=7)) == mxq.MXQ_ERR_SHAPE
    assert call(a, grp(0x110000, 0x210000, 0x310000, ld=255)) == mxq.MXQ_ERR_SHAPE
    assert call(a, grp(0x110000, 0x1001F0, 0x310000)) == mxq.MXQ_ERR_ALIAS      # b's nibbles in a's weight
    assert call(a, grp(0x110000, 0x210000, 0x2001F0)) == mxq.MXQ_ERR_ALIAS      # b's codes in a's nibbles
    assert call(a, grp(0x110000, 0x210000, 0x300010)) == mxq.MXQ_ERR_ALIAS      # code arrays overlap
    assert call(grp(0x100000, 0x100100, 0x300000)) == mxq.MXQ_ERR_ALIAS         # a single weight's own overlap
    assert call(grp(None, None, None, rows=0), grp(None, None, None, K=0)) == mxq.MXQ_OK


def test_access_shape_library_loads_and_refuses_bad_arguments():
    """libmxq_shapes.so (measurement only) exports the one entry point
    include/mxq_shapes.h declares, the header compiles as C, and the call
    turns down what does not fit before anything is launched."""
    name = "libmxq_shapes.so"
    if B.stale(name):
        B.build([name])
    path = B.library_path(name)
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    assert set(re.findall(r"\sT\s+(mxq_\w+)$", out, flags=re.M)) == {"mxq_shape_run"}
    header = os.path.join(B.ROOT, "include", "mxq_shapes.h")
    src = '#include "mxq_shapes.h"\nint main(void) { return MXQ_SHAPE_LINEAR_FOLD_NO_BARRIER == 7 ? 0 : 1; }\n'
    r = subprocess.run(["gcc", "-fsyntax-only", "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I", os.path.dirname(header),
                        "-I", "/opt/rocm/include", "-x", "c", "-"], input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    L = ctypes.CDLL(path)
    L.mxq_shape_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    fake = ctypes.c_void_p(0x100000)
    assert L.mxq_shape_run(0, 2, None, fake, fake, 8, 512, None) == 1          # null input
    assert L.mxq_shape_run(0, 3, fake, fake, fake, 8, 512, None) == 1          # element size
    assert L.mxq_shape_run(99, 2, fake, fake, fake, 8, 512, None) == 1         # no such shape
    assert L.mxq_shape_run(1, 2, fake, fake, fake, 1, 64, None) == 1           # not whole workgroups
    assert L.mxq_shape_run(4, 2, fake, fake, fake, 100, 128, None) == 1        # rows not tiles
    assert L.mxq_shape_run(6, 2, fake, fake, fake, 8, 512, None) == 1          # not whole tiles of elements
    assert L.mxq_shape_run(9, 2, fake, fake, fake, 1, 2048, None) == 1         # not whole read workgroups
    assert L.mxq_shape_run(13, 2, fake, fake, fake, 100, 128, None) == 1       # rows not tiles
    assert L.mxq_shape_run(0, 2, fake, fake, fake, 0, 512, None) == 1          # empty
