"""Seeded random sweep through every entry point against the oracle, bit for bit.

Each case draws a shape (rows 1..300, K 1..3000 -- two cases in eight up to
600 x 9000 -- or a power-of-two K), a dtype,
a row-stride pad and an element offset for the input view (views that are not
16-byte aligned, or whose stride is not a multiple of the chunk, take the
element-wise paths), and pads for every scale storage.  The values are weights
at random block exponents (including the subnormal and saturating ends) with
zeros of both signs, subnormals, Inf and NaN planted at random.  The case id is
its seed, so any failure reproduces from the test name.
"""
import numpy as np
import pytest
import torch

import microscaling_weight_quantization_amd as mxq
import oracle
from tests.test_gpu_parity import THREADS, assert_bits, to_dev, to_host

pytestmark = pytest.mark.gpu

SEEDS = list(range(1000, 1160))


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mxq.load()
    return torch.device("cuda:0")


def draw(seed):
    g = np.random.default_rng(seed)
    big = seed % 8 in (3, 6)                      # larger cases (both dtypes): longer rows, several steps per row
    rows = int(g.integers(1, 601 if big else 301))
    K = int(g.choice([32, 128, 256, 2048, 4096])) if seed % 4 == 0 else int(g.integers(1, 9001 if big else 3001))
    dtype = "fp32" if seed % 2 else "bf16"
    pad = int(g.choice([0, 0, 1, 8, 13]))         # row stride K + pad
    off = int(g.choice([0, 0, 1, 3]))             # element offset of the view
    spad = int(g.choice([0, 0, 3, 8]))            # scale-storage pad
    opad = int(g.choice([0, 0, 4, 5]))            # output row-stride pad (projection, decodes)
    nb = (K + 31) // 32
    e = g.integers(-134, 124, size=(rows, nb))
    v = g.standard_normal((rows, nb * 32)) * np.exp2(np.repeat(e, 32, axis=1).astype(np.float64))
    v = v[:, :K].astype(np.float32)
    n = rows * K
    for val, frac in ((0.0, 0.01), (-0.0, 0.01), (np.inf, 0.0005), (-np.inf, 0.0005), (np.nan, 0.0005),
                      (1e-40, 0.002), (3e38, 0.001)):
        idx = g.choice(n, size=max(1, int(n * frac)) if g.random() < 0.7 else 0, replace=True)
        v.reshape(-1)[idx] = val
    if dtype == "bf16":
        bits = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    else:
        bits = v.view(np.uint32).copy()
    return rows, K, dtype, pad, off, spad, opad, bits


def strided_view(bits, pad, off, dev):
    """The same values as a [rows, K] device view with row stride K + pad that
    starts `off` elements into its allocation."""
    rows, K = bits.shape
    tdt = torch.bfloat16 if bits.dtype == np.uint16 else torch.float32
    flat = torch.zeros(off + rows * (K + pad), dtype=tdt, device=dev)
    view = flat[off:].view(rows, K + pad)[:, :K]
    view.copy_(to_dev(bits, dev))
    return view


SENTINEL = {torch.bfloat16: 0x7E55, torch.float32: 0x7E55AA11}


def out_view(rows, K, opad, tdt, dev):
    """A [rows, K] output view with row stride K + opad whose pad columns hold a
    sentinel pattern (checked afterwards: nothing may be written there)."""
    idt = torch.int16 if tdt == torch.bfloat16 else torch.int32
    full = torch.full((rows, K + opad), SENTINEL[tdt], dtype=idt, device=dev).view(tdt)
    return full, full[:, :K]


def check_pad(full, K, what):
    if full.shape[1] > K:
        pad = full[:, K:].view(torch.int16 if full.dtype == torch.bfloat16 else torch.int32)
        assert bool((pad == SENTINEL[full.dtype]).all()), f"{what}: write into the row-stride pad"


@pytest.mark.parametrize("seed", SEEDS)
def test_random_case(dev, seed):
    rows, K, dtype, pad, off, spad, opad, bits = draw(seed)
    print(f"case {seed}: rows={rows} K={K} {dtype} pad={pad} off={off} spad={spad} opad={opad}", flush=True)
    x = strided_view(bits, pad, off, dev)
    nb, bands = (K + 31) // 32, (rows + 31) // 32
    outs = ((torch.bfloat16, oracle.BF16), (torch.float32, oracle.FP32))

    # projection, into a padded output view
    wy = oracle.fake_quantize_mxfp4(bits, threads=THREADS)
    yfull, y = out_view(rows, K, opad, x.dtype, dev)
    mxq.mxq_fake_quantize_mxfp4(x, y)
    assert_bits(to_host(y), wy, "projection")
    check_pad(yfull, K, "projection")

    # row lift, export, row decode
    scale = torch.full((rows, nb + spad), 0xA5, dtype=torch.uint8, device=dev)
    data, scale = mxq.mxq_mxfp4_to_mxfp8_row(x, scale=scale)
    wd, ws = oracle.mxfp4_to_mxfp8_row(bits, scale_ld=nb + spad, threads=THREADS, fill=0xA5)
    assert_bits(to_host(data), wd, "row payload")
    assert_bits(to_host(scale), ws, "row codes (padding untouched)")
    codes = mxq.mxq_export_mxfp8(data, scale, K)
    assert_bits(to_host(codes), oracle.export_mxfp8(ws, K), "export")
    for tdt, o in outs:
        ofull, ov = out_view(rows, K, opad, tdt, dev)
        mxq.mxq_dequantize(data, codes, out=ov)
        assert_bits(to_host(ov), oracle.dequantize(wd, ws[:, :nb], out_dtype=o, threads=THREADS), f"row decode {tdt}")
        check_pad(ofull, K, f"row decode {tdt}")

    # fused projection + row lift
    s2 = torch.full((rows, nb + spad), 0x5A, dtype=torch.uint8, device=dev)
    y2full, y2 = out_view(rows, K, opad, x.dtype, dev)
    y2, d2, s2 = mxq.mxq_fake_quantize_mxfp4_with_mxfp8_row(x, y=y2, scale=s2)
    assert_bits(to_host(y2), wy, "fused projection")
    check_pad(y2full, K, "fused projection")
    assert_bits(to_host(d2), wd, "fused payload")
    assert_bits(to_host(s2)[:, :nb], ws[:, :nb], "fused codes")

    # 128x128 fold and its decode
    bd, tc = mxq.mxq_mxfp4_to_fp8_block128(x)
    wbd, wtc = oracle.mxfp4_to_fp8_block128(bits, threads=THREADS)
    assert_bits(to_host(bd), wbd, "128x128 payload")
    assert_bits(to_host(tc), wtc, "tile codes")
    for tdt, o in outs:
        assert_bits(to_host(mxq.mxq_dequantize(bd, tc, layout=mxq.MXQ_SCALE_TILE_128X128, out_dtype=tdt)),
                    oracle.dequantize(wbd, wtc, layout=oracle.TILE_128X128, out_dtype=o, threads=THREADS),
                    f"tile decode {tdt}")

    # columnwise, row + columnwise, column decode
    cs = torch.full((bands, K + spad), 0xC3, dtype=torch.uint8, device=dev)
    cd, cs = mxq.mxq_mxfp4_to_mxfp8_col(x, scale=cs)
    wcd, wcs = oracle.mxfp4_to_mxfp8_col(bits, scale_ld=K + spad, threads=THREADS, fill=0xC3)
    assert_bits(to_host(cd), wcd, "column payload")
    assert_bits(to_host(cs), wcs, "column codes (padding untouched)")
    for tdt, o in outs:
        assert_bits(to_host(mxq.mxq_dequantize(cd, cs, layout=mxq.MXQ_SCALE_COL_32X1, out_dtype=tdt)),
                    oracle.dequantize(wcd, wcs, layout=oracle.COL_32X1, out_dtype=o, threads=THREADS),
                    f"column decode {tdt}")
    rd, rs, cd2, cs2 = mxq.mxq_mxfp4_to_mxfp8_row_col(x)
    assert_bits(to_host(rd), wd, "row+col: row payload")
    assert_bits(to_host(rs), ws[:, :nb], "row+col: row codes")
    assert_bits(to_host(cd2), wcd, "row+col: column payload")
    assert_bits(to_host(cs2), wcs[:, :K], "row+col: column codes")

    # packed MXFP4 and the conversions from it
    ps = torch.full((rows, nb + spad), 0x3C, dtype=torch.uint8, device=dev)
    packed, ps = mxq.mxq_quantize_mxfp4(x, scale=ps)
    wp, wps = oracle.quantize_mxfp4(bits, scale_ld=nb + spad, threads=THREADS, fill=0x3C)
    assert_bits(to_host(packed), wp, "packed nibbles")
    assert_bits(to_host(ps), wps, "packed codes (padding untouched)")
    for tdt, o in outs:
        ofull, ov = out_view(rows, K, opad, tdt, dev)
        mxq.mxq_dequantize_mxfp4(packed, ps, K, out=ov)
        assert_bits(to_host(ov), oracle.dequantize_mxfp4(wp, wps, K, out_dtype=o, threads=THREADS), f"packed decode {tdt}")
        check_pad(ofull, K, f"packed decode {tdt}")
    pd, pc = mxq.mxq_mxfp4_packed_to_mxfp8_row(packed, ps, K)
    wpd, wpc = oracle.mxfp4_packed_to_mxfp8_row(wp, wps, K, threads=THREADS)
    assert_bits(to_host(pd), wpd, "row lift from packed")
    assert_bits(to_host(pc), wpc, "row codes from packed")
    fd, fc = mxq.mxq_mxfp4_packed_to_fp8_block128(packed, ps, K)
    wfd, wfc = oracle.mxfp4_packed_to_fp8_block128(wp, wps, K, threads=THREADS)
    assert_bits(to_host(fd), wfd, "128x128 payload from packed")
    assert_bits(to_host(fc), wfc, "tile codes from packed")
