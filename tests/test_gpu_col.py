"""GPU parity of MXFP8 columnwise (32x1) from the MXFP4 decomposition, and of the
row + column pass, against the CPU oracle bit for bit (tolerance 0).

Inputs are the seeded workloads of ``workloads``; the same host bits feed the
oracle and the device copy.  Every weight -- the small, exhaustive,
spread-sweep, headline and MLP-shaped ones -- is compared in full."""
import numpy as np
import pytest
import torch

import microscaling_weight_quantization_amd as mxq
import oracle
import workloads as W
from tests.test_gpu_parity import assert_bits, out_dtype_of, to_dev, to_host

pytestmark = pytest.mark.gpu

THREADS = 16


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mxq.load()
    return torch.device("cuda:0")


def check_col(bits: np.ndarray, dev, pad: int = 0, lib: str = "libmxq.so", fused: bool = True):
    """Columnwise payload and codes (padding columns untouched), their decode in
    both output dtypes, and the row + column pass against row and column."""
    x = to_dev(bits, dev)
    rows, K = bits.shape
    nb = (K + 31) // 32
    bands = (rows + 31) // 32
    tdt, odt = out_dtype_of(bits)
    scale = torch.full((bands, K + pad), 0xA5, dtype=torch.uint8, device=dev)
    data, scale = mxq.mxq_mxfp4_to_mxfp8_col(x, scale=scale, lib=lib)
    wd, ws = oracle.mxfp4_to_mxfp8_col(bits, scale_ld=K + pad, threads=THREADS, fill=0xA5)
    assert_bits(to_host(data), wd, "column payload")
    assert_bits(to_host(scale), ws, "column codes (padding untouched)")
    for t, o in ((tdt, odt), (torch.float32, oracle.FP32)):
        dec = mxq.mxq_dequantize(data, scale, layout=mxq.MXQ_SCALE_COL_32X1, out_dtype=t, lib=lib)
        want = oracle.dequantize(wd, ws, layout=oracle.COL_32X1, out_dtype=o, threads=THREADS)
        assert_bits(to_host(dec), want, f"column decode to {t}")
    if fused:
        rs = torch.full((rows, nb + pad), 0x5A, dtype=torch.uint8, device=dev)
        cs = torch.full((bands, K + pad), 0x5A, dtype=torch.uint8, device=dev)
        rd, rs, cd, cs = mxq.mxq_mxfp4_to_mxfp8_row_col(x, row_scale=rs, col_scale=cs, lib=lib)
        wrd, wrs = oracle.mxfp4_to_mxfp8_row(bits, scale_ld=nb + pad, threads=THREADS, fill=0x5A)
        assert_bits(to_host(rd), wrd, "row + column pass: row payload")
        assert_bits(to_host(rs), wrs, "row + column pass: row codes")
        assert_bits(to_host(cd), wd, "row + column pass: column payload")
        ws2 = ws.copy()
        ws2[:, K:] = 0x5A
        assert_bits(to_host(cs), ws2, "row + column pass: column codes")


def test_col_c1_small(dev):
    check_col(W.c1_small(), dev, pad=4)


@pytest.mark.parametrize("natural", [False, True])
def test_col_c2_exhaustive(dev, natural):
    check_col(W.c2_exhaustive(natural=natural), dev)


def test_col_c2_planted(dev):
    check_col(W.c2_planted(), dev, pad=3)


def test_col_fp32_fuzz(dev):
    check_col(W.fp32_fuzz(1 << 18).reshape(-1, 256), dev)


def test_col_c3_spread_sweep(dev):
    check_col(W.c3_spread(), dev)


def test_col_c4_headline(dev):
    check_col(W.c4_headline(), dev)


@pytest.mark.parametrize("which", ["up", "down", "up_master"])
def test_col_c5_mlp_full(dev, which):
    """The MLP-shaped weights in full: every 32-row band's column payload and
    codes, their decodes, and the row + column pass, against the oracle."""
    check_col(W.c5_mlp(which), dev)


@pytest.mark.parametrize("rows,K", [(1, 1), (31, 7), (33, 33), (65, 100), (131, 257), (40, 2049), (96, 4096)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_col_ragged_shapes(dev, rows, K, dtype):
    if dtype == "bf16":
        flat = np.tile(W.c2_exhaustive().reshape(-1), (rows * K) // 65536 + 1)
    else:
        flat = W.fp32_fuzz(((rows * K + 31) // 32) * 32).reshape(-1)
    check_col(np.ascontiguousarray(flat[: rows * K].reshape(rows, K)), dev, pad=rows % 3)


@pytest.mark.parametrize("rows,K", [(1024, 8320), (2016, 2304), (100, 300), (2048, 2048)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_col_band_order_tails(dev, rows, K, dtype):
    """For fp32 the columnwise kernel deals its workgroups (32-row band x 256
    columns) to the XCDs in runs of 8, in groups of 64, and the last, partial
    group keeps the plain order: 1056, 567, 8 and 512 workgroups leave tails
    of 32, 55, 8 and 0.  bf16 (plain order) on the same shapes."""
    src = W.c2_planted() if dtype == "bf16" else W.c2_planted_fp32()
    bits = np.ascontiguousarray(np.resize(src.reshape(-1), rows * K).reshape(rows, K))
    check_col(bits, dev, pad=3)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_col_strided_and_misaligned_views(dev, dtype):
    base = W.c2_planted() if dtype == "bf16" else W.fp32_fuzz(64 * 200).reshape(64, 200)
    big = to_dev(np.ascontiguousarray(np.tile(base, (1, 4))), dev)
    K = 96
    for off in (0, 1, 3):
        view = big[:, off:off + K]
        bits = to_host(view)
        d, s = mxq.mxq_mxfp4_to_mxfp8_col(view)
        wd, ws = oracle.mxfp4_to_mxfp8_col(bits)
        assert_bits(to_host(d), wd, f"column payload off={off}")
        assert_bits(to_host(s), ws, f"column codes off={off}")


def test_col_decode_every_byte_and_code(dev):
    """Column layout: 256 bands of 32 rows; band b uses code b in every column
    and column c holds byte c, so every (code, byte) pair is decoded."""
    data = np.tile(np.arange(256, dtype=np.uint8), (32 * 256, 1))
    codes = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 256, axis=1)
    codes[:, 1::2] = codes[::-1, 1::2]                  # neighbouring columns use different codes
    dd, dc = to_dev(data, dev), to_dev(codes, dev)
    for fmt_dev, fmt_orc in ((mxq.MXQ_E4M3, oracle.E4M3), (mxq.MXQ_E5M2, oracle.E5M2)):
        for tdt, odt in ((torch.bfloat16, oracle.BF16), (torch.float32, oracle.FP32)):
            got = to_host(mxq.mxq_dequantize(dd, dc, layout=mxq.MXQ_SCALE_COL_32X1, fmt=fmt_dev, out_dtype=tdt))
            want = oracle.dequantize(data, codes, layout=oracle.COL_32X1, fp8=fmt_orc, out_dtype=odt, threads=THREADS)
            assert_bits(got, want, f"column decode {fmt_orc} {odt}")


def test_col_empty_and_errors(dev):
    for shape in ((0, 32), (5, 0)):
        x = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        d, s = mxq.mxq_mxfp4_to_mxfp8_col(x)
        assert d.shape == shape
    xb = torch.zeros((40, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="must cover"):  # code rows narrower than K: the binding refuses it
        mxq.mxq_mxfp4_to_mxfp8_col(xb, scale=torch.zeros((2, 63), dtype=torch.uint8, device=dev))
    with pytest.raises(mxq.MxqError) as e:
        mxq.mxq_mxfp4_to_mxfp8_col(torch.zeros((40, 64), dtype=torch.float16, device=dev))
    assert e.value.status == mxq.MXQ_ERR_DTYPE
    buf = torch.zeros((40 * 64 + 64,), dtype=torch.uint8, device=dev)
    with pytest.raises(mxq.MxqError) as e:              # column codes overlapping the column payload
        mxq.mxq_mxfp4_to_mxfp8_col(xb, data=buf[:40 * 64].view(40, 64), scale=buf[40 * 64 - 64:].view(2, 64))
    assert e.value.status == mxq.MXQ_ERR_ALIAS
    with pytest.raises(mxq.MxqError) as e:              # row payload overlapping the column payload
        d = torch.zeros((40, 64), dtype=torch.uint8, device=dev)
        mxq.mxq_mxfp4_to_mxfp8_row_col(xb, row_data=d, col_data=d)
    assert e.value.status == mxq.MXQ_ERR_ALIAS


@pytest.mark.parametrize("variant", ["libmxq_fastmath.so", "libmxq_o1.so", "libmxq_o0.so"])
def test_col_build_variants_identical_bits(dev, variant):
    for bits in (W.c2_exhaustive(natural=True), W.fp32_fuzz(1 << 16).reshape(-1, 128), W.c3_spread()[:256, :512]):
        check_col(np.ascontiguousarray(bits), dev, lib=variant)


def test_col_noop_flag_gates_the_columnwise_conversions(dev):
    bits = W.c4_headline(shape=(96, 1024))
    x = to_dev(bits, dev)
    wd, ws = oracle.mxfp4_to_mxfp8_col(bits)
    wrd, wrs = oracle.mxfp4_to_mxfp8_row(bits)
    flag = torch.ones(1, dtype=torch.int32, device=dev)
    cd = torch.full((96, 1024), 0x11, dtype=torch.uint8, device=dev)
    cs = torch.full((3, 1024), 0x22, dtype=torch.uint8, device=dev)
    rd = torch.full((96, 1024), 0x33, dtype=torch.uint8, device=dev)
    rs = torch.full((96, 32), 0x44, dtype=torch.uint8, device=dev)
    cd2 = torch.full((96, 1024), 0x55, dtype=torch.uint8, device=dev)
    cs2 = torch.full((3, 1024), 0x66, dtype=torch.uint8, device=dev)
    mxq.mxq_mxfp4_to_mxfp8_col(x, cd, cs, noop=flag)
    mxq.mxq_mxfp4_to_mxfp8_row_col(x, rd, rs, cd2, cs2, noop=flag)
    for t, v in ((cd, 0x11), (cs, 0x22), (rd, 0x33), (rs, 0x44), (cd2, 0x55), (cs2, 0x66)):
        assert (to_host(t) == v).all()
    flag.zero_()
    mxq.mxq_mxfp4_to_mxfp8_col(x, cd, cs, noop=flag)
    mxq.mxq_mxfp4_to_mxfp8_row_col(x, rd, rs, cd2, cs2, noop=flag)
    assert_bits(to_host(cd), wd, "gated column payload")
    assert_bits(to_host(cs), ws, "gated column codes")
    assert_bits(to_host(cd2), wd, "gated row + column: column payload")
    assert_bits(to_host(cs2), ws, "gated row + column: column codes")
    assert_bits(to_host(rd), wrd, "gated row + column: row payload")
    assert_bits(to_host(rs), wrs, "gated row + column: row codes")


def test_col_noop_flag_inside_a_replayed_graph(dev):
    """The row + column update captured in a graph and replayed with the flag
    set and clear, the weight changed eagerly in between; every replay checked."""
    a_bits = W.c4_headline(shape=(128, 2048))
    b_bits = np.ascontiguousarray(np.tile(W.c1_small()[:, :32], (2, 64))[:128, :2048])
    x = to_dev(a_bits, dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    rd = torch.empty((128, 2048), dtype=torch.uint8, device=dev)
    rs = torch.empty((128, 64), dtype=torch.uint8, device=dev)
    cd = torch.empty((128, 2048), dtype=torch.uint8, device=dev)
    cs = torch.empty((4, 2048), dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm up outside the graph
        mxq.mxq_mxfp4_to_mxfp8_row_col(x, rd, rs, cd, cs, noop=flag)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mxq.mxq_mxfp4_to_mxfp8_row_col(x, rd, rs, cd, cs, noop=flag)
    want = {n: oracle.mxfp4_to_mxfp8_row(b) + oracle.mxfp4_to_mxfp8_col(b) for n, b in (("a", a_bits), ("b", b_bits))}
    for step, (src, skip, expect) in enumerate([("a", 0, "a"), ("b", 1, "a"), ("b", 0, "b"), ("a", 1, "b"),
                                                ("a", 0, "a")]):
        x.copy_(to_dev(a_bits if src == "a" else b_bits, dev))
        flag.fill_(skip)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        wrd, wrs, wcd, wcs = want[expect]
        assert_bits(to_host(rd), wrd, f"replay {step} row payload")
        assert_bits(to_host(rs), wrs, f"replay {step} row codes")
        assert_bits(to_host(cd), wcd, f"replay {step} column payload")
        assert_bits(to_host(cs), wcs, f"replay {step} column codes")
