"""The grouped entry points (row lift, projection, 128x128 fold and decode)
against the oracle: mixed ragged shapes in one call, padded scale storage left
untouched, misaligned operands (the per-weight path), empty weights, more
weights than one launch's table holds, and overlaps across weights refused."""
import numpy as np
import pytest
import torch

import microscaling_weight_quantization_amd as mxq
import oracle
import workloads as W

from .test_gpu_parity import THREADS, assert_bits, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def _weight(rows, K, dtype, seed):
    if dtype == "bf16":
        return W.c4_headline(seed=seed, shape=(rows, K)) if rows * K else np.zeros((rows, K), np.uint16)
    flat = W.fp32_fuzz(((rows * K + 31) // 32) * 32 + 32, seed=seed).reshape(-1)
    return np.ascontiguousarray(flat[: rows * K].reshape(rows, K))


def _check_groups(dev, weights, xs, pads):
    scales = [torch.full((b.shape[0], (b.shape[1] + 31) // 32 + p), 0xA5, dtype=torch.uint8, device=dev)
              for b, p in zip(weights, pads)]
    datas, scales = mxq.mxq_mxfp4_to_mxfp8_row_grouped(xs, scales=scales)
    for i, (bits, d, s, p) in enumerate(zip(weights, datas, scales, pads)):
        rows, K = bits.shape
        if rows * K == 0:
            continue
        wd, ws = oracle.mxfp4_to_mxfp8_row(bits, scale_ld=(K + 31) // 32 + p, threads=THREADS, fill=0xA5)
        assert_bits(to_host(d), wd, f"group {i} ({rows}x{K}) payload")
        assert_bits(to_host(s), ws, f"group {i} ({rows}x{K}) codes, padding untouched")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_grouped_mixed_shapes(dev, dtype):
    shapes = [(100, 48), (257, 1000), (64, 4096), (1, 33), (300, 2048), (0, 64), (128, 130), (33, 7), (513, 256)]
    weights = [_weight(r, k, dtype, 40 + i) for i, (r, k) in enumerate(shapes)]
    xs = [to_dev(b, dev) if b.size else torch.empty(b.shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                                                   device=dev) for b in weights]
    _check_groups(dev, weights, xs, pads=[i % 5 for i in range(len(shapes))])


def test_grouped_with_a_misaligned_weight(dev):
    """A weight that is a view one element into its storage cannot take the
    16-byte path; the call converts it on its own and the rest grouped."""
    weights = [_weight(96, 512, "bf16", 60), _weight(70, 300, "bf16", 61), _weight(128, 256, "bf16", 62)]
    base = to_dev(np.concatenate([np.zeros((70, 1), np.uint16), weights[1]], axis=1), dev)
    xs = [to_dev(weights[0], dev), base[:, 1:], to_dev(weights[2], dev)]
    assert xs[1].data_ptr() % 16 != 0
    _check_groups(dev, weights, xs, pads=[0, 3, 1])


def test_grouped_more_weights_than_one_table(dev):
    """130 weights: several launches' worth of tables; every output equals the
    single-weight call and the oracle."""
    rng = np.random.default_rng(70)
    weights = []
    for i in range(130):
        rows, K = int(rng.integers(1, 200)), int(rng.choice([32, 64, 96, 200, 512, 1024, 1500]))
        weights.append(_weight(rows, K, "bf16", 100 + i))
    xs = [to_dev(b, dev) for b in weights]
    _check_groups(dev, weights, xs, pads=[0] * len(weights))
    for i in (0, 47, 48, 129):
        d1, s1 = mxq.mxq_mxfp4_to_mxfp8_row(xs[i])
        d2, s2 = mxq.mxq_mxfp4_to_mxfp8_row_grouped([xs[i]])
        assert torch.equal(d1, d2[0]) and torch.equal(s1, s2[0])


def test_grouped_overlapping_outputs_are_refused(dev):
    a = to_dev(_weight(64, 256, "bf16", 80), dev)
    b = to_dev(_weight(64, 256, "bf16", 81), dev)
    data = torch.empty((64, 256), dtype=torch.uint8, device=dev)
    with pytest.raises(mxq.MxqError) as e:
        mxq.mxq_mxfp4_to_mxfp8_row_grouped([a, b], datas=[data, data])
    assert e.value.status == mxq.MXQ_ERR_ALIAS
    # the same input twice is fine (inputs may overlap)
    d, s = mxq.mxq_mxfp4_to_mxfp8_row_grouped([a, a])
    assert torch.equal(d[0], d[1]) and torch.equal(s[0], s[1])


def test_prepared_grouped_call_follows_its_weights(dev):
    """GroupedRowLift builds the table once; every call converts the weights'
    current contents."""
    a_bits = [_weight(64, 512, "bf16", 90 + i) for i in range(5)]
    b_bits = [_weight(64, 512, "bf16", 95 + i) for i in range(5)]
    xs = [to_dev(b, dev) for b in a_bits]
    call = mxq.GroupedRowLift(xs, scale_ld=20)
    for bits in (a_bits, b_bits, a_bits):
        for x, b in zip(xs, bits):
            x.copy_(to_dev(b, dev))
        datas, scales = call()
        for i, b in enumerate(bits):
            wd, ws = oracle.mxfp4_to_mxfp8_row(b, scale_ld=20, threads=THREADS)
            assert_bits(to_host(datas[i]), wd, f"weight {i} payload")
            assert_bits(to_host(scales[i])[:, :16], ws[:, :16], f"weight {i} codes")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_grouped_projection_mixed_shapes(dev, dtype):
    """Mixed ragged shapes, one weight converted in place, one misaligned (the
    per-weight path), one empty, and more weights than one table holds."""
    shapes = [(100, 48), (257, 1000), (64, 4096), (1, 33), (300, 2048), (0, 64), (128, 130), (33, 7), (513, 256)]
    shapes += [(int(r), int(k)) for r, k in zip(np.random.default_rng(9).integers(1, 90, 50),
                                                np.random.default_rng(10).choice([32, 64, 200, 512, 1024], 50))]
    weights = [_weight(r, k, dtype, 200 + i) for i, (r, k) in enumerate(shapes)]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xs = [to_dev(b, dev) if b.size else torch.empty(b.shape, dtype=tdt, device=dev) for b in weights]
    base = to_dev(np.concatenate([np.zeros((weights[4].shape[0], 1), weights[4].dtype), weights[4]], axis=1), dev)
    xs[4] = base[:, 1:]                                         # misaligned view
    ys = [None] * len(xs)
    ys[2] = xs[2]                                               # in place
    ys = mxq.mxq_fake_quantize_mxfp4_grouped(xs, ys)
    assert ys[2].data_ptr() == xs[2].data_ptr()
    for i, (bits, y) in enumerate(zip(weights, ys)):
        if bits.size:
            assert_bits(to_host(y), oracle.fake_quantize_mxfp4(bits, threads=THREADS), f"weight {i} {bits.shape}")


def test_prepared_grouped_projection_and_overlaps(dev):
    a_bits = [_weight(64, 512, "bf16", 300 + i) for i in range(4)]
    b_bits = [_weight(64, 512, "bf16", 310 + i) for i in range(4)]
    xs = [to_dev(b, dev) for b in a_bits]
    call = mxq.GroupedProjection(xs)
    for bits in (a_bits, b_bits):
        for x, b in zip(xs, bits):
            x.copy_(to_dev(b, dev))
        for i, (b, y) in enumerate(zip(bits, call())):
            assert_bits(to_host(y), oracle.fake_quantize_mxfp4(b, threads=THREADS), f"weight {i}")
    y = torch.empty_like(xs[0])
    with pytest.raises(mxq.MxqError) as e:
        mxq.mxq_fake_quantize_mxfp4_grouped(xs[:2], [y, y])
    assert e.value.status == mxq.MXQ_ERR_ALIAS


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_grouped_fold_mixed_shapes(dev, dtype):
    """Mixed shapes with partial tiles, one misaligned weight (the per-weight
    path), one empty, a spread-sweep weight, and more weights than one table
    holds; each against the oracle."""
    shapes = [(128, 128), (300, 520), (1, 33), (256, 4096), (0, 64), (129, 129), (64, 2048)]
    shapes += [(int(r), int(k)) for r, k in zip(np.random.default_rng(11).integers(1, 300, 45),
                                                np.random.default_rng(12).choice([32, 128, 200, 512, 640], 45))]
    weights = [_weight(r, k, dtype, 400 + i) for i, (r, k) in enumerate(shapes)]
    spread = W.c3_spread(seed=15, shape=(256, 512))
    weights.append(spread if dtype == "fp32" else np.ascontiguousarray((spread >> 16).astype(np.uint16)))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xs = [to_dev(b, dev) if b.size else torch.empty(b.shape, dtype=tdt, device=dev) for b in weights]
    base = to_dev(np.concatenate([np.zeros((weights[3].shape[0], 1), weights[3].dtype), weights[3]], axis=1), dev)
    xs[3] = base[:, 1:]                                         # misaligned view
    datas, codes = mxq.mxq_mxfp4_to_fp8_block128_grouped(xs)
    for i, (bits, d, c) in enumerate(zip(weights, datas, codes)):
        if bits.size:
            wd, wc = oracle.mxfp4_to_fp8_block128(bits, threads=THREADS)
            assert_bits(to_host(d), wd, f"weight {i} {bits.shape} payload")
            assert_bits(to_host(c), wc, f"weight {i} {bits.shape} tile codes")


def test_prepared_grouped_fold_follows_its_weights(dev):
    a_bits = [_weight(256, 384, "bf16", 500 + i) for i in range(3)]
    b_bits = [_weight(256, 384, "bf16", 510 + i) for i in range(3)]
    xs = [to_dev(b, dev) for b in a_bits]
    call = mxq.GroupedBlock128(xs)
    for bits in (a_bits, b_bits):
        for x, b in zip(xs, bits):
            x.copy_(to_dev(b, dev))
        datas, codes = call()
        for i, b in enumerate(bits):
            wd, wc = oracle.mxfp4_to_fp8_block128(b, threads=THREADS)
            assert_bits(to_host(datas[i]), wd, f"weight {i} payload")
            assert_bits(to_host(codes[i]), wc, f"weight {i} tile codes")


def _decode_inputs(shapes, layout, seed):
    """Random payload bytes (every FP8 pattern, NaNs included) and random E8M0
    codes (0 and 255 included) in the layout's scale shape, with padding
    columns in every scale row (eight for the column layout, whose vector path
    needs a row stride that is a multiple of 8)."""
    rng = np.random.default_rng(seed)
    datas, scales = [], []
    for rows, K in shapes:
        srows = {mxq.MXQ_SCALE_ROW_1X32: rows, mxq.MXQ_SCALE_TILE_128X128: (rows + 127) // 128,
                 mxq.MXQ_SCALE_COL_32X1: (rows + 31) // 32}[layout]
        scols = {mxq.MXQ_SCALE_ROW_1X32: (K + 31) // 32, mxq.MXQ_SCALE_TILE_128X128: (K + 127) // 128,
                 mxq.MXQ_SCALE_COL_32X1: K}[layout]
        datas.append(rng.integers(0, 256, (rows, K), dtype=np.uint8))
        pad = 8 if layout == mxq.MXQ_SCALE_COL_32X1 else 2
        scales.append(rng.integers(0, 256, (srows, scols + pad), dtype=np.uint8))
    return datas, scales


def _to_dev_u8(a, dev):
    # an empty host array can arrive with a non-unit last stride: allocate it instead
    return to_dev(a, dev) if a.size else torch.empty(a.shape, dtype=torch.uint8, device=dev)


@pytest.mark.parametrize("layout", [mxq.MXQ_SCALE_ROW_1X32, mxq.MXQ_SCALE_TILE_128X128, mxq.MXQ_SCALE_COL_32X1])
@pytest.mark.parametrize("fmt", [mxq.MXQ_E4M3, mxq.MXQ_E5M2])
@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
def test_grouped_decode_mixed_shapes(dev, layout, fmt, out_dtype):
    """Mixed ragged shapes in one call, one misaligned payload and one
    misaligned output (the per-payload path), one empty, and more payloads than
    one table holds; each against the oracle."""
    shapes = [(128, 128), (300, 520), (1, 33), (256, 4096), (0, 64), (129, 136), (64, 2048), (40, 4104)]
    shapes += [(int(r), int(k)) for r, k in zip(np.random.default_rng(21).integers(1, 300, 44),
                                                np.random.default_rng(22).choice([8, 32, 128, 200, 512, 640], 44))]
    datas_h, scales_h = _decode_inputs(shapes, layout, 600 + 10 * layout + fmt)
    tdt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    datas = [_to_dev_u8(d, dev) for d in datas_h]
    scales = [_to_dev_u8(s, dev) for s in scales_h]
    r, K = shapes[3]
    base = torch.empty(r * K + 1, dtype=torch.uint8, device=dev)
    base[1:].copy_(datas[3].reshape(-1))
    datas[3] = base[1:].view(r, K)                              # payload not 8-byte aligned
    outs = [torch.empty(d.shape, dtype=tdt, device=dev) for d in datas]
    r, K = shapes[6]
    outs[6] = torch.empty(r * K + 1, dtype=tdt, device=dev)[1:].view(r, K)   # output not 16-byte aligned
    got = mxq.mxq_dequantize_grouped(datas, scales, layout=layout, fmt=fmt, outs=outs)
    code = oracle.BF16 if out_dtype == "bf16" else oracle.FP32
    for i, (d, s, o) in enumerate(zip(datas_h, scales_h, got)):
        if d.size:
            want = oracle.dequantize(d, s, layout=layout, fp8=fmt, out_dtype=code, threads=THREADS)
            assert_bits(to_host(o), want, f"payload {i} {d.shape} layout {layout} fmt {fmt}")


def test_grouped_decode_equals_single_calls_with_padded_outputs(dev):
    """Outputs with a row stride above K: the grouped call writes the same
    bytes as one mxq_dequantize per payload and leaves the padding alone.  The
    last payload is the first one again (inputs may be shared)."""
    shapes = [(200, 256), (64, 1024), (300, 96), (200, 256)]
    datas_h, scales_h = _decode_inputs(shapes, mxq.MXQ_SCALE_ROW_1X32, 31)
    datas = [to_dev(d, dev) for d in datas_h]
    scales = [to_dev(s, dev) for s in scales_h]
    datas[3], scales[3] = datas[0], scales[0]
    big = [torch.full((r, K + 24), 7.0, dtype=torch.bfloat16, device=dev) for r, K in shapes]
    one = [b.clone() for b in big]
    mxq.mxq_dequantize_grouped(datas, scales, outs=[b[:, :K] for b, (_, K) in zip(big, shapes)])
    for d, s, b, (_, K) in zip(datas, scales, one, shapes):
        mxq.mxq_dequantize(d, s, out=b[:, :K])
    for i in range(len(shapes)):
        assert_bits(to_host(big[i]), to_host(one[i]), f"payload {i}")


def test_prepared_grouped_decode_and_overlaps(dev):
    shapes = [(256, 384)] * 3
    a = _decode_inputs(shapes, mxq.MXQ_SCALE_TILE_128X128, 41)
    b = _decode_inputs(shapes, mxq.MXQ_SCALE_TILE_128X128, 42)
    datas = [to_dev(d, dev) for d in a[0]]
    scales = [to_dev(s, dev) for s in a[1]]
    call = mxq.GroupedDequantize(datas, scales, layout=mxq.MXQ_SCALE_TILE_128X128, out_dtype=torch.float32)
    for dh, sh in (a, b):
        for t, h in zip(datas + scales, dh + sh):
            t.copy_(to_dev(h, dev))
        outs = call()
        for i in range(3):
            want = oracle.dequantize(dh[i], sh[i], layout=mxq.MXQ_SCALE_TILE_128X128, out_dtype=oracle.FP32,
                                     threads=THREADS)
            assert_bits(to_host(outs[i]), want, f"payload {i}")
    o = torch.empty((256, 384), dtype=torch.bfloat16, device=dev)
    with pytest.raises(mxq.MxqError) as e:                      # two payloads into one output
        mxq.mxq_dequantize_grouped(datas[:2], scales[:2], layout=mxq.MXQ_SCALE_TILE_128X128, outs=[o, o])
    assert e.value.status == mxq.MXQ_ERR_ALIAS
    buf = torch.empty(2 * 256 * 384, dtype=torch.uint8, device=dev)
    buf[: 256 * 384].copy_(datas[0].reshape(-1))
    with pytest.raises(mxq.MxqError) as e:                      # payload 1's output over payload 0
        mxq.mxq_dequantize_grouped([buf[: 256 * 384].view(256, 384), datas[1]], scales[:2],
                                   layout=mxq.MXQ_SCALE_TILE_128X128,
                                   outs=[o, buf.view(torch.bfloat16).view(256, 384)])
    assert e.value.status == mxq.MXQ_ERR_ALIAS


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_grouped_mxfp4_encode_mixed_shapes(dev, dtype):
    """The packed MXFP4 encode of mixed shapes (odd K included) with padded
    scale storage, one misaligned weight (the per-weight path), one empty, and
    more weights than one table holds; each against the oracle."""
    shapes = [(128, 128), (300, 520), (1, 33), (256, 4096), (0, 64), (129, 129), (64, 2048), (7, 31)]
    shapes += [(int(r), int(k)) for r, k in zip(np.random.default_rng(31).integers(1, 300, 44),
                                                np.random.default_rng(32).choice([32, 64, 200, 512, 641], 44))]
    weights = [_weight(r, k, dtype, 700 + i) for i, (r, k) in enumerate(shapes)]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xs = [to_dev(b, dev) if b.size else torch.empty(b.shape, dtype=tdt, device=dev) for b in weights]
    base = to_dev(np.concatenate([np.zeros((weights[3].shape[0], 1), weights[3].dtype), weights[3]], axis=1), dev)
    xs[3] = base[:, 1:]                                         # misaligned view
    pads = [i % 3 for i in range(len(shapes))]
    scales = [torch.full((r, (k + 31) // 32 + p), 0xA5, dtype=torch.uint8, device=dev)
              for (r, k), p in zip(shapes, pads)]
    packeds, scales = mxq.mxq_quantize_mxfp4_grouped(xs, scales=scales)
    for i, (bits, pk, sc, p) in enumerate(zip(weights, packeds, scales, pads)):
        if bits.size:
            wp, ws = oracle.quantize_mxfp4(bits, scale_ld=(bits.shape[1] + 31) // 32 + p, threads=THREADS,
                                           fill=0xA5)
            assert_bits(to_host(pk), wp, f"weight {i} {bits.shape} nibbles")
            assert_bits(to_host(sc), ws, f"weight {i} {bits.shape} codes")


def test_prepared_grouped_mxfp4_encode_and_overlaps(dev):
    a_bits = [_weight(256, 384, "bf16", 800 + i) for i in range(3)]
    b_bits = [_weight(256, 384, "bf16", 810 + i) for i in range(3)]
    xs = [to_dev(b, dev) for b in a_bits]
    call = mxq.GroupedQuantizeMxfp4(xs)
    for bits in (a_bits, b_bits):
        for x, b in zip(xs, bits):
            x.copy_(to_dev(b, dev))
        packeds, scales = call()
        for i, b in enumerate(bits):
            wp, ws = oracle.quantize_mxfp4(b, threads=THREADS)
            assert_bits(to_host(packeds[i]), wp, f"weight {i} nibbles")
            assert_bits(to_host(scales[i]), ws, f"weight {i} codes")
    p = torch.empty((256, 192), dtype=torch.uint8, device=dev)
    with pytest.raises(mxq.MxqError) as e:                      # two weights into one packed output
        mxq.mxq_quantize_mxfp4_grouped(xs[:2], packeds=[p, p])
    assert e.value.status == mxq.MXQ_ERR_ALIAS
    with pytest.raises(mxq.MxqError) as e:                      # weight 1's codes inside weight 0
        mxq.mxq_quantize_mxfp4_grouped(xs[:2], scales=[None, xs[0].view(torch.uint8)[:, :12]])
    assert e.value.status == mxq.MXQ_ERR_ALIAS
