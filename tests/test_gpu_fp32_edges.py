"""fp32 at its rounding edges: every fp32 entry point against the oracle, bit for bit.

The fp32 instantiations round with the gfx950 scaled conversions of fp32
operands (E2M1 encode of fp32 pairs), which the bf16 corpora never reach.  Two
corpora drive them (page: "[PyTorch] MXFP4 weight QAT on MXFP8 and FP8
block-scaling recipes", section Test results (B200), the projection kernel's
row: every RTNE midpoint, the 2^-128 tie, the subnormal ladder and the
1.5*2^k +- 1 ulp triples):

* ``value_exponent_pairs("fp32")``: every bf16 pattern widened with the low
  halves 0x0000, 0x0001, 0xFFFF and one random low half, placed in blocks whose
  amax is 6*2^e for every e in [-126, 125] -- so every E2M1 midpoint (an exact
  tie) and its neighbours one fp32 ulp either side meet every block exponent;
* ``c2_planted_fp32``: the bf16 edge rows widened exactly plus the fp32-only
  edges (the ladder down to 2^-149, ties at e = -126, 1.5*2^k +- 1 ulp as a
  block's amax, 6*2^125 up to the largest fp32, NaN payloads).

Tolerance 0: every payload byte, code and output bit, NaNs included.
"""
import numpy as np
import pytest
import torch

import microscaling_weight_quantization_amd as mxq
import workloads as W
from tests.test_gpu_col import check_col
from tests.test_gpu_parity import THREADS, assert_bits, check_all, check_packed, to_dev, to_host

import oracle

pytestmark = pytest.mark.gpu

CORPORA = {"pairs_fp32": lambda: W.value_exponent_pairs("fp32"), "planted_fp32": W.c2_planted_fp32}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mxq.load()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def corpora():
    return {name: make() for name, make in CORPORA.items()}


def test_fp32_planted_projection_row_export_decode_fold(dev, corpora):
    """(The pairs corpus takes the same checks in test_gpu_parity's
    test_every_value_at_every_block_exponent.)"""
    bits = corpora["planted_fp32"]
    check_all(bits, dev, scale_ld=(bits.shape[1] + 31) // 32 + 3)


@pytest.mark.parametrize("name", list(CORPORA))
def test_fp32_edges_fused_projection_and_row_lift(dev, corpora, name):
    bits = corpora[name]
    rows, K = bits.shape
    nb = (K + 31) // 32
    x = to_dev(bits, dev)
    scale = torch.full((rows, nb + 2), 0x5A, dtype=torch.uint8, device=dev)
    y, data, scale = mxq.mxq_fake_quantize_mxfp4_with_mxfp8_row(x, scale=scale)
    wd, ws = oracle.mxfp4_to_mxfp8_row(bits, scale_ld=nb + 2, threads=THREADS, fill=0x5A)
    assert_bits(to_host(y), oracle.fake_quantize_mxfp4(bits, threads=THREADS), "fused projection")
    assert_bits(to_host(data), wd, "fused payload")
    assert_bits(to_host(scale), ws, "fused codes")


@pytest.mark.parametrize("name", list(CORPORA))
def test_fp32_edges_columnwise_and_row_col(dev, corpora, name):
    check_col(corpora[name], dev, pad=2)


def test_fp32_planted_packed_mxfp4(dev, corpora):
    """Encode (ties included), decode, and the row lift and fold from packed.
    (The pairs corpus takes the same checks in test_gpu_parity's test_packed_mxfp4.)"""
    bits = corpora["planted_fp32"]
    check_packed(bits, dev, scale_ld=(bits.shape[1] + 31) // 32 + 1)


def test_fp32_edges_grouped_calls(dev, corpora):
    """The grouped projection, row lift, fold, decode and packed encode run the
    single kernels' bodies; the planted rows and slices of the pairs corpus as
    a list of weights of mixed heights."""
    pairs = corpora["pairs_fp32"]
    weights = [corpora["planted_fp32"], np.ascontiguousarray(pairs[:3000]), np.ascontiguousarray(pairs[3000:3131]),
               np.ascontiguousarray(pairs[-257:])]
    xs = [to_dev(b, dev) for b in weights]
    ys = mxq.mxq_fake_quantize_mxfp4_grouped(xs)
    datas, scales = mxq.mxq_mxfp4_to_mxfp8_row_grouped(xs)
    bdatas, tcs = mxq.mxq_mxfp4_to_fp8_block128_grouped(xs)
    decs = mxq.mxq_dequantize_grouped(datas, scales, out_dtype=torch.float32)
    packeds, pscales = mxq.mxq_quantize_mxfp4_grouped(xs)
    for i, bits in enumerate(weights):
        wd, ws = oracle.mxfp4_to_mxfp8_row(bits, threads=THREADS)
        assert_bits(to_host(ys[i]), oracle.fake_quantize_mxfp4(bits, threads=THREADS), f"weight {i} projection")
        assert_bits(to_host(datas[i]), wd, f"weight {i} row payload")
        assert_bits(to_host(scales[i]), ws, f"weight {i} row codes")
        wbd, wtc = oracle.mxfp4_to_fp8_block128(bits, threads=THREADS)
        assert_bits(to_host(bdatas[i]), wbd, f"weight {i} 128x128 payload")
        assert_bits(to_host(tcs[i]), wtc, f"weight {i} tile codes")
        assert_bits(to_host(decs[i]), oracle.dequantize(wd, ws, out_dtype=oracle.FP32, threads=THREADS),
                    f"weight {i} decode")
        wp, wps = oracle.quantize_mxfp4(bits, threads=THREADS)
        assert_bits(to_host(packeds[i]), wp, f"weight {i} packed nibbles")
        assert_bits(to_host(pscales[i]), wps, f"weight {i} packed codes")
