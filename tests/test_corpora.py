"""The seeded corpora hold what the parity tests rely on (no quantization
arithmetic: only exact float64 views of the bits).

Page: "[PyTorch] MXFP4 weight QAT on MXFP8 and FP8 block-scaling recipes",
section Test results (B200) -- the projection kernel was checked on every RTNE
midpoint, the 2^-128 tie, the subnormal ladder and the 1.5*2^k +- 1 ulp
triples; the fp32 corpora must put each of those in front of the kernels."""
import numpy as np
import pytest

import workloads as W


@pytest.fixture(scope="module")
def pairs_fp32():
    return W.value_exponent_pairs("fp32")


def _blocks_and_scale(bits):
    b = bits.reshape(-1, 32)
    v = b.view(np.float32).astype(np.float64)
    scale = v[:, 0] / 6.0                                  # each block's first element is its amax 6 * 2^e
    return b, v, scale


def test_fp32_pairs_hold_every_tie_at_every_exponent(pairs_fp32):
    """Every E2M1 midpoint, exactly, at every block exponent e in [-126, 125]
    and both signs: 7 x 252 x 2 = 3528 exact ties (only the 0x0000 low half can
    sit on a midpoint, so there are no others)."""
    b, v, scale = _blocks_and_scale(pairs_fp32)
    ok = scale > 0
    t = np.abs(v[ok]) / scale[ok, None]                    # exact: a power-of-two scaling in float64
    ties = np.isin(t, W.MIDPOINTS)
    assert ties.sum() == 3528
    e = np.repeat(np.log2(scale[ok]).astype(np.int64)[:, None], 32, axis=1)[ties]
    key = (e + 1000) * 64 + np.searchsorted(W.MIDPOINTS, t[ties]) * 2 + (v[ok][ties] < 0)
    assert len(np.unique(key)) == 3528                     # each (e, midpoint, sign) once
    assert set(np.unique(e).tolist()) == set(range(-126, 126))


def test_fp32_pairs_hold_the_neighbours_of_every_midpoint(pairs_fp32):
    """For every e and midpoint m: the fp32 values one ulp below and above
    m * 2^e occur in a block whose scale exponent is e."""
    b, v, scale = _blocks_and_scale(pairs_fp32)
    e = np.where(scale > 0, np.log2(np.where(scale > 0, scale, 1.0)), -999).astype(np.int64)
    have = np.unique(((np.repeat(e, 32) + 1000) << 32) | (b.reshape(-1) & 0x7FFFFFFF).astype(np.int64))
    want = []
    for ee in range(-126, 126):
        for m in W.MIDPOINTS:
            mid = int(W.fp32_bits_of(np.ldexp(m, ee)))
            want += [((ee + 1000) << 32) | (mid - 1), ((ee + 1000) << 32) | (mid + 1)]
    assert np.isin(np.array(want, dtype=np.int64), have).all()


def test_fp32_planted_edges():
    p = W.c2_planted_fp32()
    assert p.shape == (160, 32) and p.dtype == np.uint32
    flat = set(p.reshape(-1).tolist())
    ladder = [int(W.fp32_bits_of(np.ldexp(1.0, -127 - i))) for i in range(23)]
    assert set(ladder) <= flat and 0x00000001 in flat and 0x00200000 in flat      # down to 2^-149; 2^-128
    for k in (-148, -127, -126, 0, 127):
        b = int(W.fp32_bits_of(np.ldexp(1.5, k)))
        assert {b - 1, b, b + 1} <= flat
    assert {0x7F400000, 0x7F400001, 0x7F7FFFFF, 0xFF7FFFFF} <= flat                # the cap .. FLT_MAX
    assert {0x7F800000, 0xFF800000, 0x7F800001, 0xFFC00000, 0x7FFFFFFF} <= flat    # Inf and NaNs
    # the bf16 edge rows, widened exactly
    assert np.array_equal(p[:64], W.c2_planted().astype(np.uint32) << 16)
