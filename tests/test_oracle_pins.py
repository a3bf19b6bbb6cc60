"""Pins for the CPU oracle (no GPU).

The oracle (``oracle/mxq_oracle.c``) is checked against things other than
itself: the values the pages state (``tests/golden/pages_facts.json``), closed
forms derived by hand from the E4M3 / bf16 bit layouts, library routines
(torch's float8 and bfloat16 casts), invariants the pages claim (decode of the
direct conversions reproduces the projection), and an exact-rational brute
force (``tests/frac_ref.py``) on exhaustive small inputs.  The mutation tests
plant plausible mistakes in the brute force and show the pins catch them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import frac_ref as F

BF16, FP32 = oracle.BF16, oracle.FP32


def bf16_bits(v: float) -> int:
    return int(W.bf16_bits_of(v))


# ---------------------------------------------------------------- decoding and rounding

def test_unpack_matches_numpy_and_torch():
    """Bit decoding against numpy's fp32 view (bf16) and torch's float8 dtypes."""
    for b in range(0, 65536, 7):
        neg, M, k, cls = oracle.unpack(b, oracle.FMT_BF16)
        ref = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
        if np.isnan(ref):
            assert cls == 2
        elif np.isinf(ref):
            assert cls == 1
        else:
            assert cls == 0 and (-1) ** neg * Fraction(M) * Fraction(2) ** k == Fraction(float(ref))
    for fmt, tdt in ((oracle.FMT_E4M3, torch.float8_e4m3fn), (oracle.FMT_E5M2, torch.float8_e5m2)):
        vals = torch.arange(256, dtype=torch.uint8).view(tdt).to(torch.float64).numpy()
        for b in range(256):
            neg, M, k, cls = oracle.unpack(b, fmt)
            if np.isnan(vals[b]):
                assert cls == 2
            elif np.isinf(vals[b]):
                assert cls == 1
            else:
                assert cls == 0 and (-1) ** neg * Fraction(M) * Fraction(2) ** k == Fraction(float(vals[b]))


def _fp32_samples(n, seed):
    g = np.random.default_rng(seed)
    bits = g.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    return bits[np.isfinite(bits.view(np.float32))]


def test_round_to_bf16_matches_torch_cast():
    """Nearest-even rounding into bf16 equals torch's fp32 -> bf16 cast
    (a library routine), including subnormals and overflow to Inf."""
    bits = np.concatenate([_fp32_samples(20000, 1),
                           np.arange(0, 1 << 20, 97, dtype=np.uint32),            # fp32 subnormals
                           np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x007F8000, 0x00008000], dtype=np.uint32)])
    ref = torch.from_numpy(bits.view(np.float32).copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for b, r in zip(bits, ref):
        neg, M, k, cls = oracle.unpack(int(b), oracle.FMT_FP32)
        got, _, _ = oracle.round_to_format(neg, M, k, oracle.FMT_BF16)
        assert got == r, hex(b)


def test_round_to_e4m3_matches_torch_cast():
    """Nearest-even rounding into E4M3 (subnormals included) equals torch's
    fp32 -> float8_e4m3fn cast on every value inside E4M3's range."""
    g = np.random.default_rng(2)
    mags = np.concatenate([np.ldexp(g.random(30000), g.integers(-14, 9, 30000)),
                           np.arange(0, 2 ** -5, 2 ** -13), np.array([448.0, 447.0, 2 ** -10, 3 * 2 ** -11])])
    mags = mags[mags <= 448].astype(np.float32)
    vals = np.concatenate([mags, -mags])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for v, r in zip(vals.view(np.uint32), ref):
        neg, M, k, cls = oracle.unpack(int(v), oracle.FMT_FP32)
        got, _, ovf = oracle.round_to_format(neg, M, k, oracle.FMT_E4M3)
        assert not ovf and got == r, hex(v)


# ---------------------------------------------------------------- the scale exponent

def test_scale_exponent_exhaustive_bf16_vs_brute_force(facts):
    lo, hi = facts["scale_exponent_clamp"]["value"]
    seen = set()
    for b in range(0x7F80):
        e = oracle.scale_exponent_bits(b, BF16)
        assert e == F.scale_exponent(F.bf16_value(b)), hex(b)
        seen.add(e)
    assert min(seen) == lo and max(seen) == hi


def test_scale_exponent_fp32_fuzz_vs_brute_force():
    for b in _fp32_samples(20000, 3):
        b = int(b) & 0x7FFFFFFF
        assert oracle.scale_exponent_bits(b, FP32) == F.scale_exponent(F.fp32_value(b)), hex(b)


@pytest.mark.parametrize("k", [-124, -60, -3, -1, 0, 1, 2, 60, 126])
def test_one_point_five_times_two_to_k_triples(k):
    """amax = 1.5*2^k gives amax/6 = 2^(k-2) exactly: e = k-2 there and one ulp
    below, and e flips to k-1 one ulp above (clamped at 125)."""
    b = bf16_bits(np.ldexp(1.5, k))
    assert oracle.scale_exponent_bits(b, BF16) == max(-126, min(125, k - 2))
    assert oracle.scale_exponent_bits(b - 1, BF16) == max(-126, min(125, k - 2))
    assert oracle.scale_exponent_bits(b + 1, BF16) == max(-126, min(125, k - 1))
    f = int(np.array(np.ldexp(1.5, k), dtype=np.float32).view(np.uint32))
    assert oracle.scale_exponent_bits(f + 1, FP32) == max(-126, min(125, k - 1))
    assert oracle.scale_exponent_bits(f, FP32) == max(-126, min(125, k - 2))


# ---------------------------------------------------------------- E2M1 rounding

GRID = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
# ties go to the neighbour with the even 3-bit code
TIE_RESULT = {0.25: 0, 0.75: 1, 1.25: 1, 1.75: 2, 2.5: 2, 3.5: 4, 5: 4}


@pytest.mark.parametrize("e", [-126, -122, -121, 0, 125])
def test_e2m1_grid_points_and_midpoints(e, facts):
    assert facts["e2m1_grid"]["value"] == GRID
    for c, p in enumerate(GRID):
        if p:
            assert oracle.e2m1_code_bits(bf16_bits(np.ldexp(p, e)), e) == c
    for mid, want in TIE_RESULT.items():
        b = bf16_bits(np.ldexp(mid, e))
        assert GRID[oracle.e2m1_code_bits(b, e)] == want
        below, above = max(x for x in GRID if x < mid), min(x for x in GRID if x > mid)
        assert GRID[oracle.e2m1_code_bits(b - 1, e)] == below
        assert GRID[oracle.e2m1_code_bits(b + 1, e)] == above


def test_e2m1_codes_exhaustive_vs_brute_force():
    for e in (-126, -125, -124, -3, 0, 7, 125):
        for b in range(0, 0x7F80, 3):
            t = F.bf16_value(b) / Fraction(2) ** e
            assert oracle.e2m1_code_bits(b, e) == F.e2m1_code(t), (hex(b), e)


# ---------------------------------------------------------------- projection edge cases

def test_subnormal_ladder():
    """In a block whose scale is 2^-126: 2^-127 stays, 2^-128 is the tie and goes
    to +0, 2^-129 .. 2^-133 go to 0."""
    ladder = [bf16_bits(np.ldexp(1.0, -127 - i)) for i in range(7)]
    x = np.array([ladder + [0] * 25], dtype=np.uint16)
    y = oracle.fake_quantize_mxfp4(x)[0]
    assert y[0] == 0x0040 and all(v == 0 for v in y[1:7])
    x = np.array([[bf16_bits(2.0 ** -128)] * 32], dtype=np.uint16)
    assert oracle.fake_quantize_mxfp4(x)[0].tolist() == [0] * 32


def test_saturation_at_the_cap(facts):
    assert facts["saturation_cap"]["value"] == "6*2^125"
    cap = bf16_bits(6 * 2.0 ** 125)
    assert cap == 0x7F40
    x = np.array([list(range(0x7F41, 0x7F61))], dtype=np.uint16)
    assert set(oracle.fake_quantize_mxfp4(x)[0].tolist()) == {0x7F40}
    x = np.array([list(range(0xFF60, 0xFF80))], dtype=np.uint16)
    assert set(oracle.fake_quantize_mxfp4(x)[0].tolist()) == {0xFF40}
    data, scale = oracle.mxfp4_to_mxfp8_row(x)
    assert scale[0, 0] == 125 + 121 and set(data[0].tolist()) == {0xFC}


@pytest.mark.parametrize("bad", [0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0xFFFF])
def test_non_finite_block_poisoning(bad):
    x = np.array([[0x3F80] * 31 + [bad] + [0x3F80] * 32], dtype=np.uint16)
    y = oracle.fake_quantize_mxfp4(x)[0]
    assert set(y[:32].tolist()) == {0x7FC0} and set(y[32:].tolist()) == {0x3F80}
    data, scale = oracle.mxfp4_to_mxfp8_row(x)
    assert scale[0].tolist() == [255, -2 + 121]          # a block of ones has e = -2
    assert set(data[0, :32].tolist()) == {0x7F}
    out = oracle.dequantize(data, scale)
    assert set(out[0, :32].tolist()) == {0x7FC0} and set(out[0, 32:].tolist()) == {0x3F80}


def test_negative_zero_kept():
    x = np.array([[0x8000, 0x0000, bf16_bits(-2.0 ** -10), bf16_bits(6.0)] + [0] * 28], dtype=np.uint16)
    y = oracle.fake_quantize_mxfp4(x)[0]
    assert y[0] == 0x8000 and y[1] == 0 and y[2] == 0x8000
    data, _ = oracle.mxfp4_to_mxfp8_row(x)
    assert data[0, 0] == 0x80 and data[0, 2] == 0x80


# ---------------------------------------------------------------- direct row lift

ROW_TABLE = {0: 0x00, 0.5: 0x60, 1: 0x68, 1.5: 0x6C, 2: 0x70, 3: 0x74, 4: 0x78, 6: 0x7C}


def test_row_payload_closed_table(facts):
    """p * 2^6 in E4M3 (bias 7, 3 mantissa bits) written out by hand; below
    e = -121 the scale sits at code 0 and the payload absorbs the shift, which
    lowers its exponent field by 6 - shift, i.e. the byte by 8*(6 - shift)."""
    assert facts["row_fixed_shift"]["value"] == 6
    for e in range(-126, 126):
        shift = min(6, e + 127)
        for p, byte in ROW_TABLE.items():
            for sign in (1, -1):
                vals = [6.0, sign * float(p)] + [0.0] * 30
                x = np.array([W.bf16_bits_of(np.ldexp(np.array(vals), e))], dtype=np.uint16)
                data, scale = oracle.mxfp4_to_mxfp8_row(x)
                assert scale[0, 0] == max(e + 121, 0)
                want = 0 if p == 0 else byte - 8 * (6 - shift)
                if sign < 0:
                    want |= 0x80
                assert data[0, 1] == want, (e, p, sign)
                assert data[0, 0] == ROW_TABLE[6] - 8 * (6 - shift)


def test_code_zero_and_255_decode(facts):
    assert facts["e8m0_code0"]["value"] == "2^-127" and facts["e8m0_code255"]["value"] == "NaN"
    data = np.array([[0x38, 0xB8, 0x01, 0x7E]], dtype=np.uint8)       # 1.0, -1.0, 2^-9, 448
    scale = np.array([[0]], dtype=np.uint8)
    f32 = oracle.dequantize(data, scale, out_dtype=FP32)[0]
    assert f32[0] == 0x00400000 and f32[1] == 0x80400000            # 2^-127 exactly
    assert f32[2] == 1 << (149 - 136)                                # 2^-136, an fp32 subnormal
    assert oracle.dequantize(data, scale, out_dtype=BF16)[0][:3].tolist() == [0x0040, 0x8040, 0x0000]
    nan = oracle.dequantize(data, np.array([[255]], dtype=np.uint8), out_dtype=BF16)[0]
    assert set(nan.tolist()) == {0x7FC0}
    # a block of 2^-127: e = -126, E8M0 code 0, payload 1.0 (0x38), decoding to 2^-127
    x = np.array([[0x0040] * 32], dtype=np.uint16)
    d, s = oracle.mxfp4_to_mxfp8_row(x)
    assert s[0, 0] == 0 and set(d[0].tolist()) == {0x38}
    assert set(oracle.dequantize(d, s)[0].tolist()) == {0x0040}


def _same_bits_nan_canonical(a, b):
    return np.array_equal(a, b)


CORPORA = {
    "c1": lambda: W.c1_small(),
    "c2_shuffled": lambda: W.c2_exhaustive(),
    "c2_natural": lambda: W.c2_exhaustive(natural=True),
    "c2_planted": lambda: W.c2_planted(),
}


@pytest.mark.parametrize("name", list(CORPORA))
def test_decode_of_row_lift_is_the_projection(name):
    """The pages: rowwise MXFP8 bytes decode back to the projected weight
    exactly, including 2^-127 at code 0; poisoned blocks decode to NaN."""
    x = CORPORA[name]()
    y = oracle.fake_quantize_mxfp4(x)
    data, scale = oracle.mxfp4_to_mxfp8_row(x)
    assert np.array_equal(oracle.dequantize(data, scale), y)
    assert np.array_equal(oracle.dequantize(data, scale, out_dtype=FP32), (y.astype(np.uint32) << 16))


def test_decode_of_row_lift_is_the_projection_fp32():
    x = W.fp32_fuzz(1 << 15)
    y = oracle.fake_quantize_mxfp4(x)
    data, scale = oracle.mxfp4_to_mxfp8_row(x)
    assert np.array_equal(oracle.dequantize(data, scale, out_dtype=FP32), y)


def test_exhaustive_corpus_block_count(facts):
    """Natural order: 2036 of 2048 blocks are finite and below saturation."""
    fact = facts["exhaustive_finite_below_saturation_blocks"]
    x = W.c2_exhaustive(natural=True)
    data, scale = oracle.mxfp4_to_mxfp8_row(x)
    finite = scale[:, 0] != 255
    mags = (x & 0x7FFF).astype(np.int64)
    below_cap = (mags <= 0x7F40).all(axis=1)
    assert x.shape[0] == fact["of"]
    assert int((finite & below_cap).sum()) == fact["value"]


# ---------------------------------------------------------------- 128x128 folding

def spread_row(d: int, base: int, sign_flip: bool = False) -> np.ndarray:
    """One 128-wide tile row: block 0 at exponent base holds 6 and every +-grid
    point and midpoint, block 1 sets the tile maximum base+d, blocks 2-3 are the
    low block negated / shifted."""
    low = [6.0] + [s * p for p in GRID for s in (1, -1)] + [s * m for m in TIE_RESULT for s in (1, -1)] + [-6.0]
    low = np.ldexp(np.array(low), base)
    high = np.ldexp(np.array([6.0] + [0.5] * 31), base + d)
    row = np.concatenate([low, high, -low, np.ldexp(np.array(GRID * 4), base)])
    return row


def _fp32_bits_of(v):
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(v, dtype=np.float64))
    return f.view(np.uint32)


def test_block128_exactness_boundary(facts):
    """decode(blockwise bytes) equals the projection for every tile whose block
    exponents spread by at most 2^14; at 2^15 the first values are lost."""
    exact_through = facts["block128_exact_through_log2_spread"]["value"]
    first_loss = facts["block128_first_loss_log2_spread"]["value"]
    for base in (-126, -120, -60, 0, 90):
        row = np.concatenate([spread_row(d, base) for d in range(17)])
        x = _fp32_bits_of(row)[None, :]
        y = oracle.fake_quantize_mxfp4(x)
        data, codes = oracle.mxfp4_to_fp8_block128(x)
        dec = oracle.dequantize(data, codes, layout=oracle.TILE_128X128, out_dtype=FP32)
        for d in range(17):
            sl = slice(128 * d, 128 * d + 128)
            same = np.array_equal(dec[0, sl], y[0, sl])
            if d <= exact_through:
                assert same, (base, d)
            elif base + d - 6 > -127 and d >= first_loss:
                assert not same, (base, d)
            if base + d - 6 <= -127:      # tile clamp at code 0 keeps every value exact
                assert same, (base, d)


def test_block128_closed_form_first_losses():
    """At spread d the low block's p*2^(6-d) lands on E4M3's subnormal step
    2^-9: d = 15 sends 0.5 to 0 (tie) and 1.5 to 2^-8 (tie up to even); d = 16
    sends 0.5, 1 to 0, 1.5 to 2^-9 and 3 to 2^-8; 2, 4, 6 stay exact."""
    base = 0
    for d, want in ((15, {0.5: 0, 1.5: 2.0 ** -8, 1: 2.0 ** -9, 3: 3 * 2.0 ** -9}),
                    (16, {0.5: 0, 1: 0, 1.5: 2.0 ** -9, 3: 2.0 ** -8, 2: 2.0 ** -9, 4: 2.0 ** -8, 6: 3 * 2.0 ** -9})):
        x = _fp32_bits_of(spread_row(d, base))[None, :]
        data, codes = oracle.mxfp4_to_fp8_block128(x)
        assert codes[0, 0] == base + d - 6 + 127
        vals = torch.from_numpy(data[0, :32].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        lowvals = [6.0] + [s * p for p in GRID for s in (1, -1)]
        for i, v in enumerate(lowvals):
            p = abs(v)
            if p in want:
                assert abs(vals[i]) == want[p], (d, p, vals[i])


def test_block128_tile_clamp():
    """M < -121 puts the tile scale at code 0 and the payload takes e + 127."""
    row = np.concatenate([spread_row(d, -126) for d in range(5)])
    x = _fp32_bits_of(row)[None, :]
    data, codes = oracle.mxfp4_to_fp8_block128(x)
    assert codes[0].tolist() == [0] * 5


def test_block128_poisoned_and_zero_tiles():
    x = np.zeros((128, 256), dtype=np.uint16)
    x[5, 3] = 0x7FC0                        # tile 0: one poisoned block, rest zero
    x[:, 128:] = 0x3F80                     # tile 1: all ones
    x[0, 200] = 0x7F80                      # ... with one poisoned block
    data, codes = oracle.mxfp4_to_fp8_block128(x)
    assert codes[0, 0] == 0                               # no finite nonzero block: M = -126
    assert set(data[5, 0:32].tolist()) == {0x7F}
    assert codes[0, 1] == (-2 - 6 + 127)                   # e of a block of ones is -2
    assert set(data[0, 192:224].tolist()) == {0x7F}


# ---------------------------------------------------------------- export

def test_export_shapes(facts):
    assert facts["export_scale_shape_100x48"]["value"] == [100, 2]
    x = W.c1_small()
    data, scale = oracle.mxfp4_to_mxfp8_row(x, scale_ld=4, fill=0xAB)
    out = oracle.export_mxfp8(scale, 48)
    assert list(out.shape) == [100, 2] and np.array_equal(out, scale[:, :2])
    assert (scale[:, 2:] == 0xAB).all()                   # padding never written
    x16 = W.c1_small()[:, :16].copy()
    d16, s16 = oracle.mxfp4_to_mxfp8_row(x16, scale_ld=4)
    assert oracle.export_mxfp8(s16, 16).shape == (100, facts["export_scale_cols_K16"]["value"])


@pytest.mark.parametrize("K,partial", [(48, True), (16, True), (80, True), (33, True), (32, False), (64, False),
                                       (256, False)])
def test_export_floor_mutation_breaks_exactly_the_partial_block_shapes(K, partial):
    """[EXP] Testing: taking the scale width as K // 32 instead of ceil(K/32)
    breaks the partial-block layouts -- the (100, 48) tensor and K = 16 -- and
    leaves every K that is a multiple of 32 unchanged.  The exported scales of
    each shape, built by the oracle, against the mutated export."""
    rows = 100 if K == 48 else 7
    x = np.ascontiguousarray(np.tile(W.c1_small()[:rows], (1, K // 48 + 1))[:, :K])
    _, scale = oracle.mxfp4_to_mxfp8_row(x, scale_ld=((K + 31) // 32 + 3) // 4 * 4)
    good = oracle.export_mxfp8(scale, K)
    assert good.shape == (rows, (K + 31) // 32)
    assert np.array_equal(good, F.export(scale, K))
    bad = F.export(scale, K, mutation="floor_cols")
    assert (bad.shape != good.shape) == partial
    if partial:
        assert bad.shape[1] == K // 32 < good.shape[1]    # the partial last block loses its scale
    else:
        assert np.array_equal(bad, good)


# ---------------------------------------------------------------- oracle vs brute force

@pytest.mark.parametrize("name", ["c1", "c2_shuffled", "c2_natural", "c2_planted"])
def test_oracle_matches_brute_force_bf16(name):
    x = CORPORA[name]()
    assert np.array_equal(oracle.fake_quantize_mxfp4(x), F.fake_quantize(x, "bf16"))
    d0, s0 = oracle.mxfp4_to_mxfp8_row(x)
    d1, s1 = F.row_lift(x, "bf16")
    assert np.array_equal(d0, d1) and np.array_equal(s0, s1)


def test_oracle_matches_brute_force_fp32():
    x = W.fp32_fuzz(1 << 13)
    assert np.array_equal(oracle.fake_quantize_mxfp4(x), F.fake_quantize(x, "fp32"))
    d0, s0 = oracle.mxfp4_to_mxfp8_row(x)
    d1, s1 = F.row_lift(x, "fp32")
    assert np.array_equal(d0, d1) and np.array_equal(s0, s1)


def test_oracle_matches_brute_force_fp32_edges():
    """fp32 at its edges -- the ladder 2^-127 .. 2^-149 with the 2^-128 tie,
    midpoints one ulp either side, 1.5*2^k +- 1 ulp as a block's amax down into
    the subnormals, 6*2^125 up to the largest fp32, NaN payloads -- through the
    projection, row lift, fold, columnwise conversion and packed encode,
    against exact rationals ([QAT] Test results (B200), projection kernel row)."""
    x = W.c2_planted_fp32()
    assert np.array_equal(oracle.fake_quantize_mxfp4(x), F.fake_quantize(x, "fp32"))
    d0, s0 = oracle.mxfp4_to_mxfp8_row(x)
    d1, s1 = F.row_lift(x, "fp32")
    assert np.array_equal(d0, d1) and np.array_equal(s0, s1)
    d0, c0 = oracle.mxfp4_to_fp8_block128(x)
    d1, c1 = F.block128(x, "fp32")
    assert np.array_equal(d0, d1) and np.array_equal(c0, c1)
    d0, c0 = oracle.mxfp4_to_mxfp8_col(x)
    d1, c1 = F.col_lift(x, "fp32")
    assert np.array_equal(d0, d1) and np.array_equal(c0, c1)
    p0, s0 = oracle.quantize_mxfp4(x)
    p1, s1 = F.quantize_mxfp4(x, "fp32")
    assert np.array_equal(p0, p1) and np.array_equal(s0, s1)


def test_oracle_matches_brute_force_on_every_fp32_tie():
    """Every block of the fp32 value x exponent corpus that holds an exact E2M1
    tie (each midpoint at each block exponent, both signs), through the
    projection and the row lift, against exact rationals."""
    b = W.value_exponent_pairs("fp32").reshape(-1, 32)
    v = b.view(np.float32).astype(np.float64)
    scale = v[:, 0] / 6.0
    with np.errstate(invalid="ignore", divide="ignore"):
        t = np.abs(v) / np.where(scale > 0, scale, np.nan)[:, None]
    x = np.ascontiguousarray(b[np.isin(t, W.MIDPOINTS).any(axis=1)])
    assert 1000 < len(x) <= 3528
    assert np.array_equal(oracle.fake_quantize_mxfp4(x), F.fake_quantize(x, "fp32"))
    d0, s0 = oracle.mxfp4_to_mxfp8_row(x)
    d1, s1 = F.row_lift(x, "fp32")
    assert np.array_equal(d0, d1) and np.array_equal(s0, s1)


def test_oracle_matches_brute_force_block128():
    row = np.concatenate([spread_row(d, b) for d in range(17) for b in (-126, -121, 3)])
    x = np.stack([_fp32_bits_of(row), _fp32_bits_of(-row[::-1])])
    d0, c0 = oracle.mxfp4_to_fp8_block128(x)
    d1, c1 = F.block128(x, "fp32")
    assert np.array_equal(d0, d1) and np.array_equal(c0, c1)
    xb = W.c2_planted()[:, :32]
    xb = np.ascontiguousarray(np.tile(xb, (3, 5)))       # 192 x 160: partial tiles both ways
    d0, c0 = oracle.mxfp4_to_fp8_block128(xb)
    d1, c1 = F.block128(xb, "bf16")
    assert np.array_equal(d0, d1) and np.array_equal(c0, c1)


@pytest.mark.parametrize("fp8", ["e4m3", "e5m2"])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_oracle_decode_matches_brute_force_every_byte_and_code(fp8, out):
    data = np.tile(np.arange(256, dtype=np.uint8), (256, 1))          # row r holds every byte
    scale = np.arange(256, dtype=np.uint8).reshape(256, 1).repeat(8, axis=1)   # row r uses code r
    got = oracle.dequantize(data, scale, fp8=oracle.E4M3 if fp8 == "e4m3" else oracle.E5M2,
                            out_dtype=BF16 if out == "bf16" else FP32)
    want = F.dequantize(data, scale, "row", out, fp8)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- mutation sensitivity

@pytest.mark.parametrize("mutation,where", [
    ("clamp_low_127", "proj"),
    ("ties_away", "proj"),
    ("no_absorption", "row"),
    ("tile_clamp_126", "block128"),
])
def test_pins_catch_planted_mistakes(mutation, where):
    """Each planted mistake changes some output the pins compare, so the same
    mistake in the oracle could not pass them."""
    if where == "proj":
        x = W.c2_planted()
        assert not np.array_equal(F.fake_quantize(x, "bf16", mutation), oracle.fake_quantize_mxfp4(x))
    elif where == "row":
        x = W.c2_planted()
        d1, s1 = F.row_lift(x, "bf16", mutation=mutation)
        d0, s0 = oracle.mxfp4_to_mxfp8_row(x)
        assert not (np.array_equal(d0, d1) and np.array_equal(s0, s1))
    else:
        row = np.concatenate([spread_row(d, -126) for d in range(6)])
        x = _fp32_bits_of(row)[None, :]
        d1, c1 = F.block128(x, "fp32", mutation=mutation)
        d0, c0 = oracle.mxfp4_to_fp8_block128(x)
        assert not (np.array_equal(d0, d1) and np.array_equal(c0, c1))


# ---------------------------------------------------------------- packed MXFP4 (deployment)

def _below_cap_blocks(x):
    """[rows, nblocks] mask of finite blocks whose amax is at most 6*2^125."""
    rows, K = x.shape
    nb = (K + 31) // 32
    mask = np.ones((rows, nb), dtype=bool)
    mag = (x & 0x7FFF).astype(np.int64) if x.dtype == np.uint16 else (x & 0x7FFFFFFF).astype(np.int64)
    cap = 0x7F40 if x.dtype == np.uint16 else 0x7F400000
    for j in range(nb):
        mask[:, j] = (mag[:, 32 * j:32 * j + 32] <= cap).all(axis=1)
    return mask


def test_packed_nibble_order_closed_form(facts):
    """0.5, 1, 1.5, -6 at e = 0: E2M1 codes 1, 2, 3, 7|sign; element 2i sits in
    the low nibble of byte i."""
    assert "UE8M0" in facts["deployment_format"]["value"]
    x = W.bf16_bits_of(np.array([0.5, 1.0, 1.5, -6.0] + [0.0] * 28))[None, :]
    packed, scale = oracle.quantize_mxfp4(x)
    assert packed[0, :2].tolist() == [0x21, 0xF3] and scale[0, 0] == 127 + 0
    x3 = W.bf16_bits_of(np.array([1.0, 2.0, 6.0]))[None, :]
    p3, _ = oracle.quantize_mxfp4(x3)
    assert p3.tolist() == [[0x42, 0x07]]                  # odd K: the last high nibble is 0


def test_packed_scale_moves_to_2_126_above_the_cap(facts):
    assert facts["packed_scale_above_cap"]["value"] == "2^126"
    x = np.array([list(range(0x7F41, 0x7F61))], dtype=np.uint16)          # amax above 6*2^125
    packed, scale = oracle.quantize_mxfp4(x)
    assert scale[0, 0] == 126 + 127
    # x / 2^126 lies in (3, 3.5]: p = 3, or 4 from the 3.5 tie on; 4 * 2^126 = 2^128 is
    # unmaterializable in bf16/fp32, so those decode to Inf
    nib = np.stack([packed[0] & 0xF, packed[0] >> 4], axis=1).reshape(-1)
    assert set(nib.tolist()) == {5, 6}
    dec = oracle.dequantize_mxfp4(packed, scale, 32, out_dtype=oracle.FP32).view(np.float32)
    assert all((v == 3 * 2.0 ** 126) if n == 5 else np.isinf(v) for v, n in zip(dec[0], nib))
    x = np.array([[0x7F40] * 32], dtype=np.uint16)                      # exactly the cap: scale 2^125
    assert oracle.quantize_mxfp4(x)[1][0, 0] == 125 + 127


@pytest.mark.parametrize("name", list(CORPORA))
def test_decoded_deployment_weight_is_the_projection(name):
    """[QAT] Description: training sees exactly the deployment weight -- below
    the cap the decoded packed MXFP4 equals the projection bit for bit; the row
    lift and the tile fold from the packed form equal those from the master."""
    x = CORPORA[name]()
    rows, K = x.shape
    packed, scale = oracle.quantize_mxfp4(x)
    ok = np.repeat(_below_cap_blocks(x), 32, axis=1)[:, :K]
    y = oracle.fake_quantize_mxfp4(x)
    dec = oracle.dequantize_mxfp4(packed, scale, K)
    assert np.array_equal(dec[ok], y[ok])
    d0, s0 = oracle.mxfp4_to_mxfp8_row(x)
    d1, s1 = oracle.mxfp4_packed_to_mxfp8_row(packed, scale, K)
    okb = _below_cap_blocks(x)
    assert np.array_equal(d1[ok], d0[ok]) and np.array_equal(s1[okb], s0[okb])


def test_tile_fold_from_packed_equals_fold_from_master():
    row = np.concatenate([spread_row(d, b) for d in range(17) for b in (-126, -121, 3)])
    x = np.stack([_fp32_bits_of(row), _fp32_bits_of(-row[::-1])])
    packed, scale = oracle.quantize_mxfp4(x)
    d0, c0 = oracle.mxfp4_to_fp8_block128(x)
    d1, c1 = oracle.mxfp4_packed_to_fp8_block128(packed, scale, x.shape[1])
    assert np.array_equal(d0, d1) and np.array_equal(c0, c1)


@pytest.mark.parametrize("name", ["c1", "c2_planted", "c2_natural"])
def test_packed_oracle_matches_brute_force(name):
    x = CORPORA[name]()
    K = x.shape[1]
    packed, scale = oracle.quantize_mxfp4(x)
    bp, bs = F.quantize_mxfp4(x, "bf16")
    assert np.array_equal(packed, bp) and np.array_equal(scale, bs)
    assert np.array_equal(oracle.dequantize_mxfp4(packed, scale, K), F.dequantize_mxfp4(packed, scale, K, "bf16"))
    d0, s0 = oracle.mxfp4_packed_to_mxfp8_row(packed, scale, K)
    d1, s1 = F.packed_to_row(packed, scale, K)
    assert np.array_equal(d0, d1) and np.array_equal(s0, s1)


def test_packed_fold_and_decode_every_code_vs_brute_force():
    """Every E8M0 code (0..255) with every nibble, through decode (bf16, fp32),
    the row lift and the tile fold."""
    rows = 256
    packed = np.tile(np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], dtype=np.uint8), (rows, 8))  # K = 128
    scale = np.arange(256, dtype=np.uint8).reshape(rows, 1).repeat(4, axis=1)
    scale[::7, 1] = 3                                   # mixed exponents inside tiles
    K = 128
    for out, odt in (("bf16", oracle.BF16), ("fp32", oracle.FP32)):
        assert np.array_equal(oracle.dequantize_mxfp4(packed, scale, K, out_dtype=odt),
                              F.dequantize_mxfp4(packed, scale, K, out))
    d0, s0 = oracle.mxfp4_packed_to_mxfp8_row(packed, scale, K)
    d1, s1 = F.packed_to_row(packed, scale, K)
    assert np.array_equal(d0, d1) and np.array_equal(s0, s1)
    d0, c0 = oracle.mxfp4_packed_to_fp8_block128(packed, scale, K)
    d1, c1 = F.packed_to_block128(packed, scale, K)
    assert np.array_equal(d0, d1) and np.array_equal(c0, c1)


# ---------------------------------------------------------------- MXFP8 columnwise (32x1)

def _proj_float(x):
    """The projection of x as float64 (NaN for poisoned blocks)."""
    y = oracle.fake_quantize_mxfp4(x)
    if y.dtype == np.uint16:
        return (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return y.view(np.float32).astype(np.float64)


def _col_corpora():
    return {"c1": W.c1_small(), "c2_natural": W.c2_exhaustive(natural=True),
            "c2_planted": W.c2_planted(), "fp32_fuzz": W.fp32_fuzz(1 << 12)}


def test_col_scale_rules_agree_on_projected_magnitudes():
    """Every magnitude the projection can produce (p * 2^e, p on the E2M1 grid,
    e in [-126, 125]) has at most two significant bits, so the OCP rule
    floor(log2 amax) - 8 and the rule ceil(log2(amax / 448)) give the same
    scale, and amax / 2^S (256 or 384) never saturates E4M3.  Off that domain
    the two rules differ (1.875 * 2^k), so the agreement is not vacuous."""
    for e in range(-126, 126):
        for p in F.GRID[1:]:
            v = p * Fraction(2) ** e
            S = F.col_scale(v)
            assert S == F.col_scale(v, "col_rule_448")
            assert v / Fraction(2) ** S <= 384
    v = Fraction(15, 8) * Fraction(2) ** 3
    assert F.col_scale(v) != F.col_scale(v, "col_rule_448")


@pytest.mark.parametrize("name", ["c1", "c2_natural", "c2_planted", "fp32_fuzz"])
def test_col_payload_matches_torch_cast(name):
    """Library pin: per 32x1 block, S from numpy's frexp of the finite amax, the
    payload from torch's float8_e4m3fn cast of y / 2^S (exact in float64), NaN
    elements 0x7F, and codes S + 127."""
    x = _col_corpora()[name]
    data, scale = oracle.mxfp4_to_mxfp8_col(x)
    y = _proj_float(x)
    rows, K = y.shape
    for b0 in range(0, rows, 32):
        blk = y[b0:b0 + 32]
        fin = np.where(np.isnan(blk), 0.0, np.abs(blk))
        amax = fin.max(axis=0)
        _, ex = np.frexp(amax)                                   # amax = m * 2^ex, m in [0.5, 1)
        S = np.where(amax > 0, np.maximum(ex - 1 - 8, -127), -127)
        assert np.array_equal(scale[b0 // 32], (S + 127).astype(np.uint8))
        q = np.ldexp(blk, -S[None, :])
        want = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        want = np.where(np.isnan(blk), 0x7F, want)
        assert np.array_equal(data[b0:b0 + 32], want)


@pytest.mark.parametrize("name", ["c1", "c2_natural", "c2_planted", "fp32_fuzz"])
def test_col_of_projection_equals_col_of_master(name, facts):
    """The pages: the direct columnwise bytes equal the host quantizer's bytes
    for the projected weight.  The bytes depend on the projected values only,
    so quantizing the projection (whose own decomposition may differ) gives
    the same bytes as going from the master weight."""
    assert facts["columnwise_from_decomposition"]["value"]["bytes_equal_projection_route"]
    x = _col_corpora()[name]
    d0, s0 = oracle.mxfp4_to_mxfp8_col(x)
    d1, s1 = oracle.mxfp4_to_mxfp8_col(oracle.fake_quantize_mxfp4(x))
    assert np.array_equal(d0, d1) and np.array_equal(s0, s1)


@pytest.mark.parametrize("name", ["c1", "c2_natural", "fp32_fuzz"])
def test_col_decode_is_exact_exactly_where_e4m3_holds_the_value(name):
    """decode(col(x)) equals the projection at every element whose y / 2^S is
    a multiple of 2^-9 (E4M3's smallest subnormal; it never exceeds 384), and
    differs from it everywhere else.  NaN elements decode to NaN."""
    x = _col_corpora()[name]
    data, scale = oracle.mxfp4_to_mxfp8_col(x)
    y = _proj_float(x)
    back = oracle.dequantize(data, scale, layout=oracle.COL_32X1, out_dtype=FP32).view(np.float32).astype(np.float64)
    S = np.repeat(scale.astype(np.int64) - 127, 32, axis=0)[:y.shape[0]]
    q = np.ldexp(np.nan_to_num(y), -S + 9)
    exact = q == np.round(q)
    nan = np.isnan(y)
    assert np.array_equal(np.isnan(back), nan)
    assert np.array_equal(back[exact & ~nan], y[exact & ~nan])
    assert not np.any(back[~exact & ~nan] == y[~exact & ~nan])


def test_col_special_blocks():
    """Zero blocks get code 0 with signed zero payloads; a column of 2^-127
    gets code 0 and payload 1.0 (0x38); a poisoned row block's elements are
    0x7F and leave the other rows' codes as they are; bands are 32 rows from
    row 0 and the last may be short."""
    tiny = bf16_bits(2.0 ** -127)
    x = np.zeros((40, 64), dtype=np.uint16)
    x[1, :] = 0x8000                                       # -0
    x[:, 32:] = tiny
    data, scale = oracle.mxfp4_to_mxfp8_col(x)
    assert scale.shape == (2, 64) and not scale.any()
    assert set(data[1, :32].tolist()) == {0x80} and set(data[0, :32].tolist()) == {0x00}
    assert set(data[:, 32:].ravel().tolist()) == {0x38}
    g = np.random.default_rng(5)
    zf = (g.standard_normal((40, 64)) * 2.0 ** g.integers(-4, 5, (40, 1))).astype(np.float32)
    z = torch.from_numpy(zf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    d0, s0 = oracle.mxfp4_to_mxfp8_col(z)
    zp = z.copy()
    zp[3, 5] = 0x7FC0                                      # poisons row 3, columns 0..31
    zz = z.copy()
    zz[3, :32] = 0
    d1, s1 = oracle.mxfp4_to_mxfp8_col(zp)
    d2, s2 = oracle.mxfp4_to_mxfp8_col(zz)
    assert set(d1[3, :32].tolist()) == {0x7F}
    assert np.array_equal(s1, s2)
    mask = np.ones_like(d1, dtype=bool)
    mask[3, :32] = False
    assert np.array_equal(d1[mask], d2[mask])
    assert np.array_equal(d0[32:], oracle.mxfp4_to_mxfp8_col(np.ascontiguousarray(z[32:]))[0])


@pytest.mark.parametrize("name", ["c1", "c2_planted", "c2_natural", "fp32_fuzz"])
def test_col_oracle_matches_brute_force(name):
    x = _col_corpora()[name]
    if name == "fp32_fuzz":
        x = np.ascontiguousarray(x[:, :512])
    d0, s0 = oracle.mxfp4_to_mxfp8_col(x)
    d1, s1 = F.col_lift(x, "fp32" if x.dtype == np.uint32 else "bf16")
    assert np.array_equal(d0, d1) and np.array_equal(s0, s1)


def test_col_decode_layout_matches_brute_force():
    g = np.random.default_rng(7)
    data = g.integers(0, 256, (70, 40), dtype=np.uint8)
    scale = g.integers(0, 256, (3, 40), dtype=np.uint8)
    scale[0, :4] = [0, 255, 127, 254]
    for out, od in (("bf16", BF16), ("fp32", FP32)):
        got = oracle.dequantize(data, scale, layout=oracle.COL_32X1, out_dtype=od)
        assert np.array_equal(got, F.dequantize(data, scale, "col", out))


@pytest.mark.parametrize("mutation,changes", [("col_emax7", True), ("col_nan_poisons", True), ("col_rule_448", False)])
def test_col_pins_catch_planted_mistakes(mutation, changes):
    """A wrong shift or whole-block NaN poisoning changes the bytes the pins
    compare; the other reading of the host rule (ceil(log2(amax/448))) gives
    the same bytes on projected weights, so that choice is not load-bearing."""
    x = W.c2_exhaustive(natural=True)
    d0, s0 = oracle.mxfp4_to_mxfp8_col(x)
    d1, s1 = F.col_lift(x, "bf16", mutation=mutation)
    same = np.array_equal(d0, d1) and np.array_equal(s0, s1)
    assert same != changes


def test_oracle_matches_brute_force_at_every_block_exponent():
    """Oracle vs the Fraction brute force with the block exponent swept over the
    whole clamp range: for every e in [-126, 125], two blocks anchored by
    +-6 * 2^e whose other 31 elements are random bf16 patterns of magnitude at
    most 6 * 2^e (so e is the block's scale exponent), including the grid
    midpoints and subnormals that fall under it."""
    g = np.random.default_rng(11)
    pool = np.arange(0x7F80, dtype=np.uint16)                     # finite magnitudes
    mags = (pool.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rows = []
    for e in range(-126, 126):
        cap = np.ldexp(6.0, e)
        sel = pool[mags <= cap]
        for sign in (0, 0x8000):
            blk = g.choice(sel, 31) | (g.integers(0, 2, 31).astype(np.uint16) << 15)
            rows.append(np.concatenate([[W.bf16_bits_of(cap) | sign], blk]).astype(np.uint16))
    x = np.ascontiguousarray(np.stack(rows))
    assert np.array_equal(oracle.fake_quantize_mxfp4(x), F.fake_quantize(x, "bf16"))
    d0, s0 = oracle.mxfp4_to_mxfp8_row(x)
    d1, s1 = F.row_lift(x, "bf16")
    assert np.array_equal(d0, d1) and np.array_equal(s0, s1)
    assert np.array_equal(oracle.dequantize(d0, s0), F.dequantize(d1, s1, "row", "bf16"))
    dc0, sc0 = oracle.mxfp4_to_mxfp8_col(x)
    dc1, sc1 = F.col_lift(x, "bf16")
    assert np.array_equal(dc0, dc1) and np.array_equal(sc0, sc1)


def test_every_oracle_function_is_pinned():
    """Every public function of the oracle package is exercised by this file,
    and the C library exports exactly the entry points the package binds."""
    import inspect
    import re
    import subprocess
    src = open(__file__).read()
    public = [n for n, f in inspect.getmembers(oracle, inspect.isfunction)
              if not n.startswith("_") and f.__module__ == oracle.__name__ and n not in ("build", "lib")]
    unpinned = [n for n in public if not re.search(r"oracle\." + n + r"\(", src)]
    assert not unpinned, unpinned
    nm = subprocess.run(["nm", "-D", "--defined-only", oracle.build()], capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in nm.splitlines() if " T " in l}
    bound = set(re.findall(r"L\.(orc_\w+)\.", inspect.getsource(oracle.lib)))
    assert exported == bound, (exported ^ bound)
