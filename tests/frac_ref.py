"""Exact-rational brute force, used only to pin the C oracle on small inputs.

Written independently of ``oracle/mxq_oracle.c``: values are Python Fractions,
the scale exponent is found by scanning every candidate exponent, the E2M1
code by comparing the distance to all eight grid points, and every FP8 / bf16
encoding by searching the full list of values that format can hold.  No
shortcut, bit trick or rounding formula is shared with the oracle.

Definitions follow the TransformerEngine MXFP4-QAT pull request ("[PyTorch]
MXFP4 weight QAT on MXFP8 and FP8 block-scaling recipes"), section Description
(both conversion modes and the E8M0 decode), and the export pull request
("MXFP8TensorStorage.export_components()"), section Description.

``mutation`` switches plant one plausible mistake each, so the tests can show
that the pins would notice that mistake.
"""
from __future__ import annotations

import bisect
from fractions import Fraction

import numpy as np

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
NAN = "nan"


# ---- IEEE-style decoding straight from the bit layout ---------------------------------

def decode_bits(bits: int, ebits: int, mbits: int, bias: int, fn: bool = False):
    """Fraction value, or "inf"/"-inf"/NAN."""
    sign = -1 if (bits >> (ebits + mbits)) & 1 else 1
    E = (bits >> mbits) & ((1 << ebits) - 1)
    m = bits & ((1 << mbits) - 1)
    allones = (1 << ebits) - 1
    if fn:
        if E == allones and m == (1 << mbits) - 1:
            return NAN
    elif E == allones:
        return NAN if m else ("inf" if sign > 0 else "-inf")
    if E == 0:
        mag = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        mag = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (E - bias)
    return sign * mag


def bf16_value(b):
    return decode_bits(int(b), 8, 7, 127)


def fp32_value(b):
    return decode_bits(int(b), 8, 23, 127)


def e4m3_value(b):
    return decode_bits(int(b), 4, 3, 7, fn=True)


def e5m2_value(b):
    return decode_bits(int(b), 5, 2, 15)


def is_negative_bits(bits: int, width: int) -> bool:
    return bool((bits >> (width - 1)) & 1)


# ---- nearest representable value by search over the whole format ----------------------

class Table:
    """All finite non-negative values of a format, sorted, with their bit patterns."""

    def __init__(self, width: int, value_fn):
        pairs = []
        for b in range(1 << (width - 1)):
            v = value_fn(b)
            if isinstance(v, Fraction):
                pairs.append((v, b))
        pairs.sort()
        self.values = [v for v, _ in pairs]
        self.bits = [b for _, b in pairs]
        self.signbit = 1 << (width - 1)
        self.exact = {v: b for v, b in pairs}

    def nearest_even(self, v: Fraction, neg: bool, overflow_bits=None) -> int:
        """Nearest value to |v| with ties to the even bit pattern; sign re-applied."""
        a = abs(v)
        i = bisect.bisect_left(self.values, a)
        cands = []
        for j in (i - 1, i):
            if 0 <= j < len(self.values):
                cands.append((abs(self.values[j] - a), self.bits[j] & 1, self.bits[j]))
        if a > self.values[-1] and overflow_bits is not None:
            top = self.values[-1]
            ulp = top - self.values[-2]
            if a >= top + ulp / 2:                       # IEEE: rounds to infinity
                return overflow_bits | (self.signbit if neg else 0)
        cands.sort()
        b = cands[0][2]
        return b | (self.signbit if neg else 0)

    def encode_exact(self, v: Fraction, neg: bool) -> int:
        b = self.exact[abs(v)]
        return b | (self.signbit if neg else 0)


_tables = {}


def table(name: str) -> Table:
    if name not in _tables:
        if name == "bf16":
            _tables[name] = Table(16, bf16_value)
        elif name == "e4m3":
            _tables[name] = Table(8, e4m3_value)
        elif name == "e5m2":
            _tables[name] = Table(8, e5m2_value)
        else:
            raise KeyError(name)
    return _tables[name]


FP32_MAX = (2 - Fraction(1, 1 << 23)) * Fraction(2) ** 127


def fp32_encode_exact(v: Fraction, neg: bool) -> int:
    """Bits of a value fp32 holds exactly (asserted); above the fp32 range: Inf."""
    a = abs(v)
    if a > FP32_MAX:
        return 0xFF800000 if neg else 0x7F800000
    f = np.float32(float(a))
    assert Fraction(float(f)) == a, "not exact in fp32"
    bits = int(np.array(f, dtype=np.float32).view(np.uint32))
    return bits | (0x80000000 if neg else 0)


# ---- the method -----------------------------------------------------------------------

_SIX_POW = [(e, 6 * Fraction(2) ** e) for e in range(-400, 400)]
_SIX_VALS = [v for _, v in _SIX_POW]


def scale_exponent(amax: Fraction, mutation: str | None = None) -> int:
    """Smallest integer e with 6 * 2^e >= amax (searched over every candidate
    exponent in [-400, 400)), clamped to [-126, 125]."""
    lo = -127 if mutation == "clamp_low_127" else -126
    if amax == 0:
        return lo
    e = _SIX_POW[bisect.bisect_left(_SIX_VALS, amax)][0]
    return max(lo, min(125, e))


def e2m1_code(t: Fraction, mutation: str | None = None) -> int:
    """Index of the grid point nearest to t >= 0; ties to the even index
    (mutation "ties_away": ties to the larger grid point)."""
    best, bestd = None, None
    for c, g in enumerate(GRID):
        d = abs(t - g)
        if bestd is None or d < bestd:
            best, bestd = c, d
        elif d == bestd:
            if mutation == "ties_away":
                best = c
            elif c % 2 == 0:
                best = c
    return best


def _values_and_sign(bits, dtype: str):
    vals = [bf16_value(b) if dtype == "bf16" else fp32_value(b) for b in bits]
    width = 16 if dtype == "bf16" else 32
    negs = [is_negative_bits(int(b), width) for b in bits]
    return vals, negs


def block_decomposition(bits, dtype: str, mutation: str | None = None):
    """(poisoned, e, [codes], [negs]) of one 1x32 block (or shorter last block)."""
    vals, negs = _values_and_sign(bits, dtype)
    poisoned = any(not isinstance(v, Fraction) for v in vals)
    finite = [abs(v) for v in vals if isinstance(v, Fraction)]
    e = scale_exponent(max(finite) if finite else Fraction(0), mutation)
    codes = [e2m1_code(abs(v) / Fraction(2) ** e, mutation) if isinstance(v, Fraction) else None for v in vals]
    return poisoned, e, codes, negs


def _blocks(K: int):
    return [(c0, min(c0 + 32, K)) for c0 in range(0, K, 32)]


def fake_quantize(x: np.ndarray, dtype: str, mutation: str | None = None) -> np.ndarray:
    rows, K = x.shape
    y = np.zeros_like(x)
    nan = 0x7FC0 if dtype == "bf16" else 0x7FC00000
    for r in range(rows):
        for c0, c1 in _blocks(K):
            poisoned, e, codes, negs = block_decomposition(x[r, c0:c1], dtype, mutation)
            for i, (c, neg) in enumerate(zip(codes, negs)):
                if poisoned:
                    y[r, c0 + i] = nan
                    continue
                v = GRID[c] * Fraction(2) ** e
                y[r, c0 + i] = table("bf16").encode_exact(v, neg) if dtype == "bf16" else fp32_encode_exact(v, neg)
    return y


def row_lift(x: np.ndarray, dtype: str, scale_ld: int | None = None, mutation: str | None = None):
    rows, K = x.shape
    nb = (K + 31) // 32
    data = np.zeros((rows, K), dtype=np.uint8)
    scale = np.zeros((rows, scale_ld or nb), dtype=np.uint8)
    for r in range(rows):
        for j, (c0, c1) in enumerate(_blocks(K)):
            poisoned, e, codes, negs = block_decomposition(x[r, c0:c1], dtype, mutation)
            if poisoned:
                scale[r, j] = 255
                data[r, c0:c1] = 0x7F
                continue
            S = e - 6
            if mutation != "no_absorption":
                S = max(S, -127)
            code = S + 127
            scale[r, j] = code & 0xFF
            for i, (c, neg) in enumerate(zip(codes, negs)):
                payload = GRID[c] * Fraction(2) ** (e - S)
                data[r, c0 + i] = table("e4m3").nearest_even(payload, neg)
    return data, scale


def block128(x: np.ndarray, dtype: str, mutation: str | None = None):
    rows, K = x.shape
    data = np.zeros((rows, K), dtype=np.uint8)
    codes_out = np.zeros(((rows + 127) // 128, (K + 127) // 128), dtype=np.uint8)
    for tr in range(0, rows, 128):
        for tc in range(0, K, 128):
            blocks = []
            for r in range(tr, min(tr + 128, rows)):
                for c0, c1 in _blocks(K):
                    if tc <= c0 < tc + 128:
                        blocks.append((r, c0, c1, block_decomposition(x[r, c0:c1], dtype, mutation)))
            finite_e = [b[3][1] for b in blocks if not b[3][0]]
            M = max(finite_e) if finite_e else -126
            S = max(M - 6, -126 if mutation == "tile_clamp_126" else -127)
            codes_out[tr // 128, tc // 128] = S + 127
            for r, c0, c1, (poisoned, e, codes, negs) in blocks:
                for i, (c, neg) in enumerate(zip(codes, negs)):
                    if poisoned:
                        data[r, c0 + i] = 0x7F
                    else:
                        data[r, c0 + i] = table("e4m3").nearest_even(GRID[c] * Fraction(2) ** (e - S), neg)
    return data, codes_out


_POW2 = [(k, Fraction(2) ** k) for k in range(-400, 400)]
_POW2_VALS = [v for _, v in _POW2]


def col_scale(amax: Fraction, mutation: str | None = None) -> int:
    """Shared scale exponent S of a 32x1 block: the largest k with 2^k <= amax
    (found by search over every k in [-400, 400)), minus 8 (E4M3's largest
    exponent), at least -127; amax 0 gives -127.
    mutation "col_rule_448": the smallest S with amax / 2^S <= 448 instead.
    mutation "col_emax7": floor(log2 amax) - 7."""
    if amax == 0:
        return -127
    if mutation == "col_rule_448":
        S = min(k for k, v in _POW2 if amax / v <= 448)
    else:
        k = _POW2[bisect.bisect_right(_POW2_VALS, amax) - 1][0]
        S = k - (7 if mutation == "col_emax7" else 8)
    return max(S, -127)


def col_lift(x: np.ndarray, dtype: str, scale_ld: int | None = None, mutation: str | None = None):
    """MXFP8 columnwise from the decomposition: the projected values p * 2^e,
    re-quantized over 32x1 blocks of each column.  A NaN (poisoned) element gets
    0x7F and no say in the block's amax (mutation "col_nan_poisons": any NaN
    makes the whole block code 255 / 0x7F)."""
    rows, K = x.shape
    y = [[None] * K for _ in range(rows)]                # (value, neg) or NAN
    for r in range(rows):
        for c0, c1 in _blocks(K):
            poisoned, e, codes, negs = block_decomposition(x[r, c0:c1], dtype)
            for i, (c, neg) in enumerate(zip(codes, negs)):
                y[r][c0 + i] = NAN if poisoned else (GRID[c] * Fraction(2) ** e, neg)
    data = np.zeros((rows, K), dtype=np.uint8)
    scale = np.zeros(((rows + 31) // 32, scale_ld or K), dtype=np.uint8)
    for b0 in range(0, rows, 32):
        for col in range(K):
            cells = [(r, y[r][col]) for r in range(b0, min(b0 + 32, rows))]
            finite = [v for _, t in cells if t != NAN for v in (t[0],)]
            if mutation == "col_nan_poisons" and len(finite) < len(cells):
                scale[b0 // 32, col] = 255
                for r, _ in cells:
                    data[r, col] = 0x7F
                continue
            S = col_scale(max(finite) if finite else Fraction(0), mutation)
            scale[b0 // 32, col] = S + 127
            for r, t in cells:
                data[r, col] = 0x7F if t == NAN else table("e4m3").nearest_even(t[0] / Fraction(2) ** S, t[1])
    return data, scale


def export(scale_storage: np.ndarray, K: int, mutation: str | None = None) -> np.ndarray:
    ncols = K // 32 if mutation == "floor_cols" else (K + 31) // 32
    return scale_storage[:, :ncols].copy()


def e8m0_value(code: int):
    return NAN if code == 255 else Fraction(2) ** (int(code) - 127)


def dequantize(data: np.ndarray, scale: np.ndarray, layout: str, out: str, fp8: str = "e4m3") -> np.ndarray:
    rows, K = data.shape
    res = np.zeros((rows, K), dtype=np.uint16 if out == "bf16" else np.uint32)
    nan = 0x7FC0 if out == "bf16" else 0x7FC00000
    dec = e4m3_value if fp8 == "e4m3" else e5m2_value
    for r in range(rows):
        for col in range(K):
            c = (scale[r, col // 32] if layout == "row" else scale[r // 128, col // 128] if layout == "tile"
                 else scale[r // 32, col])
            q = dec(int(data[r, col]))
            s = e8m0_value(int(c))
            neg = bool(data[r, col] & 0x80)
            if q == NAN or s == NAN:
                res[r, col] = nan
            elif isinstance(q, str):                      # E5M2 infinity
                res[r, col] = (0xFF80 if neg else 0x7F80) if out == "bf16" else (0xFF800000 if neg else 0x7F800000)
            else:
                v = q * s
                if out == "bf16":
                    res[r, col] = table("bf16").nearest_even(v, neg, overflow_bits=0x7F80)
                else:
                    res[r, col] = fp32_encode_exact(v, neg)
    return res


# ---- packed MXFP4 (deployment format) ---------------------------------------------------

def quantize_mxfp4(x: np.ndarray, dtype: str):
    """Packed E2M1 nibbles (element 2i low, 2i+1 high) and E8M0 codes with the
    scale exponent clamped to [-126, 126]."""
    rows, K = x.shape
    nb = (K + 31) // 32
    packed = np.zeros((rows, (K + 1) // 2), dtype=np.uint8)
    scale = np.zeros((rows, nb), dtype=np.uint8)
    for r in range(rows):
        for j, (c0, c1) in enumerate(_blocks(K)):
            vals, negs = _values_and_sign(x[r, c0:c1], dtype)
            if any(not isinstance(v, Fraction) for v in vals):
                scale[r, j] = 255
                continue
            amax = max(abs(v) for v in vals)
            e = -126 if amax == 0 else max(-126, min(126, _SIX_POW[bisect.bisect_left(_SIX_VALS, amax)][0]))
            scale[r, j] = e + 127
            for i, (v, neg) in enumerate(zip(vals, negs)):
                nib = (8 if neg else 0) | e2m1_code(abs(v) / Fraction(2) ** e)
                col = c0 + i
                packed[r, col // 2] |= nib << (4 * (col % 2))
    return packed, scale


def _nibble(packed, r, col):
    nib = (int(packed[r, col // 2]) >> (4 * (col % 2))) & 0xF
    return bool(nib & 8), GRID[nib & 7]


def dequantize_mxfp4(packed: np.ndarray, scale: np.ndarray, K: int, out: str):
    rows = packed.shape[0]
    res = np.zeros((rows, K), dtype=np.uint16 if out == "bf16" else np.uint32)
    for r in range(rows):
        for col in range(K):
            c = int(scale[r, col // 32])
            if c == 255:
                res[r, col] = 0x7FC0 if out == "bf16" else 0x7FC00000
                continue
            neg, p = _nibble(packed, r, col)
            v = p * Fraction(2) ** (c - 127)
            res[r, col] = (table("bf16").nearest_even(v, neg, overflow_bits=0x7F80) if out == "bf16"
                           else fp32_encode_exact(v, neg))
    return res


def packed_to_row(packed: np.ndarray, scale: np.ndarray, K: int):
    rows = packed.shape[0]
    nb = (K + 31) // 32
    data = np.zeros((rows, K), dtype=np.uint8)
    out = np.zeros((rows, nb), dtype=np.uint8)
    for r in range(rows):
        for j, (c0, c1) in enumerate(_blocks(K)):
            c = int(scale[r, j])
            if c == 255:
                out[r, j] = 255
                data[r, c0:c1] = 0x7F
                continue
            e = c - 127
            S = max(e - 6, -127)
            out[r, j] = S + 127
            for col in range(c0, c1):
                neg, p = _nibble(packed, r, col)
                data[r, col] = table("e4m3").nearest_even(p * Fraction(2) ** (e - S), neg)
    return data, out


def packed_to_block128(packed: np.ndarray, scale: np.ndarray, K: int):
    rows = packed.shape[0]
    data = np.zeros((rows, K), dtype=np.uint8)
    codes = np.zeros(((rows + 127) // 128, (K + 127) // 128), dtype=np.uint8)
    for tr in range(0, rows, 128):
        for tc in range(0, K, 128):
            blocks = [(r, j) for r in range(tr, min(tr + 128, rows)) for j in range(tc // 32, min(tc + 128, K + 31) // 32)
                      if j * 32 < K]
            finite = [int(scale[r, j]) - 127 for r, j in blocks if scale[r, j] != 255]
            M = max(finite) if finite else -126
            S = max(M - 6, -127)
            codes[tr // 128, tc // 128] = S + 127
            for r, j in blocks:
                c = int(scale[r, j])
                for col in range(j * 32, min(j * 32 + 32, K)):
                    if c == 255:
                        data[r, col] = 0x7F
                    else:
                        neg, p = _nibble(packed, r, col)
                        data[r, col] = table("e4m3").nearest_even(p * Fraction(2) ** (c - 127 - S), neg)
    return data, codes
