"""Seeded synthetic inputs for the quantization path.

Shared by the tests, the smoke check and the bench: each generator returns the
raw bits of a host array (bf16 as numpy uint16, fp32 as numpy uint32), and the
same host array feeds both the CPU oracle and the device copy.  This module
only draws and lays out values; it holds none of the quantization arithmetic.

The shapes and value distributions follow the workloads on the pages (the
TransformerEngine MXFP4-QAT pull request, section Test results (B200), and the
export pull request, section Description):

* ``c1_small``      100 x 48 bf16, N(0,1) * 2^randint(-10, 10) per row, seed 0
                    (one full and one 16-wide block per row).
* ``c2_exhaustive`` 2048 x 32 bf16 holding every bf16 bit pattern once,
                    shuffled with seed 0 (``natural=True``: row i holds patterns
                    32i..32i+31), plus ``c2_planted``, a 64 x 32 companion of
                    edge rows.
* ``c3_spread``     4096 x 4096 fp32 of 128x128 tiles whose block exponents
                    spread by d = t mod 17, mantissas on the E2M1 grid, seed 2.
* ``c4_headline``   8192 x 8192 bf16, N(0, 0.02), seed 1.
* ``c5_mlp``        28672 x 8192 (seed 2) and 8192 x 28672 (seed 3) bf16,
                    N(0, 0.02), and the fp32 master of the first.
"""
from __future__ import annotations

import numpy as np
import torch

BF16_POS_ZERO, BF16_NEG_ZERO = 0x0000, 0x8000


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    """fp32 tensor -> bf16 bits (torch's round-to-nearest-even cast)."""
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _fp32_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int32).numpy().view(np.uint32)


def bf16_bits_of(values) -> np.ndarray:
    """Exact bf16 bits of float64 values that bf16 represents exactly (checked)."""
    v = np.asarray(values, dtype=np.float64)
    f32 = v.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), v, equal_nan=True):
        raise ValueError("value not representable in fp32")
    bits = f32.view(np.uint32)
    if np.any((bits & 0xFFFF) != 0):
        raise ValueError("value not representable in bf16")
    return (bits >> 16).astype(np.uint16)


def c1_small(seed: int = 0) -> np.ndarray:
    g = torch.Generator().manual_seed(seed)
    base = torch.randn(100, 48, generator=g)
    expo = torch.randint(-10, 11, (100, 1), generator=g)
    return _bf16_bits(base * torch.exp2(expo.to(torch.float32)))


def c2_exhaustive(seed: int = 0, natural: bool = False) -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if not natural:
        perm = torch.randperm(65536, generator=torch.Generator().manual_seed(seed)).numpy()
        bits = bits[perm]
    return bits.reshape(2048, 32).copy()


# E2M1 magnitudes and the midpoints between neighbours (values on the pages'
# grid {0, .5, 1, 1.5, 2, 3, 4, 6}).
GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def c2_planted(seed: int = 0) -> np.ndarray:
    """64 x 32 bf16 edge rows: 2^-127 and code-0 absorption, +-0, the subnormal
    ladder, every grid point and midpoint at the lowest block exponents,
    1.5*2^k +- 1 ulp, saturation above 6*2^125, and non-finite poisoning."""
    rows = []
    r = lambda vals: rows.append(np.asarray(vals, dtype=np.uint16))
    two = lambda k: bf16_bits_of(np.ldexp(1.0, k))
    r([two(-127)] * 32)                                            # all 2^-127
    r([two(-127), two(-128)] * 16)                                 # 2^-127 with the 2^-128 tie
    ladder = [two(-127 - i) for i in range(7)]                      # 2^-127 .. 2^-133
    neg = [v | 0x8000 for v in ladder]
    r(ladder + neg + ladder + neg + [two(-127)] * 4)
    r([BF16_POS_ZERO, BF16_NEG_ZERO] * 16)                         # +-0
    r([BF16_NEG_ZERO] * 32)                                        # all -0
    for e in range(-126, -120):                                    # grid and midpoints at low e
        vals = [6.0] + [s * p for p in GRID for s in (1, -1)] + [s * m for m in MIDPOINTS for s in (1, -1)] + [-6.0]
        r(bf16_bits_of(np.ldexp(np.array(vals), e)))
    for e in (-126, -125, -100, 0, 100, 125):                      # midpoints +- 1 ulp
        vals = []
        for m in MIDPOINTS:
            b = int(bf16_bits_of(np.ldexp(m, e)))
            vals += [b - 1, b + 1] if b > 0 else [b, b]
        vals += [int(bf16_bits_of(np.ldexp(6.0, e)))] * (32 - len(vals))
        r(vals)
    for k in (-124, -60, -1, 0, 1, 60, 126, 127):                  # 1.5*2^k and +-1 ulp
        b = int(bf16_bits_of(np.ldexp(1.5, k)))
        r([b - 1, b, b + 1] * 10 + [b, b])
    r([0x7F40] * 16 + list(range(0x7F41, 0x7F51)))                 # 6*2^125 and above
    r(list(range(0x7F60, 0x7F80)))                                 # up to bf16 max
    r([0x7F7F, 0xFF7F] * 16)                                       # +-max
    r([0x3F80] * 31 + [0x7F80])                                    # +Inf poisons
    r([0x3F80] * 31 + [0xFF80])                                    # -Inf poisons
    r([0x7FC1] + [0x0040] * 31)                                    # NaN poisons a 2^-127 block
    r([0x3F80, 0xFFC0] + [0xBF80] * 30)                            # -NaN
    g = torch.Generator().manual_seed(seed)
    while len(rows) < 64:                                          # random rows at scattered scales
        i = len(rows)
        scale = float(2.0 ** (((i * 37) % 250) - 125))
        rows.append(_bf16_bits(torch.randn(32, generator=g) * scale))
    assert all(len(x) == 32 for x in rows)
    return np.stack(rows[:64]).astype(np.uint16)


def fp32_bits_of(values) -> np.ndarray:
    """Exact fp32 bits of float64 values that fp32 represents exactly (checked)."""
    v = np.asarray(values, dtype=np.float64)
    f32 = v.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), v, equal_nan=True):
        raise ValueError("value not representable in fp32")
    return f32.view(np.uint32).copy()


def c2_planted_fp32(seed: int = 0) -> np.ndarray:
    """160 x 32 fp32 edge rows (one 1x32 block per row): the 64 rows of
    c2_planted widened exactly, then the fp32-only edges -- the ladder
    2^-127 .. 2^-149 with the 2^-128 tie in a block of scale 2^-126, every E2M1
    midpoint one fp32 ulp either side at low, middle and top exponents,
    1.5*2^k and its fp32 neighbours as a block's amax (down into the fp32
    subnormals), values from 6*2^125 up to the largest fp32, and non-finite
    poisoning with several NaN payloads."""
    rows = [r.astype(np.uint32) << 16 for r in c2_planted(seed)]
    r = lambda vals: rows.append(np.asarray(vals, dtype=np.uint32))
    two = lambda k: int(fp32_bits_of(np.ldexp(1.0, k)))
    NEG = 0x80000000
    ladder = [two(-127 - i) for i in range(23)]                    # 2^-127 .. 2^-149 (fp32 subnormals)
    r(ladder + [v | NEG for v in ladder[1:10]])
    r([v | NEG for v in ladder] + ladder[1:10])
    r([two(-127), two(-128)] * 16)                                 # the 2^-128 tie beside 2^-127
    r([two(-128)] * 32)                                            # amax 2^-128 alone: e = -126, all ties to 0
    r([two(-128) | NEG, two(-149)] * 16)
    for e in (-126, -125, -122, -121, -100, -1, 0, 1, 100, 124, 125):
        for sign in (0, NEG):                                      # midpoints exactly and one ulp either side
            vals = [int(fp32_bits_of(np.ldexp(6.0, e)))]
            for m in MIDPOINTS:
                b = int(fp32_bits_of(np.ldexp(m, e)))
                vals += [b - 1, b, b + 1]
            vals += [int(fp32_bits_of(np.ldexp(6.0, e))) - 1, int(fp32_bits_of(np.ldexp(0.5, e))) - 1,
                     int(fp32_bits_of(np.ldexp(0.5, e))) + 1]
            vals += [vals[0]] * (32 - len(vals))
            r([v | sign for v in vals])
    for k in (-148, -140, -130, -128, -127, -126, -125, -124, -123, -60, -1, 0, 1, 60, 126, 127):
        b = int(fp32_bits_of(np.ldexp(1.5, k)))                   # 1.5*2^k - 1 ulp, exactly, + 1 ulp as amax
        for d in (-1, 0, 1):
            r([b + d, (b + d) | NEG] * 8 + [two(k - 3), two(k - 4) | NEG] * 8 if k > -146 else [b + d, (b + d) | NEG] * 16)
    sat = np.linspace(0x7F400000, 0x7F7FFFFF, 32).astype(np.int64)
    r(sat)                                                         # 6*2^125 up to FLT_MAX
    r([0x7F7FFFFF, 0xFF7FFFFF] * 8 + [0x7F400001, 0xFF400001] * 8)
    r([0x7F3FFFFF] * 16 + [0x7F400000, 0x7F400001] * 8)            # just below, at and above the cap
    r([0x3F800000] * 31 + [0x7F800000])                            # +Inf poisons
    r([0x3F800000] * 31 + [0xFF800000])                            # -Inf poisons
    r([0x7F800001] + [two(-127)] * 31)                             # signalling NaN in a 2^-127 block
    r([0x3F800000, 0xFFC00000] + [0xBF800000] * 30)                # negative quiet NaN
    r([0x7FFFFFFF] + [0x00000001] * 31)                            # NaN with a full payload beside 2^-149
    g = torch.Generator().manual_seed(seed + 1)
    while len(rows) < 160:                                         # random rows at scattered scales
        i = len(rows)
        rows.append(_fp32_bits(torch.randn(32, generator=g) * float(2.0 ** (((i * 41) % 270) - 145))))
    assert all(len(x) == 32 for x in rows) and len(rows) == 160, len(rows)
    return np.stack(rows).astype(np.uint32)


def c3_spread(seed: int = 2, shape=(4096, 4096)) -> np.ndarray:
    """fp32 bits.  Tile t (row-major) has spread d = t mod 17 and base exponent
    b uniform in [-110, 100], or b = -126 for tiles with floor(t/17) mod 4 == 0.
    Each 1x32 block gets exponent b+u with u ~ U{0..d} (block 0 of a tile u = 0,
    block 1 u = d); elements are +-p*2^(b+u) with p uniform on the E2M1 grid,
    and one element per block is +-6*2^(b+u) so that block's amax is exactly
    6*2^(b+u)."""
    R, K = shape
    if R % 128 or K % 128:
        raise ValueError("spread sweep needs 128-aligned shapes")
    g = torch.Generator().manual_seed(seed)
    tr, tc = R // 128, K // 128
    ntile = tr * tc
    t = torch.arange(ntile)
    d = t % 17
    b = torch.randint(-110, 101, (ntile,), generator=g)
    b = torch.where((t // 17) % 4 == 0, torch.full_like(b, -126), b)
    # blocks of a tile: 128 rows x 4 blocks, numbered row-major inside the tile
    u = torch.floor(torch.rand(ntile, 512, generator=g) * (d[:, None] + 1).to(torch.float32)).to(torch.int64)
    u = torch.minimum(u, d[:, None])
    u[:, 0] = 0
    u[:, 1] = d
    pidx = torch.randint(0, 8, (ntile, 512, 32), generator=g)
    sign = torch.randint(0, 2, (ntile, 512, 32), generator=g)
    force = torch.randint(0, 32, (ntile, 512), generator=g)
    grid = torch.tensor(GRID, dtype=torch.float64)
    p = grid[pidx]
    p.scatter_(2, force[:, :, None], 6.0)
    expo = (b[:, None] + u)[:, :, None].expand(-1, -1, 32)
    vals = torch.ldexp(p, expo.to(torch.float64)) * (1 - 2 * sign).to(torch.float64)
    # (tile, row-in-tile, block, elem) -> (tile-row, row, tile-col, block, elem)
    vals = vals.view(tr, tc, 128, 4, 32).permute(0, 2, 1, 3, 4).reshape(R, K)
    v = vals.numpy()
    f32 = v.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), v)
    return f32.view(np.uint32).copy()


def c3_block_exponents(seed: int = 2, shape=(4096, 4096)):
    """(d per tile, base per tile) of c3_spread, for checks on the sweep."""
    R, K = shape
    g = torch.Generator().manual_seed(seed)
    ntile = (R // 128) * (K // 128)
    t = torch.arange(ntile)
    d = t % 17
    b = torch.randint(-110, 101, (ntile,), generator=g)
    b = torch.where((t // 17) % 4 == 0, torch.full_like(b, -126), b)
    return d.numpy(), b.numpy()


def c4_headline(seed: int = 1, shape=(8192, 8192)) -> np.ndarray:
    g = torch.Generator().manual_seed(seed)
    return _bf16_bits(torch.randn(*shape, generator=g) * 0.02)


def c4_master(seed: int = 1, shape=(8192, 8192)) -> np.ndarray:
    """fp32 bits of the headline weight before its bf16 cast (the master copy)."""
    g = torch.Generator().manual_seed(seed)
    return _fp32_bits(torch.randn(*shape, generator=g) * 0.02)


def c5_mlp(which: str):
    """which: 'up' (28672 x 8192 bf16, seed 2), 'down' (8192 x 28672 bf16,
    seed 3) or 'up_master' (fp32 bits of the first before its bf16 cast)."""
    if which == "down":
        g = torch.Generator().manual_seed(3)
        return _bf16_bits(torch.randn(8192, 28672, generator=g) * 0.02)
    g = torch.Generator().manual_seed(2)
    w = torch.randn(28672, 8192, generator=g) * 0.02
    if which == "up":
        return _bf16_bits(w)
    if which == "up_master":
        return _fp32_bits(w)
    raise ValueError(which)


# Low halves that widen a bf16 pattern into the fp32 corpus: 0x0000 is the
# bf16 value itself (every E2M1 grid point and midpoint, exactly), 0x0001 its
# neighbour one fp32 ulp up, 0xFFFF the neighbour one fp32 ulp below the next
# bf16 pattern; None draws one random low half per pattern.
FP32_LOW_HALVES = (0x0000, 0x0001, 0xFFFF, None)


def value_exponent_pairs(dtype: str = "bf16", width: int = 256, seed: int = 7) -> np.ndarray:
    """Every (element value, block exponent e) pair, e in [-126, 125]: for each
    e, every finite value with |x| <= 6 * 2^e (every finite value at e = 125,
    where larger ones saturate) is placed in 1x32 blocks whose first element is
    6 * 2^e, so that is the block's amax and e its scale exponent.  bf16: all
    65536 patterns; fp32: every bf16 pattern widened with each low half of
    FP32_LOW_HALVES, so every E2M1 midpoint and its neighbours one fp32 ulp
    either side meet every e (and the fp32 subnormals 2^-149 .. occur).
    Returned as a [rows, width] bit array (zeros pad the last row)."""
    g = np.random.default_rng(seed)
    if dtype == "bf16":
        pool = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        vals = pool.astype(np.uint32).view(np.uint32) << 16
        out_t, anchor_of = np.uint16, lambda e: int(bf16_bits_of(np.ldexp(6.0, e)))
    else:
        hi = np.arange(65536, dtype=np.uint32) << 16
        pool = np.concatenate([hi | (g.integers(0, 65536, 65536).astype(np.uint32) if low is None else np.uint32(low))
                               for low in FP32_LOW_HALVES])
        vals = pool
        out_t = np.uint32
        anchor_of = lambda e: int(np.array(np.ldexp(6.0, e), dtype=np.float32).view(np.uint32))
    with np.errstate(invalid="ignore"):
        mags = np.abs(vals.view(np.float32).astype(np.float64))
    finite = np.isfinite(mags)
    blocks = []
    for e in range(-126, 126):
        sel = pool[finite & ((mags <= np.ldexp(6.0, e)) | (e == 125))]
        sel = g.permutation(sel)
        nb = (len(sel) + 30) // 31
        padded = np.zeros(nb * 31, dtype=out_t)
        padded[: len(sel)] = sel
        b = np.empty((nb, 32), dtype=out_t)
        b[:, 0] = anchor_of(e)
        b[:, 1:] = padded.reshape(nb, 31)
        blocks.append(b)
    flat = np.concatenate(blocks).reshape(-1)
    per_row = width
    rows = (len(flat) + per_row - 1) // per_row
    out = np.zeros(rows * per_row, dtype=out_t)
    out[: len(flat)] = flat
    return out.reshape(rows, per_row)


def fp32_fuzz(n: int = 1 << 16, seed: int = 5) -> np.ndarray:
    """Random fp32 bit patterns (all classes) reshaped to (n/32, 32), with a
    random per-row exponent window so blocks hold values of similar size."""
    g = torch.Generator().manual_seed(seed)
    rows = n // 32
    raw = torch.randint(0, 2**31, (rows, 32), generator=g, dtype=torch.int64)
    expo = torch.randint(0, 256, (rows, 1), generator=g, dtype=torch.int64)
    spread = torch.randint(0, 12, (rows, 32), generator=g, dtype=torch.int64)
    e = torch.clamp(expo - spread, 0, 255)
    sign = torch.randint(0, 2, (rows, 32), generator=g, dtype=torch.int64)
    bits = (sign << 31) | (e << 23) | (raw & 0x7FFFFF)
    return bits.numpy().astype(np.uint32)
