"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, bit for bit.

Tolerance is 0: every payload byte, scale code and output bit must match,
NaNs included (both sides write the canonical quiet NaN).  Inputs are the
seeded workloads of ``workloads`` -- the same host bits feed the oracle and the
device copy.  Sizes: the small and exhaustive corpora, the 4096 x 4096 spread
sweep, the 8192 x 8192 headline weight and the 28672 x 8192 / 8192 x 28672
MLP weights (and the fp32 master of the first), all compared in full.
"""
import numpy as np
import pytest
import torch

import microscaling_weight_quantization_amd as mxq
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

THREADS = 16


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mxq.load()
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray, device) -> torch.Tensor:
    if bits.dtype == np.uint16:
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    if bits.dtype == np.uint32:
        return torch.from_numpy(bits.view(np.int32)).to(device).view(torch.float32)
    return torch.from_numpy(bits).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.numpy()


def assert_bits(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches; first at {i}: got {got[i]:#x} want {want[i]:#x}")


def out_dtype_of(bits):
    return (torch.bfloat16, oracle.BF16) if bits.dtype == np.uint16 else (torch.float32, oracle.FP32)


def check_all(bits: np.ndarray, dev, scale_ld=None, tile=True, lib="libmxq.so"):
    """Projection, row lift (+ padded scale storage), export, decode and the
    128x128 fold of one weight, each against the oracle."""
    x = to_dev(bits, dev)
    rows, K = bits.shape
    nb = (K + 31) // 32
    scale_ld = scale_ld or nb
    tdt, odt = out_dtype_of(bits)
    assert_bits(to_host(mxq.mxq_fake_quantize_mxfp4(x, lib=lib)), oracle.fake_quantize_mxfp4(bits, threads=THREADS),
                "projection")
    scale = torch.full((rows, scale_ld), 0xA5, dtype=torch.uint8, device=dev)
    data, scale = mxq.mxq_mxfp4_to_mxfp8_row(x, scale=scale, lib=lib)
    wd, ws = oracle.mxfp4_to_mxfp8_row(bits, scale_ld=scale_ld, threads=THREADS, fill=0xA5)
    assert_bits(to_host(data), wd, "row payload")
    assert_bits(to_host(scale), ws, "row scale codes (padding untouched)")
    comp = mxq.export_components(data, scale, (rows, K), lib=lib)
    assert_bits(to_host(comp.scale_inv), oracle.export_mxfp8(ws, K), "exported scales")
    assert comp.data.dtype == torch.float8_e4m3fn and comp.data.data_ptr() == data.data_ptr()
    dec = mxq.mxq_dequantize(data, comp.scale_inv, out_dtype=tdt, lib=lib)
    assert_bits(to_host(dec), oracle.dequantize(wd, ws[:, :nb], out_dtype=odt, threads=THREADS), "row decode")
    if tile:
        bd, tc = mxq.mxq_mxfp4_to_fp8_block128(x, lib=lib)
        wbd, wtc = oracle.mxfp4_to_fp8_block128(bits, threads=THREADS)
        assert_bits(to_host(bd), wbd, "128x128 payload")
        assert_bits(to_host(tc), wtc, "tile codes")
        dec = mxq.mxq_dequantize(bd, tc, layout=mxq.MXQ_SCALE_TILE_128X128, out_dtype=tdt, lib=lib)
        assert_bits(to_host(dec), oracle.dequantize(wbd, wtc, layout=oracle.TILE_128X128, out_dtype=odt,
                                                    threads=THREADS), "tile decode")


# ------------------------------------------------------------------ the five workloads

def test_c1_small(dev):
    check_all(W.c1_small(), dev, scale_ld=4)


@pytest.mark.parametrize("natural", [False, True])
def test_c2_exhaustive(dev, natural):
    check_all(W.c2_exhaustive(natural=natural), dev, scale_ld=4)


def test_c2_planted(dev):
    check_all(W.c2_planted(), dev)


def test_fp32_fuzz(dev):
    check_all(W.fp32_fuzz(1 << 18).reshape(-1, 256), dev)


def test_c3_spread_sweep(dev):
    check_all(W.c3_spread(), dev)


@pytest.mark.parametrize("scale_ld", [256, 260])
def test_c4_headline(dev, scale_ld):
    """8192 x 8192 bf16, the whole weight: unpadded scale storage (the export is a
    view) and storage padded to 260 columns, the launch configuration the bench
    times (the export copies)."""
    check_all(W.c4_headline(), dev, scale_ld=scale_ld)


@pytest.mark.parametrize("which", ["up", "down", "up_master"])
def test_c5_mlp_full(dev, which):
    """The MLP-shaped weights -- 28672 x 8192 and 8192 x 28672 bf16 and the fp32
    master of the first -- compared in full, every output of every kernel
    against the oracle: projection, row lift into scale storage padded by 4
    columns (the padding checked untouched, so the export copies), the export,
    the row decode, the 128x128 fold (every band) and its decode."""
    bits = W.c5_mlp(which)
    check_all(bits, dev, scale_ld=(bits.shape[1] + 31) // 32 + 4)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_every_value_at_every_block_exponent(dev, dtype):
    """Each element value meets each scale exponent: for bf16 this is every
    (pattern, e) pair in the domain, so the kernels' rounding (including the
    hardware conversions they use) is checked over its whole input space."""
    check_all(W.value_exponent_pairs(dtype), dev)


@pytest.mark.parametrize("which", ["c1", "planted", "fuzz", "c4"])
def test_fused_projection_and_row_lift(dev, which):
    """One pass writes exactly what the two separate calls write (the oracle's
    projection and row lift), including in place."""
    bits = {"c1": W.c1_small, "planted": W.c2_planted, "fuzz": lambda: W.fp32_fuzz(1 << 16).reshape(-1, 128),
            "c4": W.c4_headline}[which]()
    rows, K = bits.shape
    nb = (K + 31) // 32
    x = to_dev(bits, dev)
    scale = torch.full((rows, nb + 3), 0x5A, dtype=torch.uint8, device=dev)
    y, data, scale = mxq.mxq_fake_quantize_mxfp4_with_mxfp8_row(x, scale=scale)
    wd, ws = oracle.mxfp4_to_mxfp8_row(bits, scale_ld=nb + 3, threads=THREADS, fill=0x5A)
    assert_bits(to_host(y), oracle.fake_quantize_mxfp4(bits, threads=THREADS), "fused projection")
    assert_bits(to_host(data), wd, "fused payload")
    assert_bits(to_host(scale), ws, "fused codes")
    if which == "c1":
        mxq.mxq_fake_quantize_mxfp4_with_mxfp8_row(x, y=x)
        assert_bits(to_host(x), oracle.fake_quantize_mxfp4(bits), "fused projection in place")


def test_noop_flag_gates_the_direct_conversions(dev):
    bits = W.c4_headline(shape=(512, 1024))
    x = to_dev(bits, dev)
    wd, ws = oracle.mxfp4_to_mxfp8_row(bits)
    wbd, wtc = oracle.mxfp4_to_fp8_block128(bits)
    flag = torch.ones(1, dtype=torch.int32, device=dev)
    data = torch.full((512, 1024), 0x11, dtype=torch.uint8, device=dev)
    scale = torch.full((512, 32), 0x22, dtype=torch.uint8, device=dev)
    bdata = torch.full((512, 1024), 0x33, dtype=torch.uint8, device=dev)
    tc = torch.full((4, 8), 0x44, dtype=torch.uint8, device=dev)
    mxq.mxq_mxfp4_to_mxfp8_row(x, data, scale, noop=flag)
    mxq.mxq_mxfp4_to_fp8_block128(x, bdata, tc, noop=flag)
    assert (to_host(data) == 0x11).all() and (to_host(scale) == 0x22).all()
    assert (to_host(bdata) == 0x33).all() and (to_host(tc) == 0x44).all()
    flag.zero_()
    mxq.mxq_mxfp4_to_mxfp8_row(x, data, scale, noop=flag)
    mxq.mxq_mxfp4_to_fp8_block128(x, bdata, tc, noop=flag)
    assert_bits(to_host(data), wd, "gated payload")
    assert_bits(to_host(scale), ws, "gated codes")
    assert_bits(to_host(bdata), wbd, "gated 128x128 payload")
    assert_bits(to_host(tc), wtc, "gated tile codes")


def test_noop_flag_inside_a_replayed_graph(dev):
    """A captured update replays conditionally: with the flag set the cached
    outputs keep their previous contents, with it clear they follow the new
    weight.  Eager work and synchronisation between replays; every replay checked."""
    a_bits = W.c4_headline(shape=(256, 2048))
    b_bits = W.c1_small()[:, :32]
    b_bits = np.ascontiguousarray(np.tile(b_bits, (3, 64))[:256, :2048])
    x = to_dev(a_bits, dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    data = torch.empty((256, 2048), dtype=torch.uint8, device=dev)
    scale = torch.empty((256, 64), dtype=torch.uint8, device=dev)
    bdata = torch.empty((256, 2048), dtype=torch.uint8, device=dev)
    tc = torch.empty((2, 16), dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm up outside the graph
        mxq.mxq_mxfp4_to_mxfp8_row(x, data, scale, noop=flag)
        mxq.mxq_mxfp4_to_fp8_block128(x, bdata, tc, noop=flag)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mxq.mxq_mxfp4_to_mxfp8_row(x, data, scale, noop=flag)
        mxq.mxq_mxfp4_to_fp8_block128(x, bdata, tc, noop=flag)
    want = {}
    for name, bits in (("a", a_bits), ("b", b_bits)):
        want[name] = oracle.mxfp4_to_mxfp8_row(bits) + oracle.mxfp4_to_fp8_block128(bits)
    for step, (src, skip, expect) in enumerate([("a", 0, "a"), ("b", 1, "a"), ("b", 0, "b"), ("a", 1, "b"),
                                                ("a", 0, "a")]):
        x.copy_(to_dev(a_bits if src == "a" else b_bits, dev))      # eager work between replays
        flag.fill_(skip)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        wd, ws, wbd, wtc = want[expect]
        assert_bits(to_host(data), wd, f"replay {step} payload")
        assert_bits(to_host(scale), ws, f"replay {step} codes")
        assert_bits(to_host(bdata), wbd, f"replay {step} 128x128 payload")
        assert_bits(to_host(tc), wtc, f"replay {step} tile codes")


def test_whole_step_in_a_replayed_graph(dev):
    """The whole path -- projection, row lift into padded scale storage, export,
    128x128 fold and both decodes -- captured in one HIP graph and replayed with
    a changing weight, eager work and synchronisation between replays; every
    replay's outputs against the oracle, bit for bit."""
    rows, K, sld = 384, 1536, 52                      # 3 tile bands x 12 tile columns; storage padded by 4
    nb = K // 32
    weights = [W.c4_headline(seed=21, shape=(rows, K)), W.c3_spread(seed=22, shape=(rows, K)).view(np.uint32)]
    weights[1] = np.ascontiguousarray((weights[1] >> 16).astype(np.uint16))   # bf16 of the spread corpus, truncated
    x = to_dev(weights[0], dev)
    y = torch.empty_like(x)
    data = torch.empty((rows, K), dtype=torch.uint8, device=dev)
    scale = torch.zeros((rows, sld), dtype=torch.uint8, device=dev)
    comp = torch.empty((rows, nb), dtype=torch.uint8, device=dev)
    bdata = torch.empty((rows, K), dtype=torch.uint8, device=dev)
    tc = torch.empty((rows // 128, K // 128), dtype=torch.uint8, device=dev)
    dec_r = torch.empty_like(x)
    dec_t = torch.empty_like(x)

    def step():
        mxq.mxq_fake_quantize_mxfp4(x, y)
        mxq.mxq_mxfp4_to_mxfp8_row(x, data, scale)
        mxq.mxq_export_mxfp8(data, scale, K, comp)
        mxq.mxq_mxfp4_to_fp8_block128(x, bdata, tc)
        mxq.mxq_dequantize(data, comp, out=dec_r)
        mxq.mxq_dequantize(bdata, tc, layout=mxq.MXQ_SCALE_TILE_128X128, out=dec_t)

    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm up outside the graph
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for replay, which in enumerate([0, 1, 1, 0, 1]):
        bits = weights[which]
        x.copy_(to_dev(bits, dev))                  # eager work between replays
        for t in (y, data, scale[:, :nb], comp, bdata, tc, dec_r, dec_t):   # the storage's padding stays
            t.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        wd, ws = oracle.mxfp4_to_mxfp8_row(bits, scale_ld=sld)
        wbd, wtc = oracle.mxfp4_to_fp8_block128(bits)
        assert_bits(to_host(y), oracle.fake_quantize_mxfp4(bits), f"replay {replay} projection")
        assert_bits(to_host(data), wd, f"replay {replay} row payload")
        assert_bits(to_host(scale)[:, :nb], ws[:, :nb], f"replay {replay} row codes")
        assert not to_host(scale)[:, nb:].any(), f"replay {replay}: scale padding written"
        assert_bits(to_host(comp), oracle.export_mxfp8(ws, K), f"replay {replay} export")
        assert_bits(to_host(bdata), wbd, f"replay {replay} 128x128 payload")
        assert_bits(to_host(tc), wtc, f"replay {replay} tile codes")
        assert_bits(to_host(dec_r), oracle.dequantize(wd, ws[:, :nb], out_dtype=oracle.BF16), f"replay {replay} row decode")
        assert_bits(to_host(dec_t), oracle.dequantize(wbd, wtc, layout=oracle.TILE_128X128, out_dtype=oracle.BF16),
                    f"replay {replay} tile decode")


# ------------------------------------------------------------------ packed MXFP4 (deployment format)

def check_packed(bits: np.ndarray, dev, scale_ld=None):
    rows, K = bits.shape
    nb = (K + 31) // 32
    scale_ld = scale_ld or nb
    x = to_dev(bits, dev)
    tdt, odt = out_dtype_of(bits)
    scale = torch.full((rows, scale_ld), 0xC3, dtype=torch.uint8, device=dev)
    packed, scale = mxq.mxq_quantize_mxfp4(x, scale=scale)
    wp, ws = oracle.quantize_mxfp4(bits, scale_ld=scale_ld, threads=THREADS, fill=0xC3)
    assert_bits(to_host(packed), wp, "packed nibbles")
    assert_bits(to_host(scale), ws, "packed codes (padding untouched)")
    assert_bits(to_host(mxq.mxq_dequantize_mxfp4(packed, scale, K, out_dtype=tdt)),
                oracle.dequantize_mxfp4(wp, ws, K, out_dtype=odt, threads=THREADS), "packed decode")
    d, c = mxq.mxq_mxfp4_packed_to_mxfp8_row(packed, scale, K)
    wd, wc = oracle.mxfp4_packed_to_mxfp8_row(wp, ws, K, threads=THREADS)
    assert_bits(to_host(d), wd, "row lift from packed")
    assert_bits(to_host(c), wc, "row codes from packed")
    d, c = mxq.mxq_mxfp4_packed_to_fp8_block128(packed, scale, K)
    wd, wc = oracle.mxfp4_packed_to_fp8_block128(wp, ws, K, threads=THREADS)
    assert_bits(to_host(d), wd, "128x128 payload from packed")
    assert_bits(to_host(c), wc, "tile codes from packed")


@pytest.mark.parametrize("name", ["c1", "c2", "c2_natural", "planted", "fuzz", "c3", "c4", "pairs_bf16", "pairs_fp32"])
def test_packed_mxfp4(dev, name):
    bits = {"c1": W.c1_small, "c2": W.c2_exhaustive, "c2_natural": lambda: W.c2_exhaustive(natural=True),
            "planted": W.c2_planted, "fuzz": lambda: W.fp32_fuzz(1 << 18).reshape(-1, 256), "c3": W.c3_spread,
            "c4": W.c4_headline, "pairs_bf16": lambda: W.value_exponent_pairs("bf16"),
            "pairs_fp32": lambda: W.value_exponent_pairs("fp32")}[name]()
    check_packed(bits, dev, scale_ld=4 if name in ("c1", "c2", "c2_natural") else None)


def test_packed_above_the_cap(dev):
    """Every bf16 magnitude above 6*2^125 as a block amax (scale 2^126), with
    every smaller pattern as the other elements."""
    big = np.arange(0x7F41, 0x7F80, dtype=np.uint16)
    rest = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    g = np.random.default_rng(3)
    rows = []
    for i in range(0, len(rest), 31):
        chunk = rest[i:i + 31]
        blk = np.zeros(32, dtype=np.uint16)
        blk[0] = big[(i // 31) % len(big)] | (0x8000 if (i // 31) % 2 else 0)
        blk[1:1 + len(chunk)] = chunk ^ (g.integers(0, 2, len(chunk)).astype(np.uint16) << 15)
        rows.append(blk)
    bits = np.stack(rows).reshape(-1, 256 if len(rows) % 8 == 0 else 32)
    check_packed(np.ascontiguousarray(bits), dev)


def test_packed_every_code_and_nibble(dev):
    rows, K = 256, 128
    packed = np.tile(np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], dtype=np.uint8), (rows, 8))
    scale = np.arange(256, dtype=np.uint8).reshape(rows, 1).repeat(4, axis=1)
    scale[::7, 1] = 3
    pd, sd = to_dev(packed, dev), to_dev(scale, dev)
    for tdt, odt in ((torch.bfloat16, oracle.BF16), (torch.float32, oracle.FP32)):
        assert_bits(to_host(mxq.mxq_dequantize_mxfp4(pd, sd, K, out_dtype=tdt)),
                    oracle.dequantize_mxfp4(packed, scale, K, out_dtype=odt), f"decode every code {odt}")
    d, c = mxq.mxq_mxfp4_packed_to_mxfp8_row(pd, sd, K)
    wd, wc = oracle.mxfp4_packed_to_mxfp8_row(packed, scale, K)
    assert_bits(to_host(d), wd, "row lift every code")
    assert_bits(to_host(c), wc, "row codes every code")
    d, c = mxq.mxq_mxfp4_packed_to_fp8_block128(pd, sd, K)
    wd, wc = oracle.mxfp4_packed_to_fp8_block128(packed, scale, K)
    assert_bits(to_host(d), wd, "fold every code")
    assert_bits(to_host(c), wc, "tile codes every code")


@pytest.mark.parametrize("K", [1, 7, 9, 31, 33, 100, 130, 257, 2500])   # 2500: both fp32-output lane groups
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_packed_ragged(dev, K, dtype):
    rows = 131
    if dtype == "bf16":
        flat = np.tile(W.c2_exhaustive().reshape(-1), (rows * K) // 65536 + 1)
    else:
        flat = W.fp32_fuzz(((rows * K + 31) // 32) * 32).reshape(-1)
    check_packed(np.ascontiguousarray(flat[: rows * K].reshape(rows, K)), dev, scale_ld=(K + 31) // 32 + 1)


@pytest.mark.parametrize("name", ["normal", "normal_elementwise", "spread"])
def test_packed_fold_partial_window(dev, name):
    """The fold from packed reorders its workgroups within whole windows of 64;
    these grids hold several whole windows and a partial last one (and ragged
    bands), so every work item must still be done exactly once."""
    bits = {"normal": lambda: W.c4_headline(seed=11, shape=(2951, 4608)),              # 24 bands x 9 groups = 216
            "normal_elementwise": lambda: W.c4_headline(seed=12, shape=(2951, 4500)),  # K % 16 != 0: 24 x 9 = 216
            "spread": lambda: W.c3_spread(seed=13, shape=(2944, 4608))}[name]()       # 23 x 9 = 207
    check_packed(bits, dev)


# ------------------------------------------------------------------ invariants on the device

def test_decode_of_row_is_projection_c4(dev):
    """The pages' invariant, checked on the device at the headline size."""
    x = to_dev(W.c4_headline(), dev)
    y = mxq.mxq_fake_quantize_mxfp4(x)
    data, scale = mxq.mxq_mxfp4_to_mxfp8_row(x)
    dec = mxq.mxq_dequantize(data, scale)
    assert torch.equal(dec.view(torch.int16), y.view(torch.int16))


# ------------------------------------------------------------------ edges

@pytest.mark.parametrize("K", [1, 7, 8, 16, 31, 33, 48, 100, 130, 257, 2049])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ragged_shapes(dev, K, dtype):
    g = np.random.default_rng(K)
    rows = 131
    if dtype == "bf16":
        flat = np.tile(W.c2_exhaustive().reshape(-1), (rows * K) // 65536 + 1)
    else:
        flat = W.fp32_fuzz(((rows * K + 31) // 32) * 32).reshape(-1)
    bits = np.ascontiguousarray(flat[: rows * K].reshape(rows, K))
    check_all(bits, dev, scale_ld=(K + 31) // 32 + int(g.integers(0, 3)))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_strided_and_misaligned_views(dev, dtype):
    """ld > K and base pointers one element off the 16-byte grid."""
    base = W.c2_planted() if dtype == "bf16" else W.fp32_fuzz(64 * 200).reshape(64, 200)
    big = to_dev(np.ascontiguousarray(np.tile(base, (1, 4))), dev)    # wider than K + 3
    K = 96
    for off in (0, 1, 3):
        view = big[:, off:off + K]                                     # row stride 3 * width
        bits = to_host(view)
        assert view.stride(0) > K
        assert_bits(to_host(mxq.mxq_fake_quantize_mxfp4(view)), oracle.fake_quantize_mxfp4(bits), f"proj off={off}")
        d, s = mxq.mxq_mxfp4_to_mxfp8_row(view)
        wd, ws = oracle.mxfp4_to_mxfp8_row(bits)
        assert_bits(to_host(d), wd, f"row off={off}")
        assert_bits(to_host(s), ws, f"codes off={off}")
        bd, tc = mxq.mxq_mxfp4_to_fp8_block128(view)
        wbd, wtc = oracle.mxfp4_to_fp8_block128(bits)
        assert_bits(to_host(bd), wbd, f"block128 off={off}")
        assert_bits(to_host(tc), wtc, f"tile codes off={off}")
        y = torch.empty((64, 2 * K), dtype=view.dtype, device=dev)[:, 1:K + 1]   # misaligned strided output
        mxq.mxq_fake_quantize_mxfp4(view, y)
        assert_bits(to_host(y), oracle.fake_quantize_mxfp4(bits), f"proj into strided y off={off}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_code_storage_alignment(dev, dtype):
    """Whole-step rows (K = 4096: whole steps of the row lift, the MXFP4 encode
    and the row lift from packed MXFP4) with the code storage at every
    alignment: a base pointer 0-3 bytes off and row strides nb .. nb + 4.  The
    full-step kernels gather a group of lanes' codes into one 4-byte (2-byte
    for the fp32 row lift and encode) store where the storage is aligned to
    that width, and store bytes otherwise; each against the oracle, with the
    storage around the codes untouched."""
    src = W.c2_planted() if dtype == "bf16" else W.c2_planted_fp32()
    rows, K = 64, 4096
    bits = np.ascontiguousarray(np.resize(src.reshape(-1), rows * K).reshape(rows, K))
    x = to_dev(bits, dev)
    nb = K // 32
    wd, ws = oracle.mxfp4_to_mxfp8_row(bits, threads=THREADS)
    wp, wps = oracle.quantize_mxfp4(bits, threads=THREADS)
    wpd, wpc = oracle.mxfp4_packed_to_mxfp8_row(wp, wps, K, threads=THREADS)
    pk, pks = to_dev(wp, dev), to_dev(wps, dev)
    for off in (0, 1, 2, 3):
        for ld in (nb, nb + 1, nb + 2, nb + 4):
            def storage():
                buf = torch.full((rows * ld + 8,), 0x5A, dtype=torch.uint8, device=dev)
                return buf, buf[off:off + rows * ld].view(rows, ld)[:, :nb]

            def expect(codes):
                want = np.full(rows * ld + 8, 0x5A, np.uint8)
                want[off:off + rows * ld].reshape(rows, ld)[:, :nb] = codes
                return want

            what = f"off={off} ld={ld}"
            buf, scale = storage()
            data, _ = mxq.mxq_mxfp4_to_mxfp8_row(x, scale=scale)
            assert_bits(to_host(data), wd, f"row payload {what}")
            assert_bits(to_host(buf), expect(ws), f"row codes {what}")
            buf, scale = storage()
            packed, _ = mxq.mxq_quantize_mxfp4(x, scale=scale)
            assert_bits(to_host(packed), wp, f"packed nibbles {what}")
            assert_bits(to_host(buf), expect(wps), f"packed codes {what}")
            buf, scale = storage()
            data, _ = mxq.mxq_mxfp4_packed_to_mxfp8_row(pk, pks, K, scale_out=scale)
            assert_bits(to_host(data), wpd, f"row-from-packed payload {what}")
            assert_bits(to_host(buf), expect(wpc), f"row-from-packed codes {what}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rows,K", [(1, 2048), (2, 2048), (3, 2048), (4, 2048), (33, 2048), (33, 4096), (129, 1024),
                                    (127, 6144), (128, 128), (256, 3072)])
def test_step_boundary_shapes(dev, dtype, rows, K):
    """Shapes at the edges of the kernels' whole-step forms: the row lift, the
    MXFP4 encode and the packed row lift take their check-free forms only for
    whole steps (2048 bf16 / 1024 fp32 elements, 1024 packed) and a step
    count that is a multiple of the steps per workgroup (2, 2 and 4), the
    fp32 fold only for whole 128-row bands.  The other step totals, single
    rows and partial bands take the checked forms; both against the
    oracle."""
    src = W.c2_planted() if dtype == "bf16" else W.c2_planted_fp32()
    bits = np.ascontiguousarray(np.resize(src.reshape(-1), rows * K).reshape(rows, K))
    check_all(bits, dev, scale_ld=(K + 31) // 32 + 4)
    check_packed(bits, dev)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rows,K", [(1024, 8320), (640, 16256), (1000, 4100), (256, 8192)])
def test_fold_tile_order_tails(dev, dtype, rows, K):
    """The 128x128 fold deals its tiles to the XCDs in runs (8 side-by-side
    tiles per XCD for bf16, 4 for fp32, so groups of 64 or 32 tiles), and the
    last, partial group keeps the plain order.  Tile counts 520, 635, 264 and
    128 leave tails of 8, 59, 8 and 0 tiles (bf16) and 8, 27, 8 and 0 (fp32);
    every tile against the oracle."""
    src = W.c2_planted() if dtype == "bf16" else W.c2_planted_fp32()
    bits = np.ascontiguousarray(np.resize(src.reshape(-1), rows * K).reshape(rows, K))
    check_all(bits, dev, scale_ld=(K + 31) // 32 + 4)


@pytest.mark.parametrize("K", [512, 640, 4096, 4128])   # ceil(K/32) = 16, 20, 128, 129
def test_export_every_unit_width(dev, K):
    """The unpadded export against the oracle for code rows of 16, 20, 128 and
    129 bytes, padded strides ceil(K/32) + 0, 1, 4 and 16, and storage and
    output bases 0, 1 or 4 bytes off: 16-byte units, 4-byte units, the
    four-4-byte-units-to-one-16-byte-store form and single bytes all run, and
    the bytes around the output stay untouched."""
    rows = 37
    nb = (K + 31) // 32
    rng = np.random.default_rng(K)
    data = torch.zeros((rows, K), dtype=torch.uint8, device=dev)
    for pad in (0, 1, 4, 16):
        ld = nb + pad
        codes = rng.integers(0, 256, size=(rows, ld), dtype=np.uint8)
        for soff in (0, 1, 4):
            sbuf = torch.from_numpy(np.concatenate([np.zeros(soff, np.uint8), codes.reshape(-1)])).to(dev)
            storage = sbuf[soff:].view(rows, ld)
            for ooff in (0, 1, 4):
                obuf = torch.full((rows * nb + 8,), 0xA5, dtype=torch.uint8, device=dev)
                out = obuf[ooff:ooff + rows * nb].view(rows, nb)
                mxq.mxq_export_mxfp8(data, storage, K, scale_out=out)
                want = np.full(rows * nb + 8, 0xA5, np.uint8)
                want[ooff:ooff + rows * nb] = oracle.export_mxfp8(codes, K).reshape(-1)
                assert_bits(to_host(obuf), want, f"export K={K} ld={ld} soff={soff} ooff={ooff}")


def test_in_place_projection(dev):
    bits = W.c1_small()
    x = to_dev(bits, dev)
    mxq.mxq_fake_quantize_mxfp4(x, x)
    assert_bits(to_host(x), oracle.fake_quantize_mxfp4(bits), "in-place projection")


def test_empty_shapes(dev):
    for shape in ((0, 32), (5, 0), (0, 0)):
        x = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        assert mxq.mxq_fake_quantize_mxfp4(x).shape == shape
        d, s = mxq.mxq_mxfp4_to_mxfp8_row(x)
        assert d.shape == shape
        bd, tc = mxq.mxq_mxfp4_to_fp8_block128(x)
        assert bd.shape == shape


def test_errors(dev):
    x = torch.zeros((4, 64), dtype=torch.float16, device=dev)
    with pytest.raises(mxq.MxqError) as e:
        mxq.mxq_fake_quantize_mxfp4(x)
    assert e.value.status == mxq.MXQ_ERR_DTYPE
    with pytest.raises(TypeError):
        mxq.fake_quantize_mxfp4(x)
    xb = torch.zeros((4, 64), dtype=torch.bfloat16, device=dev)
    buf = torch.zeros((4, 96), dtype=torch.bfloat16, device=dev)
    with pytest.raises(mxq.MxqError) as e:      # partial overlap of x and y
        mxq.mxq_fake_quantize_mxfp4(buf[:, :64], buf[:, 1:65])
    assert e.value.status == mxq.MXQ_ERR_ALIAS
    with pytest.raises(ValueError, match="must cover"):   # scale storage narrower than ceil(K/32)
        mxq.mxq_mxfp4_to_mxfp8_row(xb, scale=torch.zeros((4, 1), dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        mxq.export_components(None, None, (4, 64))
    # a host operand beside device ones is refused before any launch
    with pytest.raises(ValueError, match="device tensors"):
        mxq.mxq_fake_quantize_mxfp4(xb, torch.zeros((4, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="device tensors"):
        mxq.mxq_mxfp4_to_mxfp8_row(xb, scale=torch.zeros((4, 2), dtype=torch.uint8))


def test_undersized_operands_are_refused(dev):
    """A caller-supplied output (or code input) smaller than the region the
    call touches is refused with ValueError before any launch; the buffers are
    left as they were."""
    x = to_dev(W.c4_headline(shape=(256, 512)), dev)
    u8 = lambda *shape: torch.full(shape, 0x3C, dtype=torch.uint8, device=dev)
    data, scale, bdata, tc = u8(256, 512), u8(256, 16), u8(256, 512), u8(2, 4)
    calls = {
        "projection y": lambda: mxq.mxq_fake_quantize_mxfp4(x, torch.empty(256, 512, dtype=torch.bfloat16, device=dev)[:255]),
        "row codes, too few rows": lambda: mxq.mxq_mxfp4_to_mxfp8_row(x, data, u8(255, 16)),
        "row codes, one row": lambda: mxq.mxq_mxfp4_to_mxfp8_row(x, data, u8(1, 16 * 256)),
        "row codes, too narrow": lambda: mxq.mxq_mxfp4_to_mxfp8_row(x, data, u8(256, 15)),
        "row payload, short": lambda: mxq.mxq_mxfp4_to_mxfp8_row(x, u8(255, 512), scale),
        "fold tile codes": lambda: mxq.mxq_mxfp4_to_fp8_block128(x, bdata, u8(1, 4)),
        "column codes": lambda: mxq.mxq_mxfp4_to_mxfp8_col(x, data, u8(7, 512)),
        "row + column codes": lambda: mxq.mxq_mxfp4_to_mxfp8_row_col(x, data, u8(256, 8), bdata, u8(8, 512)),
        "fused codes": lambda: mxq.mxq_fake_quantize_mxfp4_with_mxfp8_row(x, None, data, u8(128, 16)),
        "export out": lambda: mxq.mxq_export_mxfp8(data, scale, 512, u8(255, 16)),
        "decode out": lambda: mxq.mxq_dequantize(data, scale, out=torch.empty(255, 512, dtype=torch.bfloat16, device=dev)),
        "decode codes": lambda: mxq.mxq_dequantize(data, u8(256, 15)),
        "decode tile codes": lambda: mxq.mxq_dequantize(data, u8(2, 3), layout=mxq.MXQ_SCALE_TILE_128X128),
        "packed encode codes": lambda: mxq.mxq_quantize_mxfp4(x, u8(256, 256), u8(200, 16)),
        "packed decode out": lambda: mxq.mxq_dequantize_mxfp4(u8(256, 256), scale, 512,
                                                              out=torch.empty(1, 512, dtype=torch.float32, device=dev)),
        "packed codes in": lambda: mxq.mxq_dequantize_mxfp4(u8(256, 256), u8(256, 8), 512),
        "packed row lift payload": lambda: mxq.mxq_mxfp4_packed_to_mxfp8_row(u8(256, 256), scale, 512, u8(128, 512)),
        "packed row lift codes": lambda: mxq.mxq_mxfp4_packed_to_mxfp8_row(u8(256, 256), scale, 512, data, u8(256, 1)),
        "packed fold tile codes": lambda: mxq.mxq_mxfp4_packed_to_fp8_block128(u8(256, 256), scale, 512, bdata, u8(2, 1)),
        "grouped row codes": lambda: mxq.mxq_mxfp4_to_mxfp8_row_grouped([x, x], [data, bdata], [scale, u8(64, 16)]),
        "grouped fold tile codes": lambda: mxq.mxq_mxfp4_to_fp8_block128_grouped([x], [bdata], [u8(1, 1)]),
        "grouped decode out": lambda: mxq.mxq_dequantize_grouped([data], [scale], outs=[torch.empty(3, 512, dtype=torch.bfloat16, device=dev)]),
        "grouped packed codes": lambda: mxq.mxq_quantize_mxfp4_grouped([x], [u8(256, 256)], [u8(256, 2)]),
    }
    for what, call in calls.items():
        with pytest.raises(ValueError):
            call()
            raise AssertionError(f"{what}: accepted")
    torch.cuda.synchronize()
    for t in (data, scale, bdata, tc):
        assert (to_host(t) == 0x3C).all()


def test_decode_every_byte_and_code(dev):
    """Planted payloads and codes: every (code, byte) pair, both FP8 formats,
    both output dtypes, both scale layouts."""
    data = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    codes_row = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 8, axis=1)
    dd, dr = to_dev(data, dev), to_dev(codes_row, dev)
    for fmt_dev, fmt_orc in ((mxq.MXQ_E4M3, oracle.E4M3), (mxq.MXQ_E5M2, oracle.E5M2)):
        for tdt, odt in ((torch.bfloat16, oracle.BF16), (torch.float32, oracle.FP32)):
            got = to_host(mxq.mxq_dequantize(dd, dr, fmt=fmt_dev, out_dtype=tdt))
            assert_bits(got, oracle.dequantize(data, codes_row, fp8=fmt_orc, out_dtype=odt), f"decode {fmt_orc} {odt}")
    # tile layout: 256 rows = 2 tile rows, 256 cols = 2 tile cols -> 4 codes
    tcodes = np.array([[0, 255], [1, 254]], dtype=np.uint8)
    got = to_host(mxq.mxq_dequantize(dd, to_dev(tcodes, dev), layout=mxq.MXQ_SCALE_TILE_128X128, out_dtype=torch.float32))
    assert_bits(got, oracle.dequantize(data, tcodes, layout=oracle.TILE_128X128, out_dtype=oracle.FP32), "tile decode")


@pytest.mark.parametrize("variant", ["libmxq_fastmath.so", "libmxq_o1.so", "libmxq_o0.so"])
def test_build_variants_identical_bits(dev, variant):
    """Same source built with fast-math + flushed denormals, at -O1 and at -O0:
    the same bits (the pages rebuild with fast math and compare)."""
    for bits in (W.c2_exhaustive(), W.c2_planted(), W.fp32_fuzz(1 << 16).reshape(-1, 128), W.c3_spread()[:256, :512]):
        check_all(np.ascontiguousarray(bits), dev, lib=variant)


def test_row_longer_than_2gb(dev):
    """Maximum-size edge: one bf16 row of 2^30 + 48 elements (2 GB + 96 bytes,
    beyond the 32-bit byte offsets of the vectorised projection store), so the
    projection and the fused pass take their element-wise paths.  Compared on
    sampled blocks: the start, the blocks around the 2^30-element (2^31-byte)
    mark, and the partial last block."""
    K = (1 << 30) + 48
    pat = W.c2_exhaustive().reshape(-1)
    bits = np.resize(pat, K).reshape(1, K)
    x = to_dev(bits, dev)
    y = mxq.mxq_fake_quantize_mxfp4(x)
    data, scale = mxq.mxq_mxfp4_to_mxfp8_row(x)
    torch.cuda.synchronize()
    for c0, c1 in ((0, 4096), ((1 << 30) - 2048, (1 << 30) + 2048), (K - 4096 - 16, K)):
        sub = np.ascontiguousarray(bits[:, c0:c1])
        assert_bits(to_host(y[:, c0:c1]), oracle.fake_quantize_mxfp4(sub), f"projection [{c0}, {c1})")
        wd, ws = oracle.mxfp4_to_mxfp8_row(sub)
        assert_bits(to_host(data[:, c0:c1]), wd, f"row payload [{c0}, {c1})")
        assert_bits(to_host(scale[:, c0 // 32:(c1 + 31) // 32]), ws, f"row codes [{c0}, {c1})")
    del y, data, scale
    torch.cuda.empty_cache()
    # the fused pass, whose projection stores share the 32-bit offset limit
    y, data, scale = mxq.mxq_fake_quantize_mxfp4_with_mxfp8_row(x)
    torch.cuda.synchronize()
    for c0, c1 in ((0, 4096), ((1 << 30) - 2048, (1 << 30) + 2048), (K - 4096 - 16, K)):
        sub = np.ascontiguousarray(bits[:, c0:c1])
        assert_bits(to_host(y[:, c0:c1]), oracle.fake_quantize_mxfp4(sub), f"fused projection [{c0}, {c1})")
        wd, ws = oracle.mxfp4_to_mxfp8_row(sub)
        assert_bits(to_host(data[:, c0:c1]), wd, f"fused row payload [{c0}, {c1})")
        assert_bits(to_host(scale[:, c0 // 32:(c1 + 31) // 32]), ws, f"fused row codes [{c0}, {c1})")
    del x, y, data, scale
    torch.cuda.empty_cache()


def test_concurrent_callers_on_their_own_streams(dev):
    """The library holds no state: two host threads, each on its own stream and
    its own weight, interleave the projection, row lift, fold and decode many
    times; every output matches the oracle."""
    import threading
    weights = [W.c4_headline(seed=21, shape=(512, 1024)), W.fp32_fuzz(1 << 17).reshape(512, 256)]
    want = []
    for bits in weights:
        wd, ws = oracle.mxfp4_to_mxfp8_row(bits, threads=THREADS)
        wbd, wtc = oracle.mxfp4_to_fp8_block128(bits, threads=THREADS)
        odt = oracle.FP32 if bits.dtype == np.uint32 else oracle.BF16
        want.append((oracle.fake_quantize_mxfp4(bits, threads=THREADS), wd, ws, wbd, wtc,
                     oracle.dequantize(wd, ws, out_dtype=odt, threads=THREADS)))
    errors, results = [], [None, None]

    def worker(i):
        try:
            x = to_dev(weights[i], dev)
            stream = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(stream):
                for _ in range(20):
                    y = mxq.mxq_fake_quantize_mxfp4(x)
                    d, s = mxq.mxq_mxfp4_to_mxfp8_row(x)
                    bd, tc = mxq.mxq_mxfp4_to_fp8_block128(x)
                    dec = mxq.mxq_dequantize(d, s, out_dtype=x.dtype)
            stream.synchronize()
            results[i] = (y, d, s, bd, tc, dec)
        except Exception as e:      # reported from the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(2):
        for got, exp, what in zip(results[i], want[i], ("projection", "payload", "codes", "128x128 payload",
                                                         "tile codes", "decode")):
            assert_bits(to_host(got), exp, f"caller {i}: {what}")
