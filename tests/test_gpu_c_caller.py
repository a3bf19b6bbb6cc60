"""The library from a plain C program (tests/c/c_caller.c): no PyTorch, only the
HIP runtime's C API and include/mxq.h.  The program runs the whole path on a
ragged bf16 weight on a stream of its own; its outputs must equal the oracle's
bit for bit."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "c_caller")


def test_plain_c_caller_runs_the_path(tmp_path):
    if not os.path.exists(EXE):
        raise FileNotFoundError(f"{EXE} is not built; run __graft_entry__.build()")
    # 3 tile bands (the last partial), 8 tile columns (the last partial), a 1x32
    # block of 8 at the end of each row, scale storage padded by 4 columns
    rows, K, sld = 300, 1000, 36
    nb, tr, tcn = (K + 31) // 32, (rows + 127) // 128, (K + 127) // 128
    bits = W.c4_headline(seed=31, shape=(rows, K))
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    bits.astype("<u2").tofile(src)
    print(f"c_caller {rows}x{K} scale_ld {sld}", flush=True)
    r = subprocess.run([EXE, str(rows), str(K), str(sld), str(src), str(dst)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    out = np.fromfile(dst, dtype=np.uint8)
    sizes = [2 * rows * K, rows * K, rows * nb, rows * K, tr * tcn, 2 * rows * K, 2 * rows * K]
    assert out.size == sum(sizes)
    parts, at = [], 0
    for n in sizes:
        parts.append(out[at:at + n])
        at += n
    y, data, comp, bdata, tc, dec_r, dec_t = parts
    wd, ws = oracle.mxfp4_to_mxfp8_row(bits, scale_ld=sld)
    wbd, wtc = oracle.mxfp4_to_fp8_block128(bits)
    want = {
        "projection": (y.view("<u2").reshape(rows, K), oracle.fake_quantize_mxfp4(bits)),
        "row payload": (data.reshape(rows, K), wd),
        "exported codes": (comp.reshape(rows, nb), oracle.export_mxfp8(ws, K)),
        "128x128 payload": (bdata.reshape(rows, K), wbd),
        "tile codes": (tc.reshape(tr, tcn), wtc),
        "row decode": (dec_r.view("<u2").reshape(rows, K), oracle.dequantize(wd, ws[:, :nb], out_dtype=oracle.BF16)),
        "tile decode": (dec_t.view("<u2").reshape(rows, K),
                        oracle.dequantize(wbd, wtc, layout=oracle.TILE_128X128, out_dtype=oracle.BF16)),
    }
    for what, (got, exp) in want.items():
        assert got.shape == exp.shape, what
        assert np.array_equal(got, exp.astype(got.dtype, copy=False)), f"{what} differs from the oracle"
