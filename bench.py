"""Throughput of the block-scaled weight-quantization path on one MI355X.

One step = one pass of the whole path over the 8192 x 8192 bf16 weight
(N(0, 0.02), seed 1; --shape and --weight below name the other weights):
  proj      MXFP4 projection, bf16 -> bf16
  row       direct MXFP8 rowwise lift (E4M3 payload + E8M0 codes, scale storage
            padded to 260 columns so the export has to copy)
  export    unpadded [8192, 256] scale export
  block128  direct 128x128 blockwise FP8 (E4M3 payload + tile codes)
  dec_row   decode of the rowwise payload -> bf16
  dec_tile  decode of the blockwise payload -> bf16
Inputs are resident in HBM before timing starts.  Six buffer sets rotate so that
a buffer is read again only after more than 1 GB of other traffic (the
Infinity Cache cannot serve repeated reads).  The K timed passes run
kernel-major (each kernel K times back to back, then the next), which is the
same work as K step-major passes; `value` is the steps' algorithmic bytes over
their wall time, and per-kernel times come from HIP events recorded around each
kernel's burst on the stream the kernels are launched on: "us" is the burst's
mean per launch.  After the timed region a separate pass gives "us_median" /
"us_min", the median / minimum over 5 sub-bursts of 5 launches.  Kernels
outside the step (the fused passes, packed MXFP4, columnwise) are timed the
same way after the step's timed region, and so are the access-shape reference
kernels of libmxq_shapes.so ("access_shapes": each moves one kernel's bytes in
that kernel's access pattern with no quantization arithmetic, and each kernel
with a shape reports "of_shape", the shape's time over its own; "read" and
"write" are the machine's plain read-only and write-only streams over the
weight's bytes), and the runtime's own device-to-device copy of the weight
("copy_reference", the projection's bytes).
The default of 100 timed steps keeps the fixed cost of the synchronizations
around the timed region (tens of us in all) below 1% of it.

python bench.py [--gpus 1] [--steps 100] [--warmup 5] [--no-cpu] [--calibrate] [--weight bf16|fp32]
                [--shape 8192x8192|28672x8192|8192x28672] [--orders]
(--weight fp32 runs the same step on the fp32 master copy of the weight; bf16 is the headline.
--shape runs the same step on the MLP-shaped weights instead: 28672 x 8192 (N(0,0.02), seed 2; its
fp32 master with --weight fp32) or 8192 x 28672 (seed 3, bf16 only).  The scale storage is always
padded by 4 columns, so the export copies.  --orders adds "orders": every kernel's burst mean per
launch right after a burst of the fold, after a 30 ms idle gap and after a burst of itself.)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import statistics
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
SCALE_PAD = 4                    # padded scale storage: ceil(K/32) plus 4 columns (8192: 260)
GROUPED = (48, 1024, 2048)       # outside the step: grouped calls over 48 weights of 1024 x 2048 (one launch each)
SHAPES = ("8192x8192", "28672x8192", "8192x28672")
NSETS = 6
SUB, SPREAD_BURSTS = 5, 5   # median / min: 5 sub-bursts of 5 launches, after the timed region
ORDER_REPS, ORDER_LAUNCHES = 4, 60   # --orders: bursts of 60 launches, median of 4 repetitions
# The access-shape reference kernels (libmxq_shapes.so, shape codes of include/mxq_shapes.h) timed
# after the step: name -> (shape code, input buffer, code buffer).  Each moves the bytes of the
# kernel named in SHAPE_KERNEL in that kernel's access pattern, with no quantization arithmetic;
# the tile and linear variants split the fold's pattern into its parts (tile-shaped addressing,
# the workgroup-wide barrier, the fold's workgroup), and the read and write streams give the
# machine's read-only and write-only rates.
SHAPES_OF = {"shape_copy16": (0, "x", "scale2"), "shape_row": (1, "x", "scale2"), "shape_row_codes": (2, "x", "scale2"),
             "shape_decode": (3, "data", "scale_c"), "shape_tile": (4, "x", "scale2"),
             "shape_tile_no_barrier": (5, "x", "scale2"), "shape_linear_fold": (6, "x", "scale2"),
             "shape_linear_fold_no_barrier": (7, "x", "scale2"), "shape_packed_row": (8, "packed", "pscale"),
             "shape_read": (9, "x", "scale2"), "shape_write": (10, "x", "scale2"),
             "shape_tile_loads": (11, "x", "scale2"), "shape_linear_loads": (12, "x", "scale2"),
             "shape_tile_stores": (13, "x", "scale2"), "shape_linear_stores": (14, "x", "scale2")}
SHAPE_KERNEL = {"shape_copy16": "proj", "shape_row_codes": "row", "shape_decode": "dec_row", "shape_tile": "block128",
                "shape_packed_row": "packed_to_row"}
# committed rocprofv3 counter summaries of the 8192 x 8192 weight, per dtype
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_8192x8192_{}.txt")
# The device code: the kernels and the divisor header they include.
KERNEL_SOURCES = [os.path.join(ROOT, "microscaling_weight_quantization_amd", "csrc", n)
                  for n in ("mxq.hip", "fastdiv.h")]


def algorithmic_bytes(rows: int, K: int, es: int = 2) -> dict:
    """Bytes each kernel must move (read + write) for a [rows, K] weight of
    es-byte elements (2: bf16, 4: fp32; the decodes write the same dtype)."""
    n = rows * K
    nb = rows * ((K + 31) // 32)
    tiles = ((rows + 127) // 128) * ((K + 127) // 128)
    return {
        "proj": es * n + es * n,
        "row": es * n + n + nb,
        "export": nb + nb,
        "block128": es * n + n + tiles,
        "dec_row": n + nb + es * n,
        "dec_tile": n + tiles + es * n,
    }


def fused_bytes(rows: int, K: int, es: int = 2) -> int:
    """Projection + row lift from one read: es*n in, es*n + n + n/32 out."""
    n = rows * K
    return es * n + es * n + n + rows * ((K + 31) // 32)


def packed_bytes(rows: int, K: int, es: int = 2) -> dict:
    """Bytes of the packed-MXFP4 kernels for a [rows, K] weight of es-byte elements."""
    n, nb = rows * K, rows * ((K + 31) // 32)
    tiles = ((rows + 127) // 128) * ((K + 127) // 128)
    return {"quantize_mxfp4": es * n + n // 2 + nb, "dequantize_mxfp4": n // 2 + nb + es * n,
            "packed_to_row": n // 2 + nb + n + nb, "packed_to_block128": n // 2 + nb + n + tiles}


def col_bytes(rows: int, K: int, es: int = 2) -> dict:
    """Bytes of the columnwise (32x1) kernels for a [rows, K] weight of es-byte elements."""
    n, nb, nc = rows * K, rows * ((K + 31) // 32), ((rows + 31) // 32) * K
    return {"col": es * n + n + nc, "row_col": es * n + n + nb + n + nc, "dec_col": n + nc + es * n}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, weight: str = "bf16"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary of the 8192 x 8192 weight of that dtype, or None if there is none
    or the kernels changed since."""
    try:
        lines = open(COUNTERS_FILE.format(weight)).read().splitlines()
    except OSError:
        return None
    meta = dict(l.split("=", 1) for l in lines if "=" in l and not l.startswith("#"))
    if meta.get("source_sha256_16") != kernel_source_hash():
        return None
    v = meta.get(f"traffic_bytes.{kernel}")
    return int(float(v)) if v else None


def _oracle_pass(bits, threads: int) -> dict:
    """One pass of the six steps through the CPU oracle; returns its outputs
    (the decodes in the weight's own dtype)."""
    import oracle
    odt = oracle.FP32 if bits.dtype.itemsize == 4 else oracle.BF16
    y = oracle.fake_quantize_mxfp4(bits, threads=threads)
    d, s = oracle.mxfp4_to_mxfp8_row(bits, scale_ld=(bits.shape[1] + 31) // 32 + SCALE_PAD, threads=threads)
    c = oracle.export_mxfp8(s, bits.shape[1])
    bd, tc = oracle.mxfp4_to_fp8_block128(bits, threads=threads)
    dr = oracle.dequantize(d, c, out_dtype=odt, threads=threads)
    dt = oracle.dequantize(bd, tc, layout=oracle.TILE_128X128, out_dtype=odt, threads=threads)
    return {"proj": y, "row": d, "export": c, "block128": bd, "tile_codes": tc, "dec_row": dr, "dec_tile": dt}


def host_cpu() -> dict:
    """The host's CPU as /proc/cpuinfo and the scheduler report it: the model
    string, logical CPUs, physical cores (distinct (package, core) pairs), the
    CPUs this process may run on (its affinity set) and the cgroup's CPU
    quota, which caps the time all its threads together may use."""
    model, cores, cur = "unknown", set(), {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model == "unknown":
                    model = v
                elif k in ("physical id", "core id"):
                    cur[k] = v
                elif not k and cur:
                    cores.add((cur.get("physical id"), cur.get("core id")))
                    cur = {}
        if cur:
            cores.add((cur.get("physical id"), cur.get("core id")))
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    quota = None                                   # the cgroup's CPU quota in CPUs (cgroup v2 cpu.max), if any
    try:
        q, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        quota = None if q == "max" else round(int(q) / int(period), 2)
    except (OSError, ValueError):
        pass
    return {"model": model, "logical": os.cpu_count(), "physical": len(cores) or None, "usable": usable,
            "cgroup_cpu_quota": quota}


def cpu_baseline(bits, threads: int, cpu_seconds: float = 12.0, max_passes: int = 8):
    """The CPU oracle over the same workload (whole passes of every step), as is.

    Passes repeat until the process has spent about `cpu_seconds` of CPU time
    (all threads together), so the figure rests on 10-30 s of CPU work.
    Returns the JSON object and the oracle's outputs (for the parity check)."""
    c0, t0, passes = time.process_time(), time.perf_counter(), 0
    while passes < max_passes and (passes == 0 or time.process_time() - c0 < cpu_seconds):
        outputs = _oracle_pass(bits, threads)
        passes += 1
    dt, cpu = time.perf_counter() - t0, time.process_time() - c0
    es = bits.dtype.itemsize
    wname = "fp32" if es == 4 else "bf16"
    total = passes * sum(algorithmic_bytes(*bits.shape, es).values())
    out = {"value": round(total / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "host_cpu": host_cpu(),
           "sample": f"the whole {bits.shape[0]}x{bits.shape[1]} {wname} weight, {passes} pass{'es' if passes > 1 else ''} of all six steps "
                     f"({dt:.1f} s wall, {cpu:.1f} s CPU on {threads} threads)"}
    # the same steps on one thread, over the first 2048 rows
    sub = bits[:2048]
    t0 = time.perf_counter()
    _oracle_pass(sub, 1)
    dt1 = time.perf_counter() - t0
    out["one_thread"] = {"value": round(sum(algorithmic_bytes(*sub.shape, es).values()) / dt1 / 1e9, 3), "unit": "GB/s",
                         "sample": f"rows 0..2047 of the same weight, one pass of all six steps ({dt1:.1f} s)"}
    return out, outputs


def parity(s, want: dict) -> dict:
    """The step's GPU outputs in one buffer set against the oracle's, bit for bit
    (the whole weight, in the timed launch configuration)."""
    import torch

    def host(t):
        t = t.contiguous().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view("uint16")
        if t.dtype == torch.float32:
            return t.view(torch.int32).numpy().view("uint32")
        return t.numpy()

    got = {"proj": host(s["y"]), "row": host(s["data"]), "export": host(s["scale_c"]), "block128": host(s["bdata"]),
           "tile_codes": host(s["tc"]), "dec_row": host(s["dec_r"]), "dec_tile": host(s["dec_t"])}
    res = {k: got[k].shape == want[k].shape and bool((got[k] == want[k]).all()) for k in want}
    return {"bit_exact": all(res.values()), "outputs": res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--weight", choices=["bf16", "fp32"], default="bf16",
                    help="the weight's dtype: bf16 (the headline) or its fp32 master copy")
    ap.add_argument("--shape", choices=SHAPES, default=SHAPES[0],
                    help="the weight's shape: 8192x8192 (the headline) or an MLP-shaped weight")
    ap.add_argument("--orders", action="store_true",
                    help="also time every kernel's burst after a burst of the fold, after an idle gap and after "
                         "a burst of itself (field 'orders')")
    args = ap.parse_args()
    if args.shape == "8192x28672" and args.weight == "fp32":
        ap.error("--shape 8192x28672 has no fp32 master weight (only the 28672x8192 weight has one)")
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library runs on a single MI355X and has no multi-GPU path "
              "(whole rows shard with no communication, so each GPU would run these kernels on its share).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import microscaling_weight_quantization_amd as mxq
    import workloads as W

    dev = torch.device("cuda:0")
    mxq.load()
    fp32 = args.weight == "fp32"
    es = 4 if fp32 else 2
    headline = args.shape == SHAPES[0]
    if headline:
        bits = W.c4_master() if fp32 else W.c4_headline()
    else:
        bits = W.c5_mlp("down" if args.shape == "8192x28672" else "up_master" if fp32 else "up")
    rows, K = bits.shape
    nb = (K + 31) // 32
    scale_ld = nb + SCALE_PAD
    x0 = (torch.from_numpy(bits.view(np.int32)).to(dev).view(torch.float32) if fp32
          else torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16))
    gn, gr, gk = GROUPED
    gen = torch.Generator().manual_seed(4)
    g_host = (torch.randn(gn, gr, gk, generator=gen) * 0.02).to(torch.float32 if fp32 else torch.bfloat16)
    g0 = g_host.to(dev)
    del g_host
    sets = []
    for i in range(NSETS):
        s = {
            "x": x0.clone(),
            "y": torch.empty_like(x0),
            "data": torch.empty((rows, K), dtype=torch.uint8, device=dev),
            "scale": torch.zeros((rows, scale_ld), dtype=torch.uint8, device=dev),
            "scale_c": torch.empty((rows, nb), dtype=torch.uint8, device=dev),
            "bdata": torch.empty((rows, K), dtype=torch.uint8, device=dev),
            "tc": torch.empty(((rows + 127) // 128, (K + 127) // 128), dtype=torch.uint8, device=dev),
            "tc2": torch.empty(((rows + 127) // 128, (K + 127) // 128), dtype=torch.uint8, device=dev),
            "dec_r": torch.empty_like(x0),
            "dec_t": torch.empty_like(x0),
            "dec_c": torch.empty_like(x0),
            "dec_p": torch.empty_like(x0),
            "y2": torch.empty_like(x0),
            "packed": torch.empty((rows, K // 2), dtype=torch.uint8, device=dev),
            "pscale": torch.empty((rows, nb), dtype=torch.uint8, device=dev),
            "data2": torch.empty((rows, K), dtype=torch.uint8, device=dev),
            "scale2": torch.zeros((rows, scale_ld), dtype=torch.uint8, device=dev),
            "cdata": torch.empty((rows, K), dtype=torch.uint8, device=dev),
            "cscale": torch.empty(((rows + 31) // 32, K), dtype=torch.uint8, device=dev),
            "gx": list(g0.clone().unbind(0)),
            "gdata": [torch.empty((gr, gk), dtype=torch.uint8, device=dev) for _ in range(gn)],
            "gscale": [torch.zeros((gr, gk // 32), dtype=torch.uint8, device=dev) for _ in range(gn)],
            "gy": [torch.empty((gr, gk), dtype=g0.dtype, device=dev) for _ in range(gn)],
            "gbdata": [torch.empty((gr, gk), dtype=torch.uint8, device=dev) for _ in range(gn)],
            "gtc": [torch.zeros((gr // 128, gk // 128), dtype=torch.uint8, device=dev) for _ in range(gn)],
            "gdec": [torch.empty((gr, gk), dtype=g0.dtype, device=dev) for _ in range(gn)],
            "gpk": [torch.empty((gr, gk // 2), dtype=torch.uint8, device=dev) for _ in range(gn)],
            "gps": [torch.zeros((gr, gk // 32), dtype=torch.uint8, device=dev) for _ in range(gn)],
        }
        mxq.mxq_mxfp4_to_mxfp8_row(s["x"], s["data"], s["scale"])
        mxq.mxq_export_mxfp8(s["data"], s["scale"], K, s["scale_c"])
        mxq.mxq_mxfp4_to_fp8_block128(s["x"], s["bdata"], s["tc"])
        mxq.mxq_quantize_mxfp4(s["x"], s["packed"], s["pscale"])
        mxq.mxq_mxfp4_to_mxfp8_col(s["x"], s["cdata"], s["cscale"])
        sets.append(s)
    del x0, g0
    torch.cuda.synchronize()

    names = ["proj", "row", "export", "block128", "dec_row", "dec_tile"]
    launches = {
        "proj": lambda s: mxq.mxq_fake_quantize_mxfp4(s["x"], s["y"]),
        "row": lambda s: mxq.mxq_mxfp4_to_mxfp8_row(s["x"], s["data"], s["scale"]),
        "export": lambda s: mxq.mxq_export_mxfp8(s["data"], s["scale"], K, s["scale_c"]),
        "block128": lambda s: mxq.mxq_mxfp4_to_fp8_block128(s["x"], s["bdata"], s["tc"]),
        "dec_row": lambda s: mxq.mxq_dequantize(s["data"], s["scale_c"], out=s["dec_r"]),
        "dec_tile": lambda s: mxq.mxq_dequantize(s["bdata"], s["tc"], layout=mxq.MXQ_SCALE_TILE_128X128,
                                                 out=s["dec_t"]),
    }
    # outside the step: projection + row lift fused into one pass (one read of x)
    launches["fused"] = lambda s: mxq.mxq_fake_quantize_mxfp4_with_mxfp8_row(s["x"], s["y2"], s["data2"], s["scale2"])
    # outside the step: the packed MXFP4 deployment format
    launches["quantize_mxfp4"] = lambda s: mxq.mxq_quantize_mxfp4(s["x"], s["packed"], s["pscale"])
    launches["dequantize_mxfp4"] = lambda s: mxq.mxq_dequantize_mxfp4(s["packed"], s["pscale"], K, out=s["dec_p"])
    launches["packed_to_row"] = lambda s: mxq.mxq_mxfp4_packed_to_mxfp8_row(s["packed"], s["pscale"], K, s["data2"],
                                                                              s["scale2"][:, :nb])
    launches["packed_to_block128"] = lambda s: mxq.mxq_mxfp4_packed_to_fp8_block128(s["packed"], s["pscale"], K,
                                                                                    s["data2"], s["tc2"])
    # outside the step: MXFP8 columnwise (32x1), alone and with the row lift in one pass, and its decode
    launches["col"] = lambda s: mxq.mxq_mxfp4_to_mxfp8_col(s["x"], s["cdata"], s["cscale"])
    launches["row_col"] = lambda s: mxq.mxq_mxfp4_to_mxfp8_row_col(s["x"], s["data2"], s["scale2"], s["cdata"],
                                                                     s["cscale"])
    launches["dec_col"] = lambda s: mxq.mxq_dequantize(s["cdata"], s["cscale"], layout=mxq.MXQ_SCALE_COL_32X1,
                                                       out=s["dec_c"])
    # outside the step: the row lift, the projection, the fold, the row-layout decode and the packed MXFP4
    # encode of 48 weights of 1024 x 2048, each in one grouped call
    # (prepared once per buffer set, as for weights re-converted every step)
    for s in sets:
        s["grouped"] = mxq.GroupedRowLift(s["gx"], s["gdata"], s["gscale"])
        s["grouped_proj"] = mxq.GroupedProjection(s["gx"], s["gy"])
        s["grouped_fold"] = mxq.GroupedBlock128(s["gx"], s["gbdata"], s["gtc"])
        s["grouped_dec"] = mxq.GroupedDequantize(s["gdata"], s["gscale"], outs=s["gdec"])
        s["grouped_q4"] = mxq.GroupedQuantizeMxfp4(s["gx"], s["gpk"], s["gps"])
        s["grouped"]()                                    # the payloads and codes the decode reads
    launches["row_grouped"] = lambda s: s["grouped"]()
    launches["proj_grouped"] = lambda s: s["grouped_proj"]()
    launches["block128_grouped"] = lambda s: s["grouped_fold"]()
    launches["dec_row_grouped"] = lambda s: s["grouped_dec"]()
    launches["quantize_mxfp4_grouped"] = lambda s: s["grouped_q4"]()
    extra_names = ["fused", "quantize_mxfp4", "dequantize_mxfp4", "packed_to_row", "packed_to_block128", "col",
                   "row_col", "dec_col", "row_grouped", "proj_grouped", "block128_grouped", "dec_row_grouped",
                   "quantize_mxfp4_grouped"]
    # outside the step: the access-shape reference kernels (libmxq_shapes.so), each moving its
    # kernel's bytes in that kernel's access pattern with no quantization arithmetic
    shapes_lib = ctypes.CDLL(mxq.build.library_path("libmxq_shapes.so"))
    shapes_lib.mxq_shape_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    shape_stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def shape_launch(code, src, dst, codes):
        def go(s):
            rc = shapes_lib.mxq_shape_run(code, es, s[src].data_ptr(), s[dst].data_ptr(), s[codes].data_ptr(), rows, K,
                                          shape_stream)
            if rc:
                raise RuntimeError(f"access shape {code} did not launch (status {rc})")
        return go

    for n, (code, src, codes) in SHAPES_OF.items():
        launches[n] = shape_launch(code, src, "y2", codes)
    shape_names = list(SHAPES_OF)
    # kernel -> buffer-set offset; consecutive launches of one kernel walk the six sets
    offset = {"proj": 0, "row": 2, "export": 2, "block128": 4, "dec_row": 3, "dec_tile": 5, "fused": 1,
              "quantize_mxfp4": 1, "dequantize_mxfp4": 3, "packed_to_row": 5, "packed_to_block128": 0, "col": 2,
              "row_col": 4, "dec_col": 1, "row_grouped": 0, "proj_grouped": 2, "block128_grouped": 4,
              "dec_row_grouped": 1, "quantize_mxfp4_grouped": 3}
    offset.update({n: i % NSETS for i, n in enumerate(SHAPES_OF)})

    # The timed region runs K whole passes kernel-major: each kernel is launched K
    # times back to back (rotating buffer sets) between two HIP events on the
    # launch stream, so an event pair brackets K launches and its average is the
    # kernel's own duration plus the small gap between dispatches.
    stream = torch.cuda.current_stream(dev)
    bursts = {}

    def run(i0: int, k: int, timed: bool, which=names, sub: int = 0, store=None):
        # timed: events around each kernel's burst; with sub > 0 also after
        # every `sub` launches (the spread statistics, outside the timed region)
        store = bursts if store is None else store
        for n in which:
            evs = []
            for j, i in enumerate(range(i0, i0 + k)):
                if timed and (j == 0 or (sub and j % sub == 0)):
                    evs.append(torch.cuda.Event(enable_timing=True))
                    evs[-1].record(stream)
                launches[n](sets[(i + offset[n]) % NSETS])
            if timed:
                evs.append(torch.cuda.Event(enable_timing=True))
                evs[-1].record(stream)
                store[n] = evs

    run(0, args.warmup, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.warmup, args.steps, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    run(0, args.warmup, False, extra_names + shape_names)
    run(args.warmup, args.steps, True, extra_names + shape_names)
    torch.cuda.synchronize()
    # spread of the per-launch time: SPREAD_BURSTS sub-bursts of SUB launches each
    spread = {}
    run(0, SUB * SPREAD_BURSTS, True, names + extra_names + shape_names, sub=SUB, store=spread)
    torch.cuda.synchronize()

    # For reference: the runtime's own device-to-device copy (hipMemcpyAsync) of
    # the weight into a buffer of the same size -- the projection's traffic --
    # over the same rotating buffer sets (the fused pass's output buffer, which
    # no check reads).
    for i in range(args.warmup):
        sets[i % NSETS]["y2"].copy_(sets[i % NSETS]["x"])
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for i in range(args.steps):
        sets[(i + 1) % NSETS]["y2"].copy_(sets[(i + 1) % NSETS]["x"])
    c1.record(stream)
    torch.cuda.synchronize()
    copy_us = 1e3 * c0.elapsed_time(c1) / args.steps

    orders = None
    if args.orders:
        # Each kernel's burst mean in three orders, outside the timed region: right
        # after a burst of the fold, after a 30 ms idle gap, after a burst of
        # itself (the median of ORDER_REPS repetitions).  A kernel whose speed
        # depends on the state the one before it leaves the GPU in shows it here.
        def burst(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(ORDER_LAUNCHES):
                launches[n](sets[(i + offset[n]) % NSETS])
            b.record(stream)
            return a, b

        res = {}
        for _ in range(ORDER_REPS):
            for n in names + extra_names:
                for pre in ("after_fold", "after_idle", "after_itself"):
                    torch.cuda.synchronize()
                    if pre == "after_idle":
                        time.sleep(0.03)
                    else:
                        burst("block128" if pre == "after_fold" else n)
                    a, b = burst(n)
                    torch.cuda.synchronize()
                    res.setdefault(n, {}).setdefault(pre, []).append(1e3 * a.elapsed_time(b) / ORDER_LAUNCHES)
        orders = {n: {pre: round(statistics.median(v), 2) for pre, v in d.items()} for n, d in res.items()}

    if args.calibrate:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    nbytes = algorithmic_bytes(rows, K, es)
    ms_per_step = wall * 1e3 / args.steps
    total = sum(nbytes.values())
    kernels = {}
    def burst_stats(n):
        """Mean per launch over the timed burst, and median / min of the
        spread pass's sub-burst means (us)."""
        a, b = bursts[n]
        mean = 1e3 * a.elapsed_time(b) / args.steps
        evs = spread[n]
        subs = [1e3 * evs[j].elapsed_time(evs[j + 1]) / SUB for j in range(len(evs) - 1)]
        return mean, statistics.median(subs), min(subs)

    for n in names:
        us, med, lo = burst_stats(n)
        gbs = nbytes[n] / (us * 1e-6) / 1e9
        kernels[n] = {"us": round(us, 2), "us_median": round(med, 2), "us_min": round(lo, 2), "bytes": nbytes[n],
                      "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                      # HBM bytes per launch from the committed counters (8192 x 8192 weights)
                      "traffic": read_traffic(n, args.weight) if headline else None}
    extra = {}
    extra_bytes = dict(packed_bytes(rows, K, es), fused=fused_bytes(rows, K, es), **col_bytes(rows, K, es),
                       row_grouped=gn * algorithmic_bytes(gr, gk, es)["row"],
                       proj_grouped=gn * algorithmic_bytes(gr, gk, es)["proj"],
                       block128_grouped=gn * algorithmic_bytes(gr, gk, es)["block128"],
                       dec_row_grouped=gn * algorithmic_bytes(gr, gk, es)["dec_row"],
                       quantize_mxfp4_grouped=gn * packed_bytes(gr, gk, es)["quantize_mxfp4"])
    for n in extra_names:
        us, med, lo = burst_stats(n)
        gbs = extra_bytes[n] / (us * 1e-6) / 1e9
        extra["fused_proj_row" if n == "fused" else n] = {"us": round(us, 2), "us_median": round(med, 2),
                                                          "us_min": round(lo, 2), "bytes": extra_bytes[n],
                                                          "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                                                          "traffic": read_traffic(n, args.weight) if headline else None}
    # the access shapes, each with its kernel's algorithmic bytes (the barrier-free and linear variants of
    # the fold's pattern with the fold's, the payload-only row shape without the codes)
    n_el, tiles = rows * K, ((rows + 127) // 128) * ((K + 127) // 128)
    shape_bytes = {"shape_copy16": nbytes["proj"], "shape_row": es * n_el + n_el, "shape_row_codes": nbytes["row"],
                   "shape_decode": nbytes["dec_row"], "shape_tile": nbytes["block128"],
                   "shape_tile_no_barrier": nbytes["block128"], "shape_linear_fold": es * n_el + n_el,
                   "shape_linear_fold_no_barrier": es * n_el + n_el,
                   "shape_packed_row": packed_bytes(rows, K, es)["packed_to_row"],
                   "shape_read": es * n_el, "shape_write": es * n_el, "shape_tile_loads": es * n_el,
                   "shape_linear_loads": es * n_el, "shape_tile_stores": n_el, "shape_linear_stores": n_el}
    shapes_out = {}
    for n in shape_names:
        us, med, lo = burst_stats(n)
        gbs = shape_bytes[n] / (us * 1e-6) / 1e9
        shapes_out[n[len("shape_"):]] = {"us": round(us, 2), "us_median": round(med, 2), "us_min": round(lo, 2),
                                         "bytes": shape_bytes[n], "GB/s": round(gbs, 1),
                                         "frac": round(gbs / HBM_PEAK_GBS, 4), "of_kernel": SHAPE_KERNEL.get(n)}
    for n, k in SHAPE_KERNEL.items():
        # the kernel's speed as a fraction of its access shape's (1.0: the pattern alone sets its time)
        entry = kernels[k] if k in kernels else extra[k]
        entry["of_shape"] = round(shapes_out[n[len("shape_"):]]["us"] / entry["us"], 4)
    extra["fused_proj_row"]["vs_separate_us"] = round(kernels["proj"]["us"] + kernels["row"]["us"], 2)
    extra["row_col"]["vs_separate_us"] = round(kernels["row"]["us"] + extra["col"]["us"], 2)
    dominant = max(names, key=lambda n: kernels[n]["us"])
    rl = {"kernel": dominant, "bound": "hbm", "achieved": kernels[dominant]["GB/s"], "peak": HBM_PEAK_GBS,
          "unit": "GB/s", "frac": kernels[dominant]["frac"],
          # the committed counter summaries are of the 8192 x 8192 weights
          "traffic": read_traffic(dominant, args.weight) if headline else None}
    out = {
        "metric": "GB/s and % HBM peak, MXFP4 proj + MXFP8-row/128x128 at " +
                  ("8192^2 " if headline else args.shape + " ") + args.weight,
        "value": round(total / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the weight's own type; every step is integer work on its bit patterns
        # (amax, exponent fields) plus the hardware E2M1 / E4M3 conversions
        "dtype": "fp32" if fp32 else "bf16",
        "data": "synthetic",
        "config": {"workload": (f"{rows}x{K} fp32 master weight (the bf16 weight before its cast)"
                                if fp32 else f"{rows}x{K} bf16 weight") +
                               f", N(0,0.02) seed {1 if headline else 3 if args.shape == '8192x28672' else 2}: "
                               f"proj + row (scale_ld {scale_ld}) + export + block128 + decode(row) "
                               "+ decode(tile), decodes to the weight's dtype",
                   "bytes_per_step": total, "buffer_sets": NSETS},
        "roofline": rl,
        "kernels": kernels,
        "outside_step": extra,
        "access_shapes": shapes_out,
        "copy_reference": {"what": "hipMemcpyAsync device to device of the weight (torch copy_)",
                           "us": round(copy_us, 2), "bytes": 2 * es * rows * K,
                           "GB/s": round(2 * es * rows * K / (copy_us * 1e-6) / 1e9, 1),
                           "frac": round(2 * es * rows * K / (copy_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if orders is not None:
        out["orders"] = orders
    if not args.no_cpu:
        # every CPU this process may run on (its affinity set), one oracle thread each
        out["cpu_baseline"], want = cpu_baseline(bits, threads=host_cpu()["usable"])
        # the same oracle run gives the bytes for a full-size parity check of the step
        out["parity"] = parity(sets[0], want)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
