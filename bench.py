"""Benchmark of the bf16 GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-configs]

A step is one tbg_gemm call on the 8192³ workload (bf16 A row-major, B row-major K×N, fp32
accumulation, bf16 out): host-side descriptor encoding, the tiled copies into LDS, the MFMA
main loop and the masked epilogue, with operands already resident in HBM.  A region is W
untimed steps, a synchronisation, then K steps between two HIP events on the launch stream and a
device synchronisation.  The same region first runs untimed, back to back, for --settle seconds
(reported as roofline.settle: after any idle time the device's power controller needs ~40
launches of this product before the clock settles); the region timed is the next one.  One
JSON line is printed.

Also reported in the same line:
  roofline      the GEMM kernel against the bf16 dense MFMA peak: algorithmic flops per launch
                (2MNK) over the average launch time from HIP events on the launch stream
                (launch_ms: min / median / max per launch, from a further region whose launches
                each have their own pair of events; gemm_clock_ghz: the shader clock the
                same kernel reports from inside, per workgroup, right after the timed steps);
                `traffic` is the HBM bytes per launch from the committed rocprofv3 counter
                summary when it was taken on the current kernel source, else null.
  cpu_baseline  the CPU oracle on a bounded sample of the same product (the first rows of C),
                timed on this host's cores.
  per_config    TFLOP/s and % of peak on all five GEMM workloads (for the small c1-c3 also the
                GPU time per product from HIP-graph replays, `graph_ms`), the 8192³ product with fp16 and
                with fp8 E4M3 inputs (against the fp8 peak, with the fp8 products-alone ceiling
                measured the same way as the bf16 one), the benchmark convolution layer
                (timed the same way, fewer steps), and the tiled-copy kernel (tbg_tiled_copy_many)
                on the three copy workloads: the worked 128x64 box at its 10 places, the 432 boxes of
                the 5-D tensor with NaN fill, and all 8192 boxes of the 8192x8192 operand A, each
                in achieved GB/s (in-bounds source bytes + image bytes per launch) against the
                8 TB/s HBM peak.
  roofline.ceiling  the bf16 products alone (no loads, no stores) on random register-resident
                operands, timed in the same run: what the power limit lets the matrix units
                sustain; frac_of_ceiling is the GEMM kernel's rate over it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz ("2.5 PF")
PEAK_TFLOPS = {"bf16": PEAK_BF16_TFLOPS, "f16": PEAK_BF16_TFLOPS,
               "f8e4m3": 5033.2, "f8e5m2": 5033.2}  # dense fp8: 256 CU x 8192 flop/clk x 2.4 GHz ("5.0 PF")
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E: 8 TB/s
METRIC = "bf16 GEMM TFLOP/s and % of MI355X MFMA peak at M=N=K=8192, 1 GPU"
KERNEL_SOURCES = ["tiled_bf16_gemm_amd/csrc/gemm_common.hpp", "tiled_bf16_gemm_amd/csrc/gemm_ring.hpp",
                  "tiled_bf16_gemm_amd/csrc/tile_loader.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_8192_traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch from the committed counter summary, if it matches this kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def gemm_operands(torch, w, ab="bf16"):
    """Device operands of a GEMM workload: (A view, B view, B layout, C, workspace).  ab: the input
    type; the workload's bf16 values are converted to it (8-bit inputs take B stored N×K,
    transposed once here, outside any timed region)."""
    import workloads
    A, B = workloads.gemm_inputs(w)
    A = A.cuda()
    B = B.cuda()
    Av = A[:, :w.K]
    Bv = B[:, :w.N] if w.b_layout == "kn" else B[:, :w.K]
    b_layout = w.b_layout
    if ab != "bf16":
        tdt = {"f16": torch.float16, "f8e4m3": torch.float8_e4m3fn, "f8e5m2": torch.float8_e5m2}[ab]
        Av = Av.to(tdt)
        if ab.startswith("f8") and b_layout == "kn":
            Bv, b_layout = Bv.t().contiguous(), "nk"
        Bv = Bv.to(tdt)
    C = torch.empty((w.M, w.N), dtype=torch.float32 if w.out_dtype == "f32" else torch.bfloat16, device="cuda")
    return Av, Bv, b_layout, C, gemm_workspace(torch, w, ab, Av, Bv, b_layout)


def gemm_workspace(torch, w, ab, Av, Bv, b_layout):
    """The product's workspace: twice the library's exact need, so that successive calls repack
    into alternate halves (include/tbg.h, tbg_gemm)."""
    import tiled_bf16_gemm_amd as tbg
    need = tbg.gemm_workspace_query(w.M, w.N, w.K, ab, Av.data_ptr(), Av.stride(0), Bv.data_ptr(), Bv.stride(0),
                                    b_layout)
    return torch.empty(max(2 * need, 256), dtype=torch.uint8, device="cuda")


COLD_CALLS = 20


def time_gemm_cold(torch, torch_ops, w, operands, calls: int = COLD_CALLS, flush_mib: int = 512) -> float:
    """Median ms of `calls` products each started on cold caches: before each one, a 512 MiB device
    buffer is overwritten (more than the 256 MB Infinity Cache and every XCD's L2 together), and
    the HIP events on the launch stream bracket the product only."""
    import statistics
    Av, Bv, b_layout, C, ws = operands
    flush = torch.empty(flush_mib << 20, dtype=torch.uint8, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for a, b in ev:
        flush.fill_(1)
        a.record()
        torch_ops.gemm(Av, Bv, b_layout, w.out_dtype, out=C, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    del flush
    return statistics.median(a.elapsed_time(b) for a, b in ev)


def launch_stats(per):
    """min / median / max of per-launch times (ms)."""
    import statistics
    return {"min": round(min(per), 5), "median": round(statistics.median(per), 5), "max": round(max(per), 5)}


def time_gemm_detail(torch, torch_ops, w, steps, warmup, config=None, ab="bf16", settle_s=0.0, operands=None):
    """The timed region: `warmup` untimed calls, a synchronisation, then `steps` calls between two
    HIP events on the launch stream, and a synchronisation (no event between the calls: each event
    recorded with timing costs the GPU a few microseconds, 7 µs per call measured on a 45 µs
    product).  With settle_s > 0 the same region is first run back to back, untimed, until
    settle_s seconds have passed, and the region timed is the next one.  Then one more region, of
    the same calls each bracketed by its own pair of events, gives the per-launch spread.
    Returns a dict: ms_step and ms_kernel (timed region / steps: the average launch time, the
    launches back to back), per (per-launch ms of the spread region), wall_ms (host wall time
    per step of the timed region) and settle (the number of settle regions, their seconds, and
    the time per step of the first and of each of the last five)."""
    Av, Bv, b_layout, C, ws = operands if operands is not None else gemm_operands(torch, w, ab)

    def call():
        torch_ops.gemm(Av, Bv, b_layout, w.out_dtype, out=C, workspace=ws, config=config)

    def region():
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
        return e0.elapsed_time(e1) / steps, wall / steps

    def spread():
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    settle = None
    if settle_s > 0:
        per_step = []
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < settle_s:
            per_step.append(region()[0])
        settle = {"regions": len(per_step), "seconds": round(time.perf_counter() - t0, 3),
                  "first_region_ms": round(per_step[0], 5), "last_regions_ms": [round(x, 5) for x in per_step[-5:]]}
    ms_step, wall_ms = region()
    return {"ms_step": ms_step, "ms_kernel": ms_step, "per": spread(), "wall_ms": wall_ms, "settle": settle}


def time_gemm(torch, torch_ops, w, steps, warmup, config=None, ab="bf16", settle_s=0.0):
    """Returns (ms per step over the whole timed region, the same as the average launch time, wall
    ms per step)."""
    r = time_gemm_detail(torch, torch_ops, w, steps, warmup, config=config, ab=ab, settle_s=settle_s)
    return r["ms_step"], r["ms_kernel"], r["wall_ms"]


_DIAG = None


def diag_lib():
    """The measurement library (products alone, the clock-recording GEMM), loaded once.  Load it
    before any timed region: loading a code object leaves the device idle for a moment, and
    after any idle time the first ~40 launches of the 8192^3 product run slow while the power
    controller settles."""
    global _DIAG
    if _DIAG is None:
        import ctypes
        path = os.path.join(ROOT, "tiled_bf16_gemm_amd", "diag", "libtbg_diag.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run __graft_entry__.build()")
        _DIAG = ctypes.CDLL(path)
    return _DIAG


def gemm_clock(torch, Av, Bv, C, launches: int = 40):
    """The shader clock the GEMM kernel itself runs at: the library's 8192^3 kernel built with
    clock recording (tiled_bf16_gemm_amd/diag/mfma_rate.hip, tbg_diag_gemm_clock) launched
    `launches` times back to back on the same operands; each workgroup of the last launch reports
    its shader-clock and 100 MHz real-time counter advance.  Returns min / median / max over the
    workgroups in GHz and the mean launch time in ms."""
    import ctypes
    import statistics
    lib = diag_lib()
    lib.tbg_diag_gemm_clock.restype = ctypes.c_int
    lib.tbg_diag_gemm_clock.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong,
                                        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int), ctypes.c_void_p]
    M, K = Av.shape
    N = Bv.shape[1]
    nwg = ((M + 255) // 256) * ((N + 255) // 256)
    clk = torch.zeros(2 * nwg, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    n_out = ctypes.c_int(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        rc = lib.tbg_diag_gemm_clock(Av.data_ptr(), Bv.data_ptr(), C.data_ptr(), M, N, K, Av.stride(0), Bv.stride(0),
                                     C.stride(0), clk.data_ptr(), ctypes.byref(n_out), stream)
        if rc != 0:
            raise RuntimeError(f"clock-recording GEMM launch failed ({rc})")
    e1.record()
    torch.cuda.synchronize()
    c = clk.cpu().tolist()
    ghz = [c[2 * i + 1] / (c[2 * i] / 100e6) / 1e9 for i in range(nwg) if c[2 * i] > 0]
    return {"min": round(min(ghz), 3), "median": round(statistics.median(ghz), 3), "max": round(max(ghz), 3),
            "workgroups": len(ghz), "launch_ms": round(e0.elapsed_time(e1) / launches, 5)}


def time_gemm_graph(torch, torch_ops, w, calls=20, replays=20, config=None):
    """GPU time per product with the host out of the way: `calls` products captured in one HIP
    graph (torch.cuda.graph), replayed `replays` times; returns ms per product."""
    import workloads
    A, B = workloads.gemm_inputs(w)
    A, B = A.cuda(), B.cuda()
    Av = A[:, :w.K]
    Bv = B[:, :w.N] if w.b_layout == "kn" else B[:, :w.K]
    C = torch.empty((w.M, w.N), dtype=torch.float32 if w.out_dtype == "f32" else torch.bfloat16, device="cuda")
    ws = gemm_workspace(torch, w, "bf16", Av, Bv, w.b_layout)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for _ in range(3):
            torch_ops.gemm(Av, Bv, w.b_layout, w.out_dtype, out=C, workspace=ws, config=config)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(calls):
            torch_ops.gemm(Av, Bv, w.b_layout, w.out_dtype, out=C, workspace=ws, config=config)
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / (replays * calls)
    del g, A, B, C, ws
    return ms


def copy_inbounds_bytes(w) -> int:
    """Source bytes a copy workload's boxes read: elements inside the tensor, per box (the image
    bytes are box_bytes each, fill included)."""
    esize = 2
    total = 0
    for c in w.coords:
        n = 1
        for x, b, e, d in zip(c, w.box, w.estr, w.dims):
            n *= sum(1 for j in range((b + e - 1) // e) if 0 <= x + j * e < d)
        total += n * esize
    return total


def time_copy_graph(torch, torch_ops, w, calls=20, replays=20):
    """GPU time per tbg_tiled_copy_many launch from HIP-graph replays (as time_gemm_graph)."""
    import workloads
    import tiled_bf16_gemm_amd as tbg
    src = workloads.copy_source(w).cuda()
    d = list(w.dims)
    strides, acc = [], 2
    for i in range(len(d) - 1):
        acc *= d[i]
        strides.append(acc)
    desc = torch_ops.encode(src, w.dtype, d, strides, list(w.box), list(w.estr), w.swizzle, w.oob)
    coords = torch.tensor([list(c) for c in w.coords], dtype=torch.int32, device="cuda").contiguous()
    out = torch.empty(len(w.coords) * tbg.box_bytes(desc), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for _ in range(3):
            torch_ops.tiled_copy_many(desc, coords, out=out, stream=stream)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(calls):
            torch_ops.tiled_copy_many(desc, coords, out=out, stream=stream)
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / (replays * calls)
    del g
    return ms


def time_copy(torch, torch_ops, w, steps, warmup):
    """tbg_tiled_copy_many over every box of a copy workload, one launch per step, `steps` launches
    between two HIP events; returns (ms per launch, algorithmic bytes per launch = in-bounds source
    bytes + images)."""
    import workloads
    import tiled_bf16_gemm_amd as tbg
    src = workloads.copy_source(w).cuda()
    d = list(w.dims)
    strides, acc = [], 2
    for i in range(len(d) - 1):
        acc *= d[i]
        strides.append(acc)
    desc = torch_ops.encode(src, w.dtype, d, strides, list(w.box), list(w.estr), w.swizzle, w.oob)
    coords = torch.tensor([list(c) for c in w.coords], dtype=torch.int32, device="cuda").contiguous()
    out = torch.empty(len(w.coords) * tbg.box_bytes(desc), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        torch_ops.tiled_copy_many(desc, coords, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        torch_ops.tiled_copy_many(desc, coords, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return ms, copy_inbounds_bytes(w) + len(w.coords) * tbg.box_bytes(desc)


def mfma_ceiling(torch, kind: int = 0, launches: int = 60, warmup: int = 60):
    """The matrix products alone (tiled_bf16_gemm_amd/diag/mfma_rate.hip): kind 0 bf16 16x16x32
    products on uniform[-1,1] bf16 operands, kind 1 fp8 16x16x128 products on the same values as
    E4M3, back to back on register-resident fragments, one workgroup of four waves per CU as the
    256x256 GEMM tile, four rounds of workgroups like the 8192^3 product.  Returns (TFLOP/s, median
    shader clock in GHz from the kernel's own counters): the ceiling of any GEMM kernel at the clock
    the power limit allows with such operands."""
    import ctypes
    import statistics
    lib = diag_lib()
    lib.tbg_diag_mfma_rate.restype = ctypes.c_int
    lib.tbg_diag_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p]
    nwg = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    iters = 200
    g = torch.Generator().manual_seed(77)
    if kind == 0:
        src = (torch.rand(nwg * 16 * 256 * 8, generator=g) * 2 - 1).to(torch.bfloat16).cuda()
    else:
        src = (torch.rand(nwg * 16 * 256 * 16, generator=g) * 2 - 1).to(torch.float8_e4m3fn).view(torch.uint8).cuda()
    out = torch.empty(nwg * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2 * nwg, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def go():
        rc = lib.tbg_diag_mfma_rate(kind, src.data_ptr(), out.data_ptr(), nwg, iters, clk.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"mfma rate launch failed ({rc})")
    for _ in range(warmup):
        go()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        go()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    # a 16x16x32 product is 8192 multiply-adds (16384 flops), a 16x16x128 one four times that
    flops = nwg * 4 * iters * 64 * (16384 if kind == 0 else 65536)
    c = clk.cpu().tolist()
    ghz = statistics.median(c[2 * i + 1] / (c[2 * i] / 100e6) / 1e9 for i in range(nwg) if c[2 * i] > 0)
    return flops / (ms * 1e-3) / 1e12, ghz


def time_conv(torch, torch_ops, w, steps, warmup, config=None):
    """tbg_conv2d_fwd on a convolution workload: `steps` calls between two HIP events after
    `warmup` untimed ones; returns (ms per call, the same as the average launch time)."""
    import workloads
    x, f = workloads.conv_inputs(w)
    x, f = x.cuda(), f.cuda()
    y = torch.empty((w.M, w.k), dtype=torch.float32 if w.out_dtype == "f32" else torch.bfloat16, device="cuda")
    for _ in range(warmup):
        torch_ops.conv2d(x, f, w.pad, w.stride, w.dil, w.out_dtype, out=y, config=config)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        torch_ops.conv2d(x, f, w.pad, w.stride, w.dil, w.out_dtype, out=y, config=config)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del x, f, y
    return ms, ms


def cpu_baseline(w, target_s: float = 15.0):
    """The oracle on the first rows of the product; grows the sample until it takes ~target_s."""
    import oracle
    import workloads
    orc = oracle.get()
    A, B = workloads.gemm_inputs(w)
    Ab, Bb = workloads.bits(A), workloads.bits(B)
    lda, ldb, _ = w.lds()
    threads = orc.max_threads()
    rows = max(8, threads)  # one row per thread at least, so the trial keeps every thread busy
    t0 = time.perf_counter()
    orc.gemm(Ab, Bb, w.M, w.N, w.K, lda, ldb, w.b_layout, rows=(0, rows), threads=threads)
    dt = time.perf_counter() - t0
    rows2 = max(rows, min(w.M, int(rows * target_s / max(dt, 1e-3))))
    rows2 = max(threads, (rows2 // threads) * threads)
    t0 = time.perf_counter()
    orc.gemm(Ab, Bb, w.M, w.N, w.K, lda, ldb, w.b_layout, rows=(0, rows2), threads=threads)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows2 * w.N * w.K
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows 0..{rows2 - 1} of the {w.M}x{w.N}x{w.K} product ({rows2}x{w.N}x{w.K} MACs, "
                  f"binary64 accumulation), {dt:.1f} s on {threads} host threads",
        "seconds": round(dt, 2),
        "cpu_model": _cpu_model(),
    }


def _cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "" where it cannot be read."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


# The library's kernels for the two large workloads (bf16 in, bf16 out, 256×256 ring, 2 stages):
# B stored K×N (8192³) and B stored N×K (16384×14336×4096).
C4_KERNEL = "gemm_ring_kernel<256, 256, 2, 0, 0, 1, 0, 0>"
C5_KERNEL = "gemm_ring_kernel<256, 256, 2, 0, 1, 1, 0, 0>"


def counters_driver(torch, torch_ops, w):
    """Fixed launches for counter collection: the 8192³ GEMM, the same with E4M3 inputs, the
    16384×14336×4096 GEMM, then a copy of known size (the calibration kernel)."""
    import workloads
    A, B = workloads.gemm_inputs(w)
    A = A.cuda()
    B = B.cuda()
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    for _ in range(5):
        torch_ops.gemm(A, B, w.b_layout, w.out_dtype, out=C)
    torch.cuda.synchronize()
    # the same product with E4M3 inputs (B stored N×K), for the fp8 kernel's counters
    A8 = A.to(torch.float8_e4m3fn)
    B8 = B.t().contiguous().to(torch.float8_e4m3fn)
    for _ in range(5):
        torch_ops.gemm(A8, B8, "nk", w.out_dtype, out=C)
    torch.cuda.synchronize()
    del A8, B8, A, B, C
    w5 = workloads.GEMMS["c5"]
    A, B = workloads.gemm_inputs(w5)
    A, B = A.cuda(), B.cuda()
    C = torch.empty((w5.M, w5.N), dtype=torch.bfloat16, device="cuda")
    for _ in range(5):
        torch_ops.gemm(A, B, w5.b_layout, w5.out_dtype, out=C)
    torch.cuda.synchronize()
    del A, B, C
    src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("counters driver: 5 gemm launches (8192^3 bf16), 5 with E4M3 inputs, 5 of 16384x14336x4096, "
          "5 copies of 536870912 bytes", flush=True)


def summarize_profiles(trace_db: str, fetch_db: str, write_db: str, out_dir: str, commands: dict,
                       sq_db: str = "") -> dict:
    """Write the short text summaries of rocprofv3 runs into profiles/ (and the traffic figure
    bench.py reports).  Reads rocprofv3's SQLite output with the standard library only.
    commands["bench_line"] (optional): the JSON line the traced bench run printed; its timed
    steps are the last `steps` dispatches of the 8192³ kernel in the trace."""
    import sqlite3
    import statistics

    def rows(db, q):
        c = sqlite3.connect(db)
        try:
            return list(c.execute(q))
        finally:
            c.close()

    line = commands.get("bench_line")
    top = rows(trace_db, "select name, total_calls, total_duration, average, percentage from top_kernels")
    lines = ["# GEMM kernel trace, 8192³ workload (bf16 in, fp32 accumulate, bf16 out) and the rest of the bench run",
             "", "Command (<repo> is the repository root, <out> the output folder):", "", "```", commands["trace"], "```",
             "", "Summary written by `python bench.py --summarize <out>`.", "",
             "rocprofv3 kernel statistics (durations in microseconds):", "",
             "| kernel | calls | total us | average us | % |", "|---|---|---|---|---|"]
    for name, calls, total, avg, pct in top:
        short = name if len(name) <= 110 else name[:107] + "..."
        lines.append(f"| `{short}` | {calls} | {total:.1f} | {avg:.3f} | {pct:.1f} |")
    gemm_avg = [avg for name, _, _, avg, _ in top if C4_KERNEL in name]
    try:
        disp = [d / 1e3 for n, d in rows(trace_db, "select name, duration from kernels order by start") if C4_KERNEL in n]
    except sqlite3.Error:
        disp = []
    timed_avg = None
    if line and disp:
        steps = int(line.get("steps", 20))
        # after the timed steps the same kernel runs the per-launch spread region (its own
        # warm-up and steps) and the cold-cache calls (per_config c4)
        cold = int(line.get("per_config", {}).get("c4", {}).get("cold_calls", 0))
        spread = int(line["roofline"].get("spread_calls", 0))
        after = cold + spread
        timed = disp[len(disp) - after - steps:len(disp) - after]
        timed_avg = statistics.mean(timed)
        k_ms = line["roofline"]["kernel_ms"]
        flops = line["roofline"]["flops_per_launch"]
        order = (f"its {steps} timed steps, {spread} calls of the per-launch spread region and {cold} calls on cold "
                 f"caches, in that order; the {steps} before the last {after} are the timed steps" if after else
                 f"its {steps} timed steps, in that order; the last {steps} are the timed steps")
        lines += ["", f"The 8192³ kernel's {len(disp)} dispatches are the bench's settle regions, its warm-up, {order}.",
                  "", "| dispatches | average us | median us | TFLOP/s at the average | frac of 2516.6 |",
                  "|---|---|---|---|---|",
                  f"| all {len(disp)} | {statistics.mean(disp):.2f} | {statistics.median(disp):.2f} | "
                  f"{flops / (statistics.mean(disp) * 1e-6) / 1e12:.1f} | "
                  f"{flops / (statistics.mean(disp) * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.4f} |",
                  f"| timed {steps} | {timed_avg:.2f} | {statistics.median(timed):.2f} | "
                  f"{flops / (timed_avg * 1e-6) / 1e12:.1f} | {flops / (timed_avg * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.4f} |",
                  "", f"The same run's bench line (HIP events on the launch stream): kernel_ms {k_ms} "
                      f"({k_ms * 1e3:.2f} us), roofline.achieved {line['roofline']['achieved']} TFLOP/s, frac "
                      f"{line['roofline']['frac']}; value {line['value']} TFLOP/s."]
    elif commands.get("bench_kernel_us") is not None:
        lines += ["", f"bench.py's HIP-event average for the same kernel: {commands['bench_kernel_us']} us."]
    with open(os.path.join(out_dir, "gemm_8192_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    def per_kernel(db, counter):
        vals = {}
        for name, value in rows(db, f"select kernel_name, value from counters_collection where counter_name = '{counter}'"):
            vals.setdefault(name, []).append(value)
        return vals

    fetch = per_kernel(fetch_db, "FETCH_SIZE")
    write = per_kernel(write_db, "WRITE_SIZE")
    copy_bytes = 512 << 20
    calib_f = [v for k, v in fetch.items() if "copyBuffer" in k][0]
    calib_w = [v for k, v in write.items() if "copyBuffer" in k][0]
    sf = copy_bytes / (statistics.median(calib_f) * 1024)
    sw = copy_bytes / (statistics.median(calib_w) * 1024)
    avg_us = timed_avg if timed_avg is not None else (gemm_avg[0] if gemm_avg else None)
    table, figures = [], {}
    for label, kname, (M, N, K) in (("8192³", C4_KERNEL, (8192, 8192, 8192)),
                                    ("16384×14336×4096", C5_KERNEL, (16384, 14336, 4096))):
        gf = [v for k, v in fetch.items() if kname in k]
        gw = [v for k, v in write.items() if kname in k]
        if not gf or not gw:
            continue
        fb = statistics.median(gf[0]) * 1024 * sf
        wb = statistics.median(gw[0]) * 1024 * sw
        algo = (M * K + K * N + M * N) * 2
        figures[label] = (fb, wb, algo)
        table += [f"| {label} | FETCH_SIZE | {statistics.median(gf[0]):.1f} | {len(gf[0])} | {sf:.4f} | {fb:.4g} |",
                  f"| {label} | WRITE_SIZE | {statistics.median(gw[0]):.1f} | {len(gw[0])} | {sw:.4f} | {wb:.4g} |"]
    fb, wb, algo = figures["8192³"]
    total = fb + wb
    lines = ["# HBM traffic of the GEMM kernel, 8192³ and 16384×14336×4096 workloads", "",
             "Commands (one counter per run; <repo> is the repository root, <out> the output folder):", "", "```",
             commands["fetch"], commands["write"], "```", "",
             "Summary written by `python bench.py --summarize <out>`.", "",
             "Calibration: the same runs end with five device copies of 536870912 bytes (`__amd_rocclr_copyBuffer`)",
             "that read and write exactly that many bytes; each counter is scaled by bytes/counter of that copy.", "",
             "| kernel | counter | median KiB per dispatch | dispatches | scale | bytes per dispatch |",
             "|---|---|---|---|---|---|",
             f"| calibration copy | FETCH_SIZE | {statistics.median(calib_f):.1f} | {len(calib_f)} | {sf:.4f} | {copy_bytes} |",
             f"| calibration copy | WRITE_SIZE | {statistics.median(calib_w):.1f} | {len(calib_w)} | {sw:.4f} | {copy_bytes} |",
             *table, ""]
    for label, (f_, w_, a_) in figures.items():
        lines.append(f"HBM bytes per {label} launch: {f_ + w_:.4g} (algorithmic minimum A + B + C once: {a_:.4g}; "
                     f"ratio {(f_ + w_) / a_:.2f}).")
    if avg_us:
        lines.append(f"Over the 8192³ kernel's timed launches ({avg_us:.1f} us on average): "
                     f"{total / (avg_us * 1e-6) / 1e9:.0f} GB/s of these bytes, "
                     f"{100 * total / (avg_us * 1e-6) / 1e9 / PEAK_HBM_GBS:.1f} % of the 8 TB/s HBM peak; the "
                     f"algorithmic bytes alone: {algo / (avg_us * 1e-6) / 1e9:.0f} GB/s.")
    lines.append(f"Kernel source hash of the tree summarized (the counter runs are taken on that same tree): "
                 f"{kernel_source_hash()}")
    with open(os.path.join(out_dir, "gemm_8192_hbm_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    traffic = {"kernel_source_hash": kernel_source_hash(), "hbm_bytes_per_launch": round(total),
               "fetch_bytes": round(fb), "write_bytes": round(wb), "fetch_scale": sf, "write_scale": sw,
               "algorithmic_bytes": algo, "gemm_trace_avg_us": avg_us}
    if "16384×14336×4096" in figures:
        f5, w5, a5 = figures["16384×14336×4096"]
        traffic["c5"] = {"hbm_bytes_per_launch": round(f5 + w5), "fetch_bytes": round(f5), "write_bytes": round(w5),
                         "algorithmic_bytes": a5}
    with open(os.path.join(out_dir, "gemm_8192_traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    if sq_db and os.path.exists(sq_db):
        summarize_sq(sq_db, out_dir, commands["sq"])
    copy_db = os.path.join(os.path.dirname(os.path.dirname(trace_db)), "copytrace", "run_results.db")
    if os.path.exists(copy_db):
        summarize_copies(copy_db, out_dir, commands["copytrace"])
    return traffic


def summarize_copies(db: str, out_dir: str, command: str) -> None:
    """Kernel-trace summary of the tiled-copy kernel on the three copy workloads (one rocprofv3
    --kernel-trace run of `bench.py --only-copies`); launches are told apart by their grid size
    (one workgroup per box)."""
    import sqlite3
    import statistics
    import workloads
    c = sqlite3.connect(db)
    try:
        rows = list(c.execute("select name, grid_x, workgroup_x, duration from kernels"))
    finally:
        c.close()
    by_boxes = {}
    for name, gx, wx, dur in rows:
        if "tiled_copy_kernel" in name:
            by_boxes.setdefault(gx // wx, []).append(dur / 1e3)
    lines = ["# Tiled-copy kernel trace on the three copy workloads", "",
             "Command (<repo> is the repository root, <out> the output folder):", "", "```", command, "```", "",
             "Summary written by `python bench.py --summarize <out>`.  Algorithmic bytes per launch = source",
             "bytes inside the tensor + image bytes (fill included); GB/s from the trace's average duration,",
             "against the 8 TB/s HBM peak.", "",
             "| workload | boxes per launch | launches | average us | median us | algorithmic bytes | GB/s | of 8 TB/s |",
             "|---|---|---|---|---|---|---|---|"]
    for name in ("c1_copy", "c3_copy", "c4_a_boxes"):
        w = workloads.COPIES[name]
        d = by_boxes.get(len(w.coords), [])
        if not d:
            continue
        import math
        nbytes = copy_inbounds_bytes(w) + len(w.coords) * 2 * math.prod((b + e - 1) // e for b, e in zip(w.box, w.estr))
        avg = statistics.mean(d)
        gbs = nbytes / (avg * 1e-6) / 1e9
        lines.append(f"| {name} | {len(w.coords)} | {len(d)} | {avg:.2f} | {statistics.median(d):.2f} | {nbytes} | "
                     f"{gbs:.0f} | {100 * gbs / PEAK_HBM_GBS:.1f} % |")
    with open(os.path.join(out_dir, "copy_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
               "SQ_INSTS_MFMA", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "GRBM_GUI_ACTIVE"]


def summarize_sq(db: str, out_dir: str, command: str) -> None:
    """MFMA utilisation and LDS bank conflicts of the GEMM kernels from one rocprofv3 --pmc run.

    SQ_VALU_MFMA_BUSY_CYCLES counts busy cycles of every SIMD's matrix unit, SQ_BUSY_CU_CYCLES
    busy cycles of every CU (4 SIMDs each): their ratio / 4 is the fraction of the kernel's
    cycles the matrix units worked, at whatever clock the chip ran.  SQ_LDS_BANK_CONFLICT and
    SQ_LDS_IDX_ACTIVE are cycles, summed over CUs, so they divide by SQ_BUSY_CU_CYCLES.
    SQ_WAIT_ANY and SQ_WAVE_CYCLES are per wave (same units), their ratio the waiting share."""
    import sqlite3
    import statistics
    c = sqlite3.connect(db)
    try:
        rows = list(c.execute("select kernel_name, dispatch_id, counter_name, value, duration from counters_collection"))
    finally:
        c.close()
    per = {}
    for name, disp, cn, v, dur in rows:
        if "gemm_" not in name:
            continue
        d = per.setdefault(name, {}).setdefault(disp, {})
        d[cn] = v
        d["duration_ns"] = dur
    lines = ["# MFMA utilisation and LDS bank conflicts of the GEMM kernels, 8192³ (bf16 and E4M3) and 16384×14336×4096", "",
             "Command (<repo> is the repository root, <out> the output folder):", "", "```", command, "```", "",
             "Summary written by `python bench.py --summarize <out>`.  Medians over the dispatches.", "",
             "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 × SQ_BUSY_CU_CYCLES): the share of CU-busy cycles the",
             "  matrix units worked, at the clock the chip actually ran (the % of the 2.4 GHz peak is lower",
             "  by the clock ratio);",
             "- bank conflict = SQ_LDS_BANK_CONFLICT / SQ_BUSY_CU_CYCLES; LDS active = SQ_LDS_IDX_ACTIVE / the same;",
             "- waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES (waves at s_waitcnt or s_barrier);",
             "- MFMA instructions: SQ_INSTS_MFMA per dispatch (2MNK / flops per instruction: 16x16x32 bf16",
             "  16384, 16x16x128 fp8 65536);",
             "- clock = GRBM_GUI_ACTIVE / 8 / dispatch duration: the counter sums the active cycles of the 8 XCDs",
             "  (this division reproduces the clock the kernels measure themselves with s_memtime, and gives",
             "  ≈2.45 GHz for the memory-bound device copies of the same run); listed per dispatch in order,",
             "  the dispatches running back to back.", "",
             "| kernel | dispatches | MFMA busy | bank conflict | LDS active | waiting | MFMA instructions | clock per dispatch (GHz) |",
             "|---|---|---|---|---|---|---|---|"]
    for name, disps in per.items():
        def med(f):
            vals = [f(d) for d in disps.values() if all(k in d for k in SQ_COUNTERS[:7])]
            return statistics.median(vals) if vals else float("nan")
        mf = med(lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * d["SQ_BUSY_CU_CYCLES"]))
        bc = med(lambda d: d["SQ_LDS_BANK_CONFLICT"] / d["SQ_BUSY_CU_CYCLES"])
        la = med(lambda d: d["SQ_LDS_IDX_ACTIVE"] / d["SQ_BUSY_CU_CYCLES"])
        wt = med(lambda d: d["SQ_WAIT_ANY"] / d["SQ_WAVE_CYCLES"])
        ni = med(lambda d: d["SQ_INSTS_MFMA"])
        clocks = ", ".join(f"{d['GRBM_GUI_ACTIVE'] / 8 / d['duration_ns']:.2f}" for _, d in sorted(disps.items())
                           if "GRBM_GUI_ACTIVE" in d and d.get("duration_ns"))
        lines.append(f"| `{name}` | {len(disps)} | {100 * mf:.1f} % | {100 * bc:.1f} % | {100 * la:.1f} % | "
                     f"{100 * wt:.1f} % | {ni:.4g} | {clocks} |")
    with open(os.path.join(out_dir, "gemm_8192_mfma_lds_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


# Every built (pipeline, tile, stages) configuration, as include/tbg.h lists them.
SWEEP_CONFIGS = ([("ring", "256x256", 2)] + [("ring", t, st) for t in ("256x128", "128x256") for st in (2, 3)]
                 + [("ring", "128x128", st) for st in (2, 3, 4, 5)] + [("ring", "64x64", st) for st in range(2, 7)]
                 + [("producer", t, st) for t in ("256x128", "128x256") for st in (2, 3)]
                 + [("producer", "128x128", st) for st in (2, 3, 4)]
                 + [("producer", "64x64", st) for st in range(2, 7)])

# The fp16 and 8-bit configurations built (include/tbg.h, tbg_gemm_typed).
SWEEP_CONFIGS_F16 = ([("ring", t, 2) for t in ("256x256", "256x128", "128x256", "128x128", "64x64")] + [("ring", "64x64", 3)]
                     + [("producer", t, 2) for t in ("256x128", "128x256")]
                     + [("producer", t, 3) for t in ("128x128", "64x64")])
SWEEP_CONFIGS_F8 = [("ring", t, 2) for t in ("256x256", "128x128", "64x64")]


def sweep(torch, torch_ops, names, steps, warmup):
    """Time every built configuration on the named workloads; one JSON line per measurement."""
    import tiled_bf16_gemm_amd as tbg
    import workloads
    results = []
    for name in names:
        if name in workloads.CONVS:
            w = workloads.CONVS[name]
            # the im2col tiles (two-stage ring) and the halo kernel (tile 448x128, four filter stages)
            for tile, st in (("256x256", 2), ("256x128", 2), ("128x128", 2), ("64x64", 2), ("448x128", 4)):
                ms, _ = time_conv(torch, torch_ops, w, steps, warmup, config=tbg.gemm_config(tile, st, "ring"))
                tf = w.flops / (ms * 1e-3) / 1e12
                r = {"workload": name, "pipeline": "ring", "tile": tile, "stages": st, "ms": round(ms, 5),
                     "tflops": round(tf, 2), "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
                print(json.dumps(r), flush=True)
                results.append(r)
            torch.cuda.empty_cache()
            continue
        wname, _, ab = name.partition("@")
        ab = ab or "bf16"
        w = workloads.GEMMS[wname]
        configs = SWEEP_CONFIGS
        if ab == "f16":
            configs = SWEEP_CONFIGS_F16
        elif ab.startswith("f8"):
            configs = SWEEP_CONFIGS_F8
        # operands once per workload; every configuration gets a short settle of its own region
        # first (after idle time the device runs the first launches slow, see time_gemm_detail)
        ops = gemm_operands(torch, w, ab)
        for pipe, tile, st in configs:
            cfg = tbg.gemm_config(tile, st, pipe)
            ms = time_gemm_detail(torch, torch_ops, w, steps, warmup, config=cfg, ab=ab, settle_s=0.1,
                                  operands=ops)["ms_step"]
            tf = w.flops / (ms * 1e-3) / 1e12
            r = {"workload": name, "pipeline": pipe, "tile": tile, "stages": st, "ms": round(ms, 5),
                 "tflops": round(tf, 2), "pct_peak": round(100 * tf / PEAK_TFLOPS[ab], 2)}
            if ab == "bf16" and wname in ("c1", "c2", "c3"):
                # launch-bound products: the GPU time per product from graph replays as well
                gms = time_gemm_graph(torch, torch_ops, w, config=cfg)
                r["graph_ms"] = round(gms, 5)
                r["graph_tflops"] = round(w.flops / (gms * 1e-3) / 1e12, 2)
            print(json.dumps(r), flush=True)
            results.append(r)
        del ops
        torch.cuda.empty_cache()
    return results


SWEEP_CMD = "python -u bench.py --sweep c1,c2,c3,c4,c5,conv_b,c4@f16,c4@f8e4m3,c5@f8e4m3 > <out>/sweep.jsonl"


# The barrier-ring configurations tbg_diag_gemm_timeline instruments: (name, BM, BN, stages).
TIMELINE_CFGS = [("ring 128x128/2", 128, 128, 2), ("ring 256x128/3", 256, 128, 3), ("ring 256x256/2", 256, 256, 2),
                 ("ring 64x64/3", 64, 64, 3)]


def timeline_stats(tl, ktiles: int, tile_bytes: int) -> dict:
    """Summary of one launch's per-workgroup timelines (gemm_ring.hpp, CLK 2: eight values per
    workgroup: real-time counter at start, first tile landed, K loop done, stores done (100 MHz
    ticks); shader-clock ticks over the whole; HW_ID; XCC_ID).  Times in µs from the first
    workgroup's start.  The copy rate is per CU: the tile bytes every workgroup on a CU copied,
    over the span of those workgroups' K loops, in bytes per shader clock, for the CUs holding the
    most workgroups."""
    import statistics
    med = statistics.median
    t0 = min(r[0] for r in tl)
    us = lambda x: x / 100.0  # noqa: E731  (100 MHz ticks)
    start = [us(r[0] - t0) for r in tl]
    first = [us(r[1] - r[0]) for r in tl]
    loop = [us(r[2] - r[1]) for r in tl]
    epi = [us(r[3] - r[2]) for r in tl]
    end = [us(r[3] - t0) for r in tl]
    ghz = med([r[4] / (us(r[3] - r[0]) * 1e3) for r in tl if r[3] > r[0]])
    # the CU: XCD, shader engine, shader array and CU fields of HW_ID
    cus = {}
    for r in tl:
        cu = (r[6] & 0xF, (r[5] >> 13) & 7, (r[5] >> 12) & 1, (r[5] >> 8) & 0xF)
        cus.setdefault(cu, []).append(r)
    most = max(len(v) for v in cus.values())
    rates = []
    for v in cus.values():
        if len(v) == most:
            t = us(max(r[2] for r in v) - min(r[1] for r in v))
            if t > 0:
                rates.append(len(v) * ktiles * tile_bytes / (t * 1e3 * ghz))
    return {"workgroups": len(tl), "cus": len(cus), "max_wg_per_cu": most,
            "start_us": {"median": round(med(start), 2), "max": round(max(start), 2)},
            "first_tile_us": round(med(first), 2), "k_loop_us": round(med(loop), 2),
            "per_k_tile_us": round(med(loop) / ktiles, 3), "epilogue_us": round(med(epi), 2),
            "end_us": {"min": round(min(end), 2), "median": round(med(end), 2), "max": round(max(end), 2)},
            "clock_ghz": round(ghz, 3), "copy_bytes_per_clk_per_cu": round(med(rates), 1) if rates else None,
            "xcds": _timeline_xcds(tl)}


def _timeline_xcds(tl) -> list:
    """Per XCD (XCC_ID): workgroups, median shader clock (GHz) and median K-loop time (µs) of its
    workgroups, and the correlation of the two over the XCDs (None with fewer than 3 XCDs)."""
    import statistics
    by = {}
    for r in tl:
        by.setdefault(r[6] & 0xF, []).append(r)
    out = []
    for x in sorted(by):
        v = by[x]
        ghz = statistics.median(r[4] / ((r[3] - r[0]) * 10.0) for r in v if r[3] > r[0])
        out.append({"xcd": x, "workgroups": len(v), "clock_ghz": round(ghz, 3),
                    "k_loop_us": round(statistics.median((r[2] - r[1]) / 100.0 for r in v), 2)})
    return out


def _correlation(xs, ys):
    n = len(xs)
    if n < 3:
        return None
    mx, my = sum(xs) / n, sum(ys) / n
    sxy = sum((a - mx) * (b - my) for a, b in zip(xs, ys))
    sxx = sum((a - mx) ** 2 for a in xs)
    syy = sum((b - my) ** 2 for b in ys)
    return round(sxy / (sxx * syy) ** 0.5, 3) if sxx > 0 and syy > 0 else None


def timeline(torch, names=("c2", "c3", "c4")) -> None:
    """Per-workgroup timelines of the barrier ring on the launch-bound products, one JSON line per
    (workload, configuration): tbg_diag_gemm_timeline on the operands in the form the product
    runs on (rows padded with zeros to a multiple of 8 elements, K rounded up to 8: what the
    library's repack produces), 30 untimed launches, then 20 launches timed with HIP events and
    the timelines of the last."""
    import ctypes
    import statistics
    import workloads
    lib = diag_lib()
    ci, ll, vp = ctypes.c_int, ctypes.c_longlong, ctypes.c_void_p
    lib.tbg_diag_gemm_timeline.restype = ci
    lib.tbg_diag_gemm_timeline.argtypes = [ci, vp, vp, vp, ci, ci, ci, ll, ll, ll, ci, vp, ctypes.POINTER(ci), vp]
    for name in names:
        w = workloads.GEMMS[name]
        assert w.b_layout == "kn"
        A, B = workloads.gemm_inputs(w)
        r8 = lambda x: (x + 7) // 8 * 8  # noqa: E731
        K8, N8 = r8(w.K), r8(w.N)
        Ap = torch.zeros((w.M, K8), dtype=torch.bfloat16)
        Ap[:, :w.K] = A[:, :w.K]
        Bp = torch.zeros((K8, N8), dtype=torch.bfloat16)
        Bp[:w.K, :w.N] = B[:, :w.N]
        Ap, Bp = Ap.cuda(), Bp.cuda()
        out_bf16 = 1 if w.out_dtype == "bf16" else 0
        C = torch.empty((w.M, w.N), dtype=torch.bfloat16 if out_bf16 else torch.float32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        for cfg, (cname, bm, bn, stages) in enumerate(TIMELINE_CFGS):
            nwg = ((w.M + bm - 1) // bm) * ((w.N + bn - 1) // bn)
            tl = torch.zeros(8 * nwg, dtype=torch.int64, device="cuda")
            got = ci(0)

            def launch():
                st = lib.tbg_diag_gemm_timeline(cfg, Ap.data_ptr(), Bp.data_ptr(), C.data_ptr(), w.M, w.N, K8, K8, N8,
                                                w.N, out_bf16, tl.data_ptr(), ctypes.byref(got), stream)
                if st != 0:
                    raise RuntimeError(f"tbg_diag_gemm_timeline: hipError {st}")
            for _ in range(30):
                launch()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
            for a, b in ev:
                a.record()
                launch()
                b.record()
            torch.cuda.synchronize()
            assert got.value == nwg
            stats = timeline_stats(tl.view(-1, 8).cpu().tolist(), (K8 + 63) // 64, (bm + bn) * 64 * 2)
            line = {"timeline": name, "M": w.M, "N": w.N, "K": w.K, "out": w.out_dtype, "config": cname,
                    "launch_us": round(1e3 * statistics.median(a.elapsed_time(b) for a, b in ev), 2)}
            line.update(stats)
            print(json.dumps(line), flush=True)


def write_timeline_profile(jsonl: str, out_dir: str) -> None:
    """profiles/gemm_ring_timeline.md from the JSON lines of one `--timeline` run."""
    rows = [json.loads(l) for l in open(jsonl) if l.startswith("{")]
    lines = ["# Per-workgroup timelines of the barrier ring: the launch-bound products and 8192³", "",
             "Each workgroup of the library's barrier-ring kernel, built with timeline recording "
             "(`tiled_bf16_gemm_amd/csrc/gemm_ring.hpp`, CLK 2; `tiled_bf16_gemm_amd/diag/mfma_rate.hip`, "
             "`tbg_diag_gemm_timeline`), records the 100 MHz real-time counter at its start, once its first K "
             "tile has landed in LDS, after its K loop and once its stores have completed, the shader clock "
             "over the whole, and the CU it ran on.  Operands in the form the product runs on (the repack's "
             "zero-padded rows).  Medians over the workgroups of one launch, after 30 untimed launches; "
             "\"launch\" is the median of 20 launches timed with HIP events on the launch stream (it includes the "
             "dispatch of the grid).  Copy rate: the K tiles' bytes copied by all workgroups of a CU over the "
             "span of their K loops, per shader clock, for the CUs holding the most workgroups.", "",
             "Command (run from the repository root on an MI355X; <out> an output folder), then "
             "`python bench.py --timeline-md <out>/timeline.jsonl`:", "", "```",
             "python -u bench.py --timeline > <out>/timeline.jsonl", "```", ""]
    for name in dict.fromkeys(r["timeline"] for r in rows):
        rs = [r for r in rows if r["timeline"] == name]
        r0 = rs[0]
        lines += [f"## {name}: {r0['M']}×{r0['N']}×{r0['K']} (B K×N, {r0['out']} out)", "",
                  "| configuration | workgroups | CUs | max per CU | launch µs | last store done µs | first tile µs | "
                  "K loop µs | per K tile µs | epilogue µs | clock GHz | copy B/clk per CU |",
                  "|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for r in rs:
            lines.append(f"| {r['config']} | {r['workgroups']} | {r['cus']} | {r['max_wg_per_cu']} | {r['launch_us']} | "
                         f"{r['end_us']['max']} | {r['first_tile_us']} | {r['k_loop_us']} | {r['per_k_tile_us']} | "
                         f"{r['epilogue_us']} | {r['clock_ghz']} | {r['copy_bytes_per_clk_per_cu']} |")
        lines.append("")
        # per XCD, for the configuration the library picks on this workload
        pick = {"c2": "ring 64x64/3", "c3": "ring 128x128/2", "c4": "ring 256x256/2"}.get(name)
        rp = [r for r in rs if r["config"] == pick and r.get("xcds")]
        if rp:
            xs = rp[0]["xcds"]
            corr = _correlation([x["clock_ghz"] for x in xs], [x["k_loop_us"] for x in xs])
            lines += [f"Per XCD, {pick} (correlation of clock and K-loop time over the XCDs: {corr}):", "",
                      "| XCD | workgroups | clock GHz | K loop µs |", "|---|---|---|---|"]
            lines += [f"| {x['xcd']} | {x['workgroups']} | {x['clock_ghz']} | {x['k_loop_us']} |" for x in xs]
            lines.append("")
    with open(os.path.join(out_dir, "gemm_ring_timeline.md"), "w") as f:
        f.write("\n".join(lines))


def write_sweep_profiles(jsonl: str, out_dir: str) -> None:
    """profiles/gemm_pipeline_sweep.md, gemm_f16_f8_sweep.md and conv_pipeline_sweep.md from the
    JSON lines of one `--sweep` run: one table per workload, the fastest configuration marked
    (by GPU time from graph replays where measured), and for the bf16 configurations the throughput
    on c4 and c5 relative to the 256x256 ring (the efficiencies of the automatic choice)."""
    import workloads
    rows = [json.loads(l) for l in open(jsonl) if l.startswith("{")]
    by = {}
    for r in rows:
        by.setdefault(r["workload"], []).append(r)
    desc = {"c1": "256³ (B K×N, fp32 out)", "c2": "1024³ (B K×N, bf16 out)",
            "c3": "3001×2049×777 (B K×N, fp32 out, repack path)", "c4": "8192³ (B K×N, bf16 out)",
            "c5": "16384×14336×4096 (B N×K, bf16 out)", "c4@f16": "8192³, fp16 inputs",
            "c4@f8e4m3": "8192³, E4M3 inputs (B N×K)", "c5@f8e4m3": "16384×14336×4096, E4M3 inputs"}

    def table(name, rs, peak_note):
        graph = any("graph_ms" in r for r in rs)
        key = (lambda r: r["graph_ms"]) if graph else (lambda r: r["ms"])
        best = min(key(r) for r in rs)
        lines = [f"## {name}: {desc.get(name, name)}", ""]
        if graph:
            lines += ["| pipeline | tile | stages | µs per call | µs GPU (graph) | TFLOP/s (graph) | % peak (graph) |",
                      "|---|---|---|---|---|---|---|"]
            for r in rs:
                b = " **best**" if key(r) == best else ""
                lines.append(f"| {r['pipeline']} | {r['tile']} | {r['stages']} | {1e3 * r['ms']:.1f} | "
                             f"{1e3 * r['graph_ms']:.2f} | {r['graph_tflops']}{b} | "
                             f"{100 * r['graph_tflops'] / peak_note:.2f} |")
        else:
            lines += ["| pipeline | tile | stages | µs | TFLOP/s | % peak |", "|---|---|---|---|---|---|"]
            for r in rs:
                b = " **best**" if key(r) == best else ""
                lines.append(f"| {r['pipeline']} | {r['tile']} | {r['stages']} | {1e3 * r['ms']:.1f} | "
                             f"{r['tflops']}{b} | {r['pct_peak']} |")
        return lines + [""]

    head = ["Command (run from the repository root on an MI355X; <out> an output folder), then "
            "`python bench.py --sweep-md <out>/sweep.jsonl`:", "", "```", SWEEP_CMD, "```", "",
            "Each configuration: its region (5 warm-up calls, then 20 calls between two HIP events on the launch "
            "stream; per-call times include the host where it is slower than the GPU) run untimed for 0.1 s, then "
            "once timed; operands generated "
            "once per workload; for c1-c3 also 20 products captured in a HIP graph and replayed 20 times "
            "(GPU time per product).  One pass on one MI355X; boxes differ by a few per cent.", ""]
    # bf16 GEMM
    lines = ["# GEMM pipeline × tile × stages sweep", "",
             "Every built configuration of `tbg_gemm_configured` (barrier ring and producer/consumer ring, each "
             "workgroup tile, each stage count that fits LDS and the vmcnt counter).  % of the 2516.6 TFLOP/s dense "
             "bf16 peak.", ""] + head
    rel = {}
    for name in ("c4", "c5"):
        rs = by.get(name, [])
        ref = [r["tflops"] for r in rs if r["pipeline"] == "ring" and r["tile"] == "256x256"]
        for r in rs:
            if ref:
                rel.setdefault((r["pipeline"], r["tile"], r["stages"]), []).append(r["tflops"] / ref[0])
    if rel:
        lines += ["Throughput relative to the 256×256 ring on c4 and c5 (the automatic choice's efficiencies are "
                  "taken from these):", "", "| pipeline | tile | stages | c4 | c5 | mean |", "|---|---|---|---|---|---|"]
        for (pipe, tile, st), v in rel.items():
            cells = " | ".join(f"{x:.2f}" for x in v) + (" | " if len(v) == 1 else "")
            lines.append(f"| {pipe} | {tile} | {st} | {cells} | {sum(v) / len(v):.2f} |")
        lines.append("")
    for name in ("c1", "c2", "c3", "c4", "c5"):
        if name in by:
            lines += table(name, by[name], PEAK_BF16_TFLOPS)
    with open(os.path.join(out_dir, "gemm_pipeline_sweep.md"), "w") as f:
        f.write("\n".join(lines))
    # fp16 / fp8
    lines = ["# fp16 and fp8 GEMM configurations: 8192³ and 16384×14336×4096", "",
             "Inputs: the workload's values converted to the input type; 8-bit inputs take B stored N×K.  Peaks: "
             "fp16 2516.6 TFLOP/s, fp8 5033.2 TFLOP/s (dense).", ""] + head
    for name in ("c4@f16", "c4@f8e4m3", "c5@f8e4m3"):
        if name in by:
            lines += table(name, by[name], PEAK_TFLOPS[name.partition("@")[2]])
    with open(os.path.join(out_dir, "gemm_f16_f8_sweep.md"), "w") as f:
        f.write("\n".join(lines))
    # convolution
    cw = workloads.CONVS["conv_b"]
    lines = ["# Implicit-GEMM convolution: tile sweep on the benchmark layer", "",
             f"Layer conv_b: batch {cw.n}, {cw.h}×{cw.w}, {cw.c} → {cw.k} channels, {cw.r}×{cw.s} filter, padding 1, "
             f"bf16 in, fp32 accumulate, bf16 out (NHWC / KRSC / NHWK).  As a GEMM: {cw.M} × {cw.k} × "
             f"{cw.r * cw.s * cw.c}.  Tile forced through the configuration: the im2col kernels (ring, two "
             f"stages) and the halo kernel (tile 448x128: the input window copied into LDS once per "
             f"32-channel block, four filter stages; nine-tap loop for this 3×3 filter).", ""] + head
    if "conv_b" in by:
        lines += table("conv_b", by["conv_b"], PEAK_BF16_TFLOPS)
    with open(os.path.join(out_dir, "conv_pipeline_sweep.md"), "w") as f:
        f.write("\n".join(lines))


def _read_bench_line(path: str):
    """The last JSON line a bench run wrote to `path`, or None."""
    try:
        with open(path) as f:
            lines = [ln for ln in f.read().splitlines() if ln.startswith("{")]
        return json.loads(lines[-1]) if lines else None
    except (OSError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--settle", type=float, default=0.25, metavar="SECONDS",
                    help="untimed calls of the headline product right before its warm-up, for at least this long "
                         "(reported as roofline.settle; 0: none).  After any idle time the device needs about 40 "
                         "launches of this product (~30 ms) before its power controller settles; the per-workload "
                         "rows get a settle of a third of this")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the GEMM's own shader clock (a clock-recording build of the same kernel, after the "
                         "timed steps)")
    ap.add_argument("--sweep-md", default="", metavar="JSONL",
                    help="write the sweep summaries in profiles/ from the JSON lines of a --sweep run (no GPU needed)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the products-alone ceiling measured next to the GEMM (roofline.ceiling)")
    ap.add_argument("--only-copies", action="store_true",
                    help="time only the tiled-copy kernel on the three copy workloads; one JSON line each")
    ap.add_argument("--counters", action="store_true",
                    help="profiling driver: 5 GEMM launches on the 8192^3 workload, then 5 plain device copies "
                         "of 512 MiB (the calibration kernel for HBM byte counters); prints no JSON")
    ap.add_argument("--summarize", default="", metavar="DIR",
                    help="write the profiles/ summaries from rocprofv3 runs under DIR (DIR/trace with the traced "
                         "bench line in DIR/trace/bench_line.json, DIR/fetch, DIR/write and optionally DIR/sq and "
                         "DIR/copytrace, each made with -o run as the summaries' commands show); the traced bench "
                         "line is also written to profiles/bench_8192_line.json; runs on any host, no GPU needed")
    ap.add_argument("--bench-kernel-us", type=float, default=None,
                    help="with --summarize: the bench line's HIP-event kernel average, quoted beside the trace")
    ap.add_argument("--timeline", action="store_true",
                    help="per-workgroup timelines of the barrier ring on c2, c3 and c4 (tbg_diag_gemm_timeline); one "
                         "JSON line per configuration instead of the bench line")
    ap.add_argument("--timeline-md", default="", metavar="JSONL",
                    help="write profiles/gemm_ring_timeline.md from the JSON lines of a --timeline run (no GPU)")
    ap.add_argument("--sweep", default="",
                    help="comma-separated workloads (c1..c5, conv_b; a GEMM name may carry an input type, e.g. "
                         "c4@f16, c4@f8e4m3): time every built pipeline/tile/stages configuration on each and print "
                         "one JSON line per measurement instead of the bench line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the GEMM shards across GPUs "
              "by rows or columns of C with no exchange, which this single-GPU build does not run.",
              file=sys.stderr)
        sys.exit(2)

    if args.sweep_md:
        write_sweep_profiles(args.sweep_md, os.path.join(ROOT, "profiles"))
        return
    if args.timeline_md:
        write_timeline_profile(args.timeline_md, os.path.join(ROOT, "profiles"))
        return

    if args.summarize:
        d = args.summarize
        cmds = {
            "trace": "cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -d <out>/trace -o run -- "
                     "python3 -u <repo>/bench.py --gpus 1 --steps 20 --warmup 5 > <out>/trace/bench_line.json",
            "fetch": "cd /tmp && TMPDIR=/tmp rocprofv3 --pmc FETCH_SIZE -d <out>/fetch -o run -- "
                     "python -u <repo>/bench.py --counters",
            "write": "cd /tmp && TMPDIR=/tmp rocprofv3 --pmc WRITE_SIZE -d <out>/write -o run -- "
                     "python -u <repo>/bench.py --counters",
            "sq": "cd /tmp && TMPDIR=/tmp rocprofv3 --pmc " + " ".join(SQ_COUNTERS) + " -d <out>/sq -o run -- "
                  "python -u <repo>/bench.py --counters",
            "copytrace": "cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -d <out>/copytrace -o run -- "
                         "python -u <repo>/bench.py --only-copies",
            "bench_kernel_us": args.bench_kernel_us,
            "bench_line": _read_bench_line(os.path.join(d, "trace", "bench_line.json")),
        }
        t = summarize_profiles(os.path.join(d, "trace", "run_results.db"), os.path.join(d, "fetch", "run_results.db"),
                               os.path.join(d, "write", "run_results.db"), os.path.join(ROOT, "profiles"), cmds,
                               os.path.join(d, "sq", "run_results.db"))
        if cmds["bench_line"]:
            with open(os.path.join(ROOT, "profiles", "bench_8192_line.json"), "w") as f:
                f.write(json.dumps(cmds["bench_line"]) + "\n")
        print(json.dumps(t))
        return

    import torch
    from tiled_bf16_gemm_amd import torch_ops
    import workloads

    torch.cuda.set_device(0)
    w = workloads.GEMMS["c4"]
    if args.counters:
        counters_driver(torch, torch_ops, w)
        return
    if args.sweep:
        sweep(torch, torch_ops, args.sweep.split(","), 20, 5)
        return
    if args.timeline:
        timeline(torch)
        return
    if args.only_copies:
        for name in ("c1_copy", "c3_copy", "c4_a_boxes"):
            ms_c, nbytes = time_copy(torch, torch_ops, workloads.COPIES[name], 50, 20)
            gbs = nbytes / (ms_c * 1e-3) / 1e9
            print(json.dumps({"copy": name, "ms": round(ms_c, 5), "bytes": nbytes, "gb_per_s": round(gbs, 1),
                              "frac": round(gbs / PEAK_HBM_GBS, 4)}), flush=True)
            torch.cuda.empty_cache()
        return
    # The headline: an untimed settle of the same product first (a device that has been idle
    # starts below its working clock; the settle's first and last launches are reported), then
    # the driver's warm-up and timed steps.
    if not args.no_clock or not args.no_ceiling:
        diag_lib()
    ops = gemm_operands(torch, w)
    head = time_gemm_detail(torch, torch_ops, w, args.steps, args.warmup, settle_s=args.settle, operands=ops)
    ms_step, ms_kernel = head["ms_step"], head["ms_kernel"]
    tflops = w.flops / (ms_step * 1e-3) / 1e12
    achieved = w.flops / (ms_kernel * 1e-3) / 1e12
    clock = None if args.no_clock else gemm_clock(torch, ops[0], ops[1], ops[3])
    cold_ms = None if args.no_configs else time_gemm_cold(torch, torch_ops, w, ops)
    del ops
    torch.cuda.empty_cache()

    per_config = {}
    if not args.no_configs:
        for name in ("c1", "c2", "c3", "c5"):
            cw = workloads.GEMMS[name]
            s, k, _ = time_gemm(torch, torch_ops, cw, 50, 50, settle_s=args.settle / 3)
            tf = cw.flops / (s * 1e-3) / 1e12
            per_config[name] = {"M": cw.M, "N": cw.N, "K": cw.K, "b_layout": cw.b_layout, "out": cw.out_dtype,
                                "ms": round(s, 5), "tflops": round(tf, 2), "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
            if name in ("c1", "c2", "c3"):
                # launch-bound shapes: also the GPU time per product from graph replays
                gms = time_gemm_graph(torch, torch_ops, cw)
                per_config[name]["graph_ms"] = round(gms, 5)
                per_config[name]["graph_tflops"] = round(cw.flops / (gms * 1e-3) / 1e12, 2)
            torch.cuda.empty_cache()
        per_config["c4"] = {"M": w.M, "N": w.N, "K": w.K, "b_layout": w.b_layout, "out": w.out_dtype,
                            "ms": round(ms_step, 5), "tflops": round(tflops, 2),
                            "pct_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
                            # each product after a 512 MiB overwrite: operands from HBM, not the caches
                            "cold_ms": round(cold_ms, 5), "cold_tflops": round(w.flops / (cold_ms * 1e-3) / 1e12, 2),
                            "cold_calls": COLD_CALLS}
        for ab in ("f16", "f8e4m3"):
            s_, _, _ = time_gemm(torch, torch_ops, w, 50, 50, ab=ab, settle_s=args.settle / 3)
            tf = w.flops / (s_ * 1e-3) / 1e12
            per_config[f"c4_{ab}"] = {"M": w.M, "N": w.N, "K": w.K, "inputs": ab,
                                      "b_layout": "nk" if ab.startswith("f8") else w.b_layout, "out": w.out_dtype,
                                      "ms": round(s_, 5), "tflops": round(tf, 2), "peak": PEAK_TFLOPS[ab],
                                      "pct_peak": round(100 * tf / PEAK_TFLOPS[ab], 2)}
            torch.cuda.empty_cache()
        for name in ("c1_copy", "c3_copy", "c4_a_boxes"):
            cw = workloads.COPIES[name]
            ms_c, nbytes = time_copy(torch, torch_ops, cw, 50, 20)
            gbs = nbytes / (ms_c * 1e-3) / 1e9
            per_config[name] = {"boxes": len(cw.coords), "box": list(cw.box), "estr": list(cw.estr),
                                "swizzle": cw.swizzle, "oob": cw.oob, "bytes": nbytes, "ms": round(ms_c, 5),
                                "gb_per_s": round(gbs, 1), "peak_gb_per_s": PEAK_HBM_GBS,
                                "frac": round(gbs / PEAK_HBM_GBS, 4)}
            if name != "c4_a_boxes":
                # launch-bound copies: the GPU time per launch from graph replays as well
                gms = time_copy_graph(torch, torch_ops, cw)
                per_config[name]["graph_ms"] = round(gms, 5)
                per_config[name]["graph_gb_per_s"] = round(nbytes / (gms * 1e-3) / 1e9, 1)
            torch.cuda.empty_cache()
        cw = workloads.CONVS["conv_b"]
        s_, _ = time_conv(torch, torch_ops, cw, 50, 20)
        tf = cw.flops / (s_ * 1e-3) / 1e12
        per_config["conv_b"] = {"conv": f"N={cw.n} H=W={cw.h} C={cw.c} K={cw.k} {cw.r}x{cw.s} pad 1 (implicit GEMM "
                                        f"{cw.M}x{cw.k}x{cw.r * cw.s * cw.c})", "out": cw.out_dtype, "ms": round(s_, 5),
                                "tflops": round(tf, 2), "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}

    ceiling = None
    if not args.no_ceiling:
        c_tf, c_ghz = mfma_ceiling(torch, 0)
        ceiling = {"what": "bf16 16x16x32 products alone on register-resident random operands (no loads, no stores), "
                           "same process, after the GEMM", "tflops": round(c_tf, 1), "clock_ghz": round(c_ghz, 3),
                   "frac_of_peak": round(c_tf / PEAK_BF16_TFLOPS, 4)}
    if ceiling and "c4_f8e4m3" in per_config:
        f_tf, f_ghz = mfma_ceiling(torch, 1)
        fc = per_config["c4_f8e4m3"]
        fc["ceiling"] = {"what": "fp8 16x16x128 products alone on register-resident random E4M3 operands",
                         "tflops": round(f_tf, 1), "clock_ghz": round(f_ghz, 3),
                         "frac_of_peak": round(f_tf / PEAK_TFLOPS["f8e4m3"], 4)}
        fc["frac_of_ceiling"] = round(fc["tflops"] / f_tf, 4)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w)

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": "gemm M=N=K=8192, A bf16 row-major, B bf16 row-major KxN, uniform[-1,1] "
                               "(seeds 4001/4002), fp32 accumulate, bf16 out",
                   "M": w.M, "N": w.N, "K": w.K, "global_batch": 1, "parallelism": "none (1 GPU)"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": load_traffic(),
            "kernel_ms": round(ms_kernel, 5),
            "launch_ms": launch_stats(head["per"]),
            # the per-launch spread: a region after the timed one, its warm-up and its launches
            # each bracketed by a pair of events
            "spread_calls": args.warmup + args.steps,
            "flops_per_launch": w.flops,
            "settle": head["settle"],
            "gemm_clock_ghz": clock,
            "ceiling": ceiling,
            "frac_of_ceiling": round(achieved / ceiling["tflops"], 4) if ceiling else None,
        },
        "cpu_baseline": cpu,
        "per_config": per_config,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
