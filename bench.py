#!/usr/bin/env python3
"""Benchmark of the exact low-bit GEMM on one MI355X.

One step is one pass of the whole hot path over the benchmarked workload: one
library call with automatic variant choice (the library looks the shape up in
its selection table, then launches the chosen kernel) on operands already
resident in HBM.  The default workload is the signed-int4
GEMM at M = N = K = 4096 (A row-major, B column-major, both packed two per
byte along K, C int32), on seeded uniform inputs over [-8, 7].

Prints ONE JSON line with the throughput in TOPS (2*M*N*K per GEMM), the
roofline of the GEMM kernel against MI355X's dense int8 MFMA peak, and the CPU
oracle timed on a bounded sample of the same workload.  Extra fields report the
int4 and int8 GEMMs at 4096^3, the 1-bit GEMM at 4096 x 4096 x 8192 bits and the
int8 linear layer (whole, and one GPU's share of it split eight ways by columns
or by rows), each with its selected and default variants (kernel time from
HIP-graph replays, so that host launch cost is excluded), and, as context, the
vendor library's int8 GEMM (hipBLASLt via torch._int_mm) at the same sizes; and
four low-bit convolution layers with their roofline and the time of the dense
GEMM of the same M, N, K.  ``--workload`` also accepts a convolution layer.

Usage: python bench.py [--gpus 1] [--steps 300] [--warmup 100]
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

# MI355X spec-sheet peaks (dense, no sparsity).  int8 MFMA: 256 CUs x 4 SIMDs
# x 32768 ops per 16-cycle v_mfma_i32_16x16x64_i8 x 2.4 GHz.  The 1-bit GEMM
# feeds bit planes to the FP4 MFMA, one e2m1 MAC per bit-MAC, so it is measured
# against the FP4 peak: 65536 ops per 16-cycle 16x16x128 instruction, 10.07
# P op/s (spec sheet: 10.1 PFLOP/s dense fp4).  int4 has no MFMA of its own
# and counts against the int8 peak.
PEAK_INT8_TOPS = 256 * 2.4e9 * 8192 / 1e12          # 5033.2 TOP/s, int8 MFMA
PEAK_FP4_TOPS = 256 * 2.4e9 * 16384 / 1e12          # 10066.3 TOP/s, FP4 MFMA
PEAK_HBM_GBS = 8000.0


def peak_tops(dtype):
    return PEAK_FP4_TOPS if dtype == "b1" else PEAK_INT8_TOPS


WORKLOADS = {
    # name: (dtype, M, N, K, seeds)
    "s4_gemm_4096": ("s4", 4096, 4096, 4096, (2001, 2002)),
    "s8_gemm_4096": ("s8", 4096, 4096, 4096, (4_000_001, 4_500_001)),
    "b1_gemm_4096x4096x8192": ("b1", 4096, 4096, 8192, (3001, 3002)),
    "s8_linear_8192x11008x4096": ("linear", 8192, 11008, 4096, (5001, 5002, 5003, 5004)),
    "s8_gemm_256": ("s8", 256, 256, 256, (1001, 1002)),
    # one GPU's share of the linear layer split over 8 GPUs, by columns of W
    # (and the output) and by rows of X: the shapes each GPU would run
    "s8_linear_colshard8_8192x1376x4096": ("linear", 8192, 1376, 4096, (5001, 5002, 5003, 5004)),
    "s8_linear_rowshard8_1024x11008x4096": ("linear", 1024, 11008, 4096, (5001, 5002, 5003, 5004)),
}

# Convolution layers (synthetic NHWC batches; shapes of common CNN stages, not
# a published benchmark suite): name -> (dtype, N, H, W, C, Co, Kh, Kw, stride, pad, seeds)
CONV_LAYERS = {
    "s8_conv3x3_n32_56x56x64": ("s8", 32, 56, 56, 64, 64, 3, 3, (1, 1), (1, 1), (6001, 6002)),
    "s8_conv3x3_n128_14x14x256": ("s8", 128, 14, 14, 256, 256, 3, 3, (1, 1), (1, 1), (6003, 6004)),
    "s4_conv3x3_n128_14x14x256": ("s4", 128, 14, 14, 256, 256, 3, 3, (1, 1), (1, 1), (6005, 6006)),
    "s8_conv1x1_n128_14x14x1024": ("s8", 128, 14, 14, 1024, 256, 1, 1, (1, 1), (0, 0), (6007, 6008)),
    # 7x7 stride-2 stem with the 3 input channels zero-padded to 16
    "s8_conv7x7s2_n32_224x224x16": ("s8", 32, 224, 224, 16, 64, 7, 7, (2, 2), (3, 3), (6009, 6010)),
}


# Sources that define the device code of the GEMM kernels (not the host-side
# selection table or ABI checks): counter profiles stay valid while these match.
KERNEL_SOURCES = ("lb_device.hpp", "lb_internal.hpp", "lb_mfma.hip")


def _code_only(text: str) -> str:
    """Source text without comments and blank lines (string literals in these
    files hold no comment markers), so that a comment edit keeps the hash."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln.strip())


def kernel_source_sha() -> str:
    """Hash of the device code (comments ignored); counter profiles carry it."""
    d = os.path.join(ROOT, "bit_integer_gemm_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(f.encode())
        h.update(_code_only(open(os.path.join(d, f)).read()).encode())
    return h.hexdigest()[:16]


def make_operands(dtype, M, N, K, seeds, torch):
    import inputs

    def d(a):
        return torch.from_numpy(a).cuda()
    if dtype == "s8":
        return d(inputs.s8_rows(M, K, seeds[0])), d(inputs.s8_rows(N, K, seeds[1]))
    if dtype == "s4":
        return d(inputs.s4_rows(M, K, seeds[0])), d(inputs.s4_rows(N, K, seeds[1]))
    if dtype == "b1":
        return (d(inputs.b1_rows(M, K, seeds[0])).view(torch.int32),
                d(inputs.b1_rows(N, K, seeds[1])).view(torch.int32))
    X, W = d(inputs.s8_rows(M, K, seeds[0])), d(inputs.s8_rows(N, K, seeds[1]))
    return X, W, d(inputs.scales(M, seeds[2])), d(inputs.scales(N, seeds[3]))


def step_fn(dtype, ops_, out, lb):
    """One pass of the hot path: select the variant for the shape, launch the GEMM."""
    code = {"s8": lb.LB_S8, "s4": lb.LB_S4, "b1": lb.LB_B1, "linear": lb.LB_S8}[dtype]
    if dtype == "linear":
        X, W, sx, sw = ops_
        M, K, N = X.shape[0], X.shape[1], W.shape[0]
    else:
        A, B = ops_
        M, N = A.shape[0], B.shape[0]
        K = {"s8": A.shape[1], "s4": 2 * A.shape[1], "b1": 32 * A.shape[1]}[dtype]

    def run(variant=None):
        # variant None = LB_AUTO: the library picks the variant for the shape on every call
        v = lb.LB_AUTO if variant is None else variant
        if dtype == "s8":
            lb.lb_gemm_s8(A, B, out, v)
        elif dtype == "s4":
            lb.lb_gemm_s4(A, B, out, v)
        elif dtype == "b1":
            lb.lb_gemm_b1(A, B, out, v)
        else:
            lb.lb_gemm_s8_linear(X, W, sx, sw, out, v)
        return v

    def selected():
        return lb.lb_select_variant(code, M, N, K, 0)[0]
    run.selected = selected
    return run, (M, N, K)


def conv_step(name, torch, lb):
    """One convolution call with automatic variant choice; returns run, (M, N, K), bytes."""
    import inputs
    dtype, N, H, W, C, Co, Kh, Kw, st, pd, seeds = CONV_LAYERS[name]
    mk = inputs.s8_nhwc if dtype == "s8" else inputs.s4_nhwc
    X = torch.from_numpy(mk(N, H, W, C, seeds[0])).cuda()
    F = torch.from_numpy(mk(Co, Kh, Kw, C, seeds[1])).cuda()
    Ho, Wo = lb.conv_out_dims(H, W, Kh, Kw, st, pd)
    Y = torch.empty((N, Ho, Wo, Co), dtype=torch.int32, device="cuda")
    fn = lb.lb_conv2d_s8 if dtype == "s8" else lb.lb_conv2d_s4
    M, K = N * Ho * Wo, Kh * Kw * C

    def run(variant=None):
        v = lb.LB_AUTO if variant is None else variant
        fn(X, F, Y, st, pd, v)
        return v

    def selected():
        # the convolution's automatic choice (include/lb_gemm.h): the small tile
        # for at most 64 output channels, else the GEMM's choice for the shape
        if Co <= 64:
            return 0
        return lb.lb_select_variant(lb.LB_S8 if dtype == "s8" else lb.LB_S4, M, Co, K, 0)[0]

    def auto_tile():
        # the tile an automatic call runs: for at most 64 output channels with a
        # window of several taps and at most 1024 bytes, the 64x64 tile with
        # two 64-byte stages; else the selected variant's tile
        kb = Kh * Kw * (C if dtype == "s8" else C // 2)
        if Co <= 64 and kb <= 1024 and Kh * Kw > 1:
            return "64x64, two 64-byte stages"
        info = lb.lb_variant_info(lb.LB_S8 if dtype == "s8" else lb.LB_S4, selected())
        return f"{info['tile_m']}x{info['tile_n']}, {info['stages']} stages (variant {selected()})"
    run.selected = selected
    run.auto_tile = auto_tile
    nbytes = X.numel() + F.numel() + 4 * Y.numel()
    return run, (M, Co, K), nbytes


def conv_roofline(ops, nbytes, t):
    """Bound of a convolution from its algorithmic intensity against the MFMA ridge."""
    if ops / nbytes >= PEAK_INT8_TOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        a = ops / t / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": round(PEAK_INT8_TOPS, 1),
                "unit": "TOP/s", "frac": round(a / PEAK_INT8_TOPS, 4)}
    a = nbytes / t / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(a / PEAK_HBM_GBS, 4)}


def measure_conv(name, torch, lb):
    """Convolution layer: kernel time of the automatic call (HIP-graph replay), its roofline, and the
    GEMM of the same M, N, K on dense operands (the cost of gathering windows)."""
    from bit_integer_gemm_amd.sweep import time_calls
    dtype = CONV_LAYERS[name][0]
    run, (M, N, K), nbytes = conv_step(name, torch, lb)
    sel = run.selected()
    ops_ = make_operands(dtype, M, N, K, (7001, 7002), torch)
    out = out_buffer(dtype, M, N, torch)
    grun, _ = step_fn(dtype, ops_, out, lb)
    time_calls(lambda: run(), torch, target_ms=10.0, groups=1)   # see measure()
    t = tg = float("inf")
    for _ in range(2):
        t = min(t, time_calls(lambda: run(), torch, target_ms=30.0, groups=5)[0])
        tg = min(tg, time_calls(lambda: grun(sel), torch, target_ms=30.0, groups=5)[0])
    ops = 2.0 * M * N * K
    return {"gemm_shape": [M, N, K], "variant": sel, "automatic_tile": run.auto_tile(),
            "us_per_call": round(t * 1e6, 2),
            "tops": round(ops / t / 1e12, 2), "roofline": conv_roofline(ops, nbytes, t),
            "algorithmic_bytes": nbytes, "same_shape_gemm_us": round(tg * 1e6, 2),
            "conv_over_gemm_time": round(t / tg, 4)}


def time_steps(run, steps, warmup, torch, variant=None):
    for _ in range(warmup):
        run(variant)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        run(variant)
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1e3, wall   # seconds (HIP events), seconds (host clock)


def out_buffer(dtype, M, N, torch):
    return torch.empty(M, N, dtype=torch.float32 if dtype == "linear" else torch.int32, device="cuda")


def load_traffic(workload: str, sha: str):
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None, "no counter profile"
    t = json.load(open(p))
    if t.get("kernel_src_sha") != sha:
        return None, "kernel changed since the counters were taken"
    return t.get("hbm_bytes_per_launch"), t.get("note")


def cpu_baseline(dtype, M, N, K, seeds, rows, min_seconds=10.0, max_runs=5):
    """The CPU oracle on the first `rows` rows of A against all of B (a bounded
    sample), repeated until about `min_seconds` of CPU work; the rate is the
    sample's ops over the mean time of a run."""
    import inputs
    import oracle
    if dtype == "s4":
        A, B = inputs.s4_rows(rows, K, seeds[0]), inputs.s4_rows(N, K, seeds[1])
        f = lambda: oracle.gemm_s4(A, B, K)  # noqa: E731
    elif dtype == "s8":
        A, B = inputs.s8_rows(rows, K, seeds[0]), inputs.s8_rows(N, K, seeds[1])
        f = lambda: oracle.gemm_s8(A, B)  # noqa: E731
    elif dtype == "b1":
        A, B = inputs.b1_rows(rows, K, seeds[0]), inputs.b1_rows(N, K, seeds[1])
        f = lambda: oracle.gemm_b1(A, B, K)  # noqa: E731
    else:
        raise ValueError(dtype)
    oracle.lib()
    times = []
    while len(times) < max_runs and sum(times) < min_seconds:
        t0 = time.perf_counter()
        f()
        times.append(time.perf_counter() - t0)
    dt = sum(times) / len(times)
    return {"value": round(2.0 * rows * N * K / dt / 1e12, 6), "unit": "TOPS",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{dtype} GEMM, first {rows} of {M} rows of A x all {N} columns, K={K} "
                      f"({rows / M:.1%} of the workload), {len(times)} runs, "
                      f"{dt:.2f} s wall each (mean)"}


def measure(workload, torch, lb):
    """One workload, kernel time only (HIP-graph replay): the automatic choice (what
    a caller gets: the selected variant, or for large tiles with a nearly empty
    last round of tiles two launches), the selected variant alone, and the
    default variant."""
    from bit_integer_gemm_amd.sweep import time_calls
    dtype, M, N, K, seeds = WORKLOADS[workload]
    ops_ = make_operands(dtype, M, N, K, seeds, torch)
    out = out_buffer(dtype, M, N, torch)
    run, (M, N, K) = step_fn(dtype, ops_, out, lb)
    sel = run.selected()
    # The first timed batch after a change of workload can read 10-15% slow;
    # time the selected and the default variant twice each, alternating, and
    # keep each one's faster median.
    time_calls(lambda: run(), torch, target_ms=10.0, groups=1)
    t_auto = t_sel = t_def = float("inf")
    for _ in range(2):
        t_auto = min(t_auto, time_calls(lambda: run(), torch, target_ms=30.0, groups=5)[0])
        t_sel = min(t_sel, time_calls(lambda: run(sel), torch, target_ms=30.0, groups=5)[0])
        t_def = min(t_def, time_calls(lambda: run(lb.LB_DEFAULT_VARIANT), torch, target_ms=30.0, groups=5)[0])
    t_cold = time_cold(lambda: run(), torch)
    t_int8_route = None
    if dtype == "b1":
        # the 1-bit GEMM's int8 route (weighted bit planes on the int8 MFMA)
        # beside the FP4 route that the library uses: the A/B of that choice
        os.environ["LB_B1_ROUTE"] = "int8"
        try:
            t_int8_route = min(time_calls(lambda: run(), torch, target_ms=30.0, groups=5)[0] for _ in range(2))
        finally:
            del os.environ["LB_B1_ROUTE"]
    ops = 2.0 * M * N * K
    peak = peak_tops(dtype)
    tops = ops / t_auto / 1e12
    res = {"tops": round(tops, 2), "frac_of_peak": round(tops / peak, 4), "peak_tops": round(peak, 1),
           "us_per_call": round(t_auto * 1e6, 2), "variant": sel,
           "selected_variant_alone_us": round(t_sel * 1e6, 2),
           "default_variant_us": round(t_def * 1e6, 2),
           "speedup_vs_default": round(t_def / t_auto, 4),
           "cold_us_per_call": round(t_cold * 1e6, 2), "cold_tops": round(ops / t_cold / 1e12, 2)}
    if dtype != "b1":
        res.update(vendor_int8(M, N, K, torch, t_sel))
    else:
        res.update({"int8_route_us": round(t_int8_route * 1e6, 2),
                    "fp4_route_speedup_vs_int8_route": round(t_int8_route / t_auto, 4),
                    "int8_route_frac_of_int8_peak": round(ops / t_int8_route / 1e12 / PEAK_INT8_TOPS, 4)})
        res.update(valu_b1_baseline(ops_, out, ops, t_auto, torch))
    return res


def valu_b1_baseline(ops_, out, ops, t_auto, torch):
    """The 1-bit GEMM on the vector ALUs (AND + popcount-add; the probe
    module's kernel, not part of the library) on the same operands: its time,
    its fraction of the vector-ALU peak, and whether its C equals the
    library's.  Empty when the probe library is not built."""
    from bit_integer_gemm_amd import probe
    if not os.path.exists(probe.LIB):
        return {"valu_popcount_note": "probe library not built"}
    A, B = ops_
    C = torch.empty_like(out)
    probe.valu_b1(A, B, C)
    torch.cuda.synchronize()
    same = bool(torch.equal(C, out))
    reps = 20
    probe.valu_b1(A, B, C, 3)
    t = min(probe.valu_b1(A, B, C, reps) for _ in range(3)) / reps * 1e-3
    return {"valu_popcount_us": round(t * 1e6, 2), "valu_popcount_tops": round(ops / t / 1e12, 1),
            "valu_popcount_frac_of_valu_peak": round(ops / t / 1e12 / probe.VALU_B1_PEAK_TOPS, 4),
            "speedup_vs_valu_popcount": round(t / t_auto, 3), "valu_popcount_identical": same}


def time_cold(fn, torch, reps=15, flush_mib=512):
    """Median seconds of single calls that each start with cold caches: a
    512 MiB write (twice the 256 MB last-level cache) runs before every call,
    outside its HIP-event bracket, so the operands come from HBM."""
    scratch = torch.empty(flush_mib << 20, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (e0, e1) in enumerate(ev):
        scratch.fill_(i & 0xFF)
        e0.record(s)
        fn()
        e1.record(s)
    torch.cuda.synchronize()
    del scratch
    return sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2] / 1e3


def vendor_int8(M, N, K, torch, t_ours):
    """Context only: the vendor library's int8 GEMM (hipBLASLt behind
    torch._int_mm) at the same M, N, K with the same operand layout (B stored
    N x K).  It has no int4 path and no fused dequant, so for the int4 GEMM and
    the linear layer this is the nearest library call, not the same operation."""
    from bit_integer_gemm_amd.sweep import time_calls
    try:
        a = torch.randint(-128, 128, (M, K), dtype=torch.int8, device="cuda")
        b = torch.randint(-128, 128, (N, K), dtype=torch.int8, device="cuda")
        t, _ = time_calls(lambda: torch._int_mm(a, b.t()), torch, target_ms=30.0, groups=5, graph=False)
    except Exception as e:  # the comparison is optional context
        return {"vendor_int8_note": f"torch._int_mm unavailable: {type(e).__name__}"}
    return {"vendor_int8_us": round(t * 1e6, 2), "vendor_int8_tops": round(2.0 * M * N * K / t / 1e12, 2),
            "speedup_vs_vendor_int8": round(t / t_ours, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--prewarm-ms", type=float, default=150.0,
                    help="untimed steps before the warmup steps, to let the GPU reach steady clocks")
    ap.add_argument("--workload", default="s4_gemm_4096", choices=sorted(WORKLOADS) + sorted(CONV_LAYERS))
    ap.add_argument("--cpu-rows", type=int, default=4096, help="rows of A in the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--only", action="store_true",
                    help="time only the workload (for profiler runs): no extras, no CPU leg")
    ap.add_argument("--variant", type=int, default=None,
                    help="force one kernel variant (0..8) instead of the library's choice (A/B profiling)")
    ap.add_argument("--shape", type=int, nargs=3, metavar=("M", "N", "K"), default=None,
                    help="override M, N, K of a GEMM workload (A/B profiling)")
    ap.add_argument("--lib", default=None,
                    help="load this build of the library instead of the package's (A/B profiling builds "
                         "from `python -m bit_integer_gemm_amd._build --ab NAME`)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB device copy (the reference for HBM byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the GEMM shards across GPUs without communication, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 5}))
        return
    import bit_integer_gemm_amd as lb
    if args.lib:
        lb.load(os.path.abspath(args.lib))
    lb.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)

    conv = args.workload in CONV_LAYERS
    if conv and args.shape:
        sys.exit("--shape applies to GEMM workloads only")
    if conv:
        dtype, seeds = CONV_LAYERS[args.workload][0], CONV_LAYERS[args.workload][-1]
        run, (M, N, K), conv_bytes = conv_step(args.workload, torch, lb)
    else:
        dtype, M, N, K, seeds = WORKLOADS[args.workload]
        if args.shape:
            M, N, K = args.shape
        ops_ = make_operands(dtype, M, N, K, seeds, torch)
        out = out_buffer(dtype, M, N, torch)
        run, (M, N, K) = step_fn(dtype, ops_, out, lb)
    variant = run.selected() if args.variant is None else args.variant
    if args.variant is not None:
        auto_run = run

        def run(v=None):
            return auto_run(args.variant if v is None else v)
    run()
    torch.cuda.synchronize()
    # The GPU raises its clocks over the first ~30 ms of sustained work; run
    # untimed steps for at least args.prewarm_ms before the warmup steps so that
    # the timed steps see steady-state clocks.
    t_end = time.perf_counter() + args.prewarm_ms / 1e3
    while time.perf_counter() < t_end:
        for _ in range(20):
            run()
        torch.cuda.synchronize()
    t, wall = time_steps(run, args.steps, args.warmup, torch)
    ms_per_step = t / args.steps * 1e3
    ops = 2.0 * M * N * K
    value = ops * args.steps / t / 1e12
    peak = peak_tops(dtype)
    sha = kernel_source_sha()
    traffic, traffic_note = load_traffic(args.workload, sha)

    result = {
        "metric": "low-bit GEMM TOPS (int8/int4/1-bit) at 4096^3; % of chip peak",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"s4": "int4 (int8 MFMA, int32 acc)", "s8": "int8 (int32 acc)",
                  "b1": "1-bit (bit planes on the FP4 MFMA, exact fp32 acc)",
                  "linear": "int8 (int32 acc) + fp32 dequant"}[dtype],
        "data": "synthetic (seeded uniform operands, resident in HBM)",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K, "variant": variant,
                   "variant_forced": args.variant is not None,
                   "variant_tile": lb.lb_variant_info({"s8": 0, "s4": 1, "b1": 2, "linear": 0}[dtype], variant),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(value, 2),
                     "peak": round(peak, 1), "unit": "TOP/s", "frac": round(value / peak, 4),
                     "traffic": traffic},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", "?"),
                   "cu": props.multi_processor_count},
        "kernel_src_sha": sha,
        "timed_wall_s": round(wall, 4),
    }
    if conv:
        geom = CONV_LAYERS[args.workload]
        result["metric"] = "low-bit convolution TOPS (NHWC, windows gathered into the GEMM)"
        result["config"].update({"conv": {"N": geom[1], "H": geom[2], "W": geom[3], "C": geom[4],
                                          "Co": geom[5], "Kh": geom[6], "Kw": geom[7],
                                          "stride": list(geom[8]), "pad": list(geom[9])}})
        rl = conv_roofline(ops, conv_bytes, t / args.steps)
        rl["traffic"] = traffic
        result["roofline"] = rl
    if traffic is None:
        result["roofline"]["traffic_note"] = traffic_note

    if not args.only and not args.no_extras:
        extras = {}
        for w in ("s4_gemm_4096", "s8_gemm_4096", "b1_gemm_4096x4096x8192", "s8_linear_8192x11008x4096",
                  "s8_linear_colshard8_8192x1376x4096", "s8_linear_rowshard8_1024x11008x4096", "s8_gemm_256"):
            extras[w] = measure(w, torch, lb)
        for w in CONV_LAYERS:
            extras[w] = measure_conv(w, torch, lb)
        result["extras"] = extras

    if not args.only and not args.no_cpu_baseline and not conv:
        result["cpu_baseline"] = cpu_baseline(dtype if dtype != "linear" else "s8", M, N, K, seeds,
                                              min(args.cpu_rows, M))
        cb = result["cpu_baseline"]["value"]
        result["gpu_over_cpu"] = round(value / cb, 1) if cb else None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
