"""Shape sweep over the nine kernel variants and the selection table it yields.

This is the data-collection step of the tuning method in the digest of
"Leveraging Large-Scale Data for Efficient Low-Bit CUTLASS GEMM Optimization via
Neural Networks" (Research results, item 2): every template (3 tile sizes x 3
pipeline depths) is timed on each (M, N, K) of a grid on the target GPU, and each
shape is labelled with its fastest template.  Timings are measured on the GPU
(median of repeated HIP-event timings of graph-replayed batches, hot caches), not
simulated.

  python -m bit_integer_gemm_amd.sweep run   --dtype s8 --out sweep_s8.jsonl
  python -m bit_integer_gemm_amd.sweep table sweep_s8.jsonl [...] --write

`run` appends one JSON line per (shape, variant) and skips those already in the
output file, so an interrupted sweep resumes.  It also checks that all nine
variants return identical C on every shape.  `table` turns measurements into
labels: the fastest variant, where every variant within EPS of the fastest
counts as tied and a tie goes to the default variant, else to the lowest index
(timing noise on short kernels must not make the selected variant slower than
the default, nor flip labels between near-equal variants), and writes
csrc/selector_table.inc: each grid shape's label and runner-up, and its nine
times over the fastest in thousandths (from which the library's table mode
takes, for a shape off the grid, the variant with the best worst case over the
grid shapes that bracket it).

Inputs: for each K, one seeded uniform operand pair of the largest M and N is
drawn (int8 over [-128, 127], int4 over [-8, 7], Bernoulli(0.5) bits) and each
shape uses its leading rows, which are contiguous for row-major A and for B's
(N, K) rows.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TABLE = os.path.join(PKG, "csrc", "selector_table.inc")

DTYPES = {"s8": 0, "s4": 1, "b1": 2}
GRID_MN = [2 ** e for e in range(6, 15)]          # 64 .. 16384
GRID_K = {"s8": [256, 1024, 4096, 8192], "s4": [256, 1024, 4096, 8192], "b1": [1024, 4096, 8192, 32768]}
EPS = 0.02
DEFAULT = 7


def time_calls(fn, torch, target_ms=12.0, min_reps=3, max_reps=2000, groups=3, graph=True):
    """Median per-call seconds of fn() over `groups` HIP-event-timed batches.

    With graph=True the batch of calls is captured once into a HIP graph and
    replayed, so that host-side launch cost (Python marshalling, ~10 us per
    call) does not pad the timings of kernels shorter than it.
    """
    fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    fn()
    e1.record(s)
    torch.cuda.synchronize()
    est = max(e0.elapsed_time(e1) / 1e3, 1e-6)
    reps = int(min(max_reps, max(min_reps, math.ceil(target_ms / 1e3 / est / groups))))
    run_batch = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        torch.cuda.synchronize()
        run_batch = g.replay
        run_batch()
        torch.cuda.synchronize()
    else:
        def run_batch():
            for _ in range(reps):
                fn()
    samples = []
    s = torch.cuda.current_stream()
    for _ in range(groups):
        e0.record(s)
        run_batch()
        e1.record(s)
        torch.cuda.synchronize()
        samples.append(e0.elapsed_time(e1) / 1e3 / reps)
    return statistics.median(samples), reps


def _operands(dtype, K, torch, Mmax, Nmax):
    sys.path.insert(0, ROOT)
    import inputs
    kidx = GRID_K[dtype].index(K) if K in GRID_K[dtype] else K
    sa, sb = 4_000_000 + 100 * DTYPES[dtype] + kidx, 4_500_000 + 100 * DTYPES[dtype] + kidx
    if dtype == "s8":
        A, B = inputs.s8_rows(Mmax, K, sa), inputs.s8_rows(Nmax, K, sb)
    elif dtype == "s4":
        A, B = inputs.s4_rows(Mmax, K, sa), inputs.s4_rows(Nmax, K, sb)
    else:
        A, B = inputs.b1_rows(Mmax, K, sa), inputs.b1_rows(Nmax, K, sb)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    if dtype == "b1":
        dA, dB = dA.view(torch.int32), dB.view(torch.int32)
    return dA, dB


def prewarm(torch, ms=200.0):
    """Keep the GPU busy for `ms` so that timings start at steady-state clocks."""
    x = torch.empty(4096, 4096, device="cuda")
    t_end = time.perf_counter() + ms / 1e3
    while time.perf_counter() < t_end:
        for _ in range(10):
            x = torch.mm(x, x)
        torch.cuda.synchronize()
    del x


def run_sweep(dtype, out_path, Ms=None, Ns=None, Ks=None, check=True, log=print):
    import torch
    import bit_integer_gemm_amd as lb
    lb.load()
    prewarm(torch)
    Ms, Ns, Ks = Ms or GRID_MN, Ns or GRID_MN, Ks or GRID_K[dtype]
    done = set()
    if os.path.exists(out_path):
        for line in open(out_path):
            r = json.loads(line)
            done.add((r["M"], r["N"], r["K"], r["variant"]))
    call = {"s8": lb.lb_gemm_s8, "s4": lb.lb_gemm_s4, "b1": lb.lb_gemm_b1}[dtype]
    f = open(out_path, "a")
    for K in Ks:
        dA, dB = _operands(dtype, K, torch, max(Ms), max(Ns))
        for M in Ms:
            for N in Ns:
                todo = [v for v in range(9) if (M, N, K, v) not in done]
                if (M, N, K, "auto") not in done:
                    todo.append("auto")
                if not todo:
                    continue
                A, B = dA[:M], dB[:N]
                C = torch.empty(M, N, dtype=torch.int32, device="cuda")
                ref = None
                if check:
                    call(A, B, C, DEFAULT)
                    ref = C.clone()
                line_t = []
                sel = lb.lb_select_variant(DTYPES[dtype], M, N, K, 0)
                for v in todo:
                    # "auto": the library's own choice (LB_AUTO), which may add a
                    # two-launch split or K bands on top of the selected variant;
                    # the selected variant is timed again right before it, so
                    # that the two compare at the same clocks
                    vv = lb.LB_AUTO if v == "auto" else v
                    t_adj = time_calls(lambda: call(A, B, C, sel[0]), torch)[0] if v == "auto" else None
                    t, reps = time_calls(lambda: call(A, B, C, vv), torch)
                    agree = bool(torch.equal(C, ref)) if check else None
                    rec = {"dtype": dtype, "M": M, "N": N, "K": K, "variant": v, "sec": t, "reps": reps,
                           "tops": 2.0 * M * N * K / t / 1e12, "agrees_with_default": agree,
                           "selected": sel[0], "second": sel[1]}
                    if t_adj is not None:
                        rec["selected_sec_adjacent"] = t_adj
                    f.write(json.dumps(rec) + "\n")
                    line_t.append(f"{'' if v == 'auto' else 'v'}{v}:{t * 1e6:.1f}")
                    if check and not agree:
                        raise RuntimeError(f"variant {v} disagrees with the default at {dtype} {M}x{N}x{K}")
                f.flush()
                del C, ref
                log(f"[sweep] {dtype} M={M} N={N} K={K} " + " ".join(line_t))
        del dA, dB
        torch.cuda.empty_cache()
    f.close()


def load_records(paths, auto=False):
    """Timings keyed by (dtype, M, N, K, variant): the nine variants, or with
    auto=True the records of the library's own choice (variant "auto").
    Reads both record formats: one line per (shape, variant) from `run`, and
    one line per shape with all nine times from `heldout`."""
    recs = {}
    for p in paths:
        for line in open(p):
            r = json.loads(line)
            if isinstance(r.get("sec"), list):
                if auto:
                    if r.get("auto_sec") is not None:
                        recs[(r["dtype"], r["M"], r["N"], r["K"], "auto")] = {"sec": r["auto_sec"]}
                    continue
                for v, t in enumerate(r["sec"]):
                    recs[(r["dtype"], r["M"], r["N"], r["K"], v)] = {"sec": t}
                continue
            if (r["variant"] == "auto") != auto:
                continue
            recs[(r["dtype"], r["M"], r["N"], r["K"], r["variant"])] = r
    return recs


def labels(recs, eps=EPS, default=DEFAULT):
    """{(dtype, M, N, K): (best, second, times[9])} with hysteresis toward the default."""
    shapes = {}
    for (d, M, N, K, v), r in recs.items():
        shapes.setdefault((d, M, N, K), [None] * 9)[v] = r["sec"]
    out = {}
    for key, ts in shapes.items():
        if any(t is None for t in ts):
            continue
        # On the times over the fastest in thousandths, as the library stores
        # them: variants within eps of the fastest are ties, the default wins a
        # tie, then the lowest index (fewest stages, then smallest tile), so
        # labels do not follow timing noise between near-equal variants.
        r = regret_permille(ts)
        order = sorted(range(9), key=lambda v: (r[v], v))
        tied = [v for v in range(9) if r[v] <= (1 + eps) * r[order[0]]]
        best = default if default in tied else min(tied)
        second = next(v for v in order if v != best)
        out[key] = (best, second, ts)
    return out


def regret_permille(ts):
    """Each variant's time over the fastest, in thousandths (capped at 65535)."""
    t0 = min(ts)
    return [min(65535, int(round(1000.0 * t / t0))) for t in ts]


def write_table(lab, path=TABLE):
    lines = ["// Generated by bit_integer_gemm_amd/sweep.py -- do not edit by hand.",
             "// Labels from variant timings measured on MI355X (median of HIP-event timings).",
             "// {dtype, log2(M), log2(N), K, best variant, second variant,",
             "//  each variant's time over the fastest in thousandths}",
             "static const SelEntry kTable[] = {"]
    items = sorted(lab.items())
    for (d, M, N, K), (b, s, ts) in items:
        r = ", ".join(str(x) for x in regret_permille(ts))
        lines.append(f"    {{{DTYPES[d]}, {int(math.log2(M))}, {int(math.log2(N))}, {K}, {b}, {s}, {{{r}}}}},")
    if not items:
        lines.append("    {-1, 0, 0, 1, 7, 8, {1000, 1000, 1000, 1000, 1000, 1000, 1000, 1000, 1000}},")
    lines.append("};")
    lines.append(f"static const int kTableLen = {len(items)};")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def evaluate(table_files, eval_files, eps=EPS, default=DEFAULT):
    """Score the compiled selection against an independent timing run.

    Uses the `selected`/`second` fields recorded by `run` (what the library's
    lb_select_variant returned) and the second run's timings as truth.
    """
    recs = load_records(eval_files)
    auto_recs = load_records(eval_files, auto=True)
    autos = {k[:4]: r["sec"] for k, r in auto_recs.items()}
    adjacent = {k[:4]: r["selected_sec_adjacent"] for k, r in auto_recs.items() if "selected_sec_adjacent" in r}
    shapes = {}
    sel = {}
    for (d, M, N, K, v), r in recs.items():
        shapes.setdefault((d, M, N, K), [None] * 9)[v] = r["sec"]
        sel[(d, M, N, K)] = (r.get("selected"), r.get("second"))
    rows = []
    for key, ts in sorted(shapes.items()):
        if any(t is None for t in ts):
            continue
        b, s2 = sel[key]
        best = min(range(9), key=lambda v: (ts[v], v))
        rows.append({"shape": key, "t": ts, "sel": b, "second": s2, "best": best})
    n = len(rows)
    if not n:
        return {"shapes": 0}
    viol = [r for r in rows if r["t"][r["sel"]] > (1 + eps) * r["t"][default]]
    sp_def = [r["t"][default] / r["t"][r["sel"]] for r in rows]
    sp_best = [r["t"][r["best"]] / r["t"][r["sel"]] for r in rows]
    # best single fixed variant: lowest geometric-mean slowdown vs per-shape best
    def gm(xs):
        return math.exp(sum(math.log(x) for x in xs) / len(xs))
    fixed = min(range(9), key=lambda v: gm([r["t"][v] / r["t"][r["best"]] for r in rows]))
    sp_fixed = [r["t"][fixed] / r["t"][r["sel"]] for r in rows]
    near = lambda r, v: r["t"][v] <= (1 + eps) * r["t"][r["best"]]  # noqa: E731
    top1 = sum(1 for r in rows if r["sel"] == r["best"]) / n
    top2 = sum(1 for r in rows if r["best"] in (r["sel"], r["second"])) / n
    top1e = sum(1 for r in rows if near(r, r["sel"])) / n
    auto = {}
    ar = [(r, autos[r["shape"]]) for r in rows if r["shape"] in autos]
    if ar:
        sp_a_def = [r["t"][default] / ta for r, ta in ar]
        # against the selected variant timed right before the automatic path
        # when the run has it (same clocks), else its own timing in the run
        sp_a_sel = [adjacent.get(r["shape"], r["t"][r["sel"]]) / ta for r, ta in ar]
        sp_a_best = [r["t"][r["best"]] / ta for r, ta in ar]
        auto = {"automatic_path": {
            "shapes": len(ar),
            "speedup_vs_default": {"geomean": gm(sp_a_def), "max": max(sp_a_def), "min": min(sp_a_def)},
            "speedup_vs_selected_variant": {"geomean": gm(sp_a_sel), "max": max(sp_a_sel), "min": min(sp_a_sel)},
            "speedup_vs_fastest_variant": {"geomean": gm(sp_a_best), "max": max(sp_a_best), "min": min(sp_a_best)},
            "slower_than_default": sum(1 for x in sp_a_def if x < 1 / (1 + eps))}}
    return {**auto,
        "shapes": n, "eps": eps, "default_variant": default,
        "violations_slower_than_default": len(viol),
        "violation_shapes": [r["shape"] for r in viol],
        "speedup_vs_default": {"geomean": gm(sp_def), "max": max(sp_def), "min": min(sp_def)},
        "best_fixed_variant": fixed,
        "speedup_vs_best_fixed": {"geomean": gm(sp_fixed), "max": max(sp_fixed), "min": min(sp_fixed)},
        "selected_vs_oracle_best": {"geomean": gm(sp_best), "min": min(sp_best)},
        "top1_accuracy": top1, "top2_accuracy": top2, "top1_within_eps": top1e,
    }


# ---------------------------------------------------------------------------
# held-out evaluation: off-grid shapes the table and the classifier never saw
# ---------------------------------------------------------------------------

K_RANGE = {"s8": (256, 16384), "s4": (256, 16384), "b1": (1024, 65536)}
K_ALIGN = {"s8": 16, "s4": 32, "b1": 128}


def train_shapes(dtype, n=500, seed=31337):
    """Seeded random shapes for building the selection (training data beside
    the grid): log-uniform M, N in 48..16384 and K over the dtype's range,
    aligned, at most 2^40 multiply-adds.  Drawn from another seed than the
    held-out shapes, so the two sets share no shape by construction."""
    import numpy as np
    g = np.random.Generator(np.random.PCG64(seed + DTYPES[dtype]))
    lo, hi = K_RANGE[dtype]
    al = K_ALIGN[dtype]
    out = []
    while len(out) < n:
        M = int(round(2 ** g.uniform(math.log2(48), 14)))
        N = int(round(2 ** g.uniform(math.log2(48), 14)))
        K = max(al, int(round(2 ** g.uniform(math.log2(lo), math.log2(hi)) / al)) * al)
        if M * N * K <= (1 << 40):
            out.append((M, N, K))
    return out


def grid_shapes(dtype):
    return [(M, N, K) for K in GRID_K[dtype] for M in GRID_MN for N in GRID_MN]


def heldout_shapes(dtype, n_random=80, seed=20260):
    """Seeded off-grid shapes for scoring the selection on data it was not
    built from: `n_random` shapes log-uniform over the sweep's range (M, N in
    48..16384, K over the dtype's range, K rounded to the alignment rule,
    powers of two avoided), then shapes that reach the automatic path's
    two-launch split (a large-tile grid whose last round is at most half
    full) and its K bands (few tiles, long K)."""
    import numpy as np
    g = np.random.Generator(np.random.PCG64(seed + DTYPES[dtype]))
    lo, hi = K_RANGE[dtype]
    al = K_ALIGN[dtype]

    def off_pow2(x, step=1):
        while x & (x - 1) == 0:
            x += step
        return x
    shapes = []
    while len(shapes) < n_random:
        M = off_pow2(int(round(2 ** g.uniform(math.log2(48), 14))))
        N = off_pow2(int(round(2 ** g.uniform(math.log2(48), 14))))
        K = off_pow2(int(round(2 ** g.uniform(math.log2(lo), math.log2(hi)) / al)) * al, al)
        if M * N * K > (1 << 40):   # keep every single call under ~0.5 s
            continue
        shapes.append((M, N, K))
    # two-launch split: tiles of 256, T > 256 CUs, last round at most half full
    for (tm, tn) in [(16, 19), (19, 16), (12, 23), (21, 13), (18, 17), (33, 9)]:
        K = [1536, 2560, 3584, 4608, 2816, 3328][len(shapes) % 6] * (1 if dtype != "b1" else 4)
        shapes.append((tm * 256 - 40, tn * 256 - 24, K))
    # K bands: few tiles, long K
    for (M, N) in [(96, 80), (200, 150), (300, 260), (130, 520), (520, 130), (60, 1000)]:
        K = {"s8": 12288, "s4": 16384, "b1": 49152}[dtype] + 3 * al
        shapes.append((M, N, K))
    # medium shapes near grid midpoints (sqrt(2) between two measured sizes)
    for (M, N, K) in [(362, 724, 1448), (1448, 2896, 2896), (5792, 2896, 1456), (2896, 11584, 720),
                      (724, 5792, 5792), (11584, 1448, 2896), (181, 181, 11584), (2048 + 96, 3072, 2048 + 160)]:
        K = off_pow2(max(lo, min(hi, K)) // al * al, al)
        shapes.append((M, N, K))
    return shapes


def run_heldout(dtype, out_path, shapes=None, log=print, passes=2, auto=True):
    """Time the nine variants, `passes` times (in alternating orders, keeping
    each one's faster median), plus the library's automatic path, on each
    shape (default: the held-out shapes); record what the table and the
    classifier select.  Also checks that every variant returns the same C as
    the default."""
    import torch
    import bit_integer_gemm_amd as lb
    lb.load()
    prewarm(torch)
    shapes = shapes or heldout_shapes(dtype)
    done = set()
    if os.path.exists(out_path):
        for line in open(out_path):
            r = json.loads(line)
            done.add((r["M"], r["N"], r["K"]))
    call = {"s8": lb.lb_gemm_s8, "s4": lb.lb_gemm_s4, "b1": lb.lb_gemm_b1}[dtype]
    gen = torch.Generator(device="cuda")
    f = open(out_path, "a")
    for i, (M, N, K) in enumerate(shapes):
        if (M, N, K) in done:
            continue
        gen.manual_seed(7_000_000 + 1000 * DTYPES[dtype] + i)
        if dtype == "s8":
            A = torch.randint(-128, 128, (M, K), generator=gen, device="cuda", dtype=torch.int8)
            B = torch.randint(-128, 128, (N, K), generator=gen, device="cuda", dtype=torch.int8)
        elif dtype == "s4":
            A = torch.randint(0, 256, (M, K // 2), generator=gen, device="cuda", dtype=torch.uint8)
            B = torch.randint(0, 256, (N, K // 2), generator=gen, device="cuda", dtype=torch.uint8)
        else:
            A = torch.randint(-2 ** 31, 2 ** 31, (M, K // 32), generator=gen, device="cuda", dtype=torch.int32)
            B = torch.randint(-2 ** 31, 2 ** 31, (N, K // 32), generator=gen, device="cuda", dtype=torch.int32)
        C = torch.empty(M, N, dtype=torch.int32, device="cuda")
        call(A, B, C, DEFAULT)
        ref = C.clone()
        sel_net = lb.lb_select_variant(DTYPES[dtype], M, N, K, 0)
        old = os.environ.get("LB_SELECTOR")
        os.environ["LB_SELECTOR"] = "table"
        sel_table = lb.lb_select_variant(DTYPES[dtype], M, N, K, 0)
        if old is None:
            os.environ.pop("LB_SELECTOR")
        else:
            os.environ["LB_SELECTOR"] = old
        order = list(range(9)) + (["auto"] if auto else [])
        best = {}
        agree = True
        for rnd in range(passes):
            for v in (order if rnd == 0 else order[::-1]):
                vv = lb.LB_AUTO if v == "auto" else v
                t, _ = time_calls(lambda: call(A, B, C, vv), torch)
                best[v] = min(best.get(v, float("inf")), t)
                if rnd == 0:
                    agree = agree and bool(torch.equal(C, ref))
        rec = {"dtype": dtype, "M": M, "N": N, "K": K, "sec": [best[v] for v in range(9)],
               "auto_sec": best.get("auto"), "table": list(sel_table), "network": list(sel_net),
               "agree": agree}
        f.write(json.dumps(rec) + "\n")
        f.flush()
        log(f"[heldout] {dtype} {M}x{N}x{K} network v{sel_net[0]} table v{sel_table[0]} "
            + " ".join(f"v{v}:{best[v] * 1e6:.1f}" for v in range(9))
            + (f" auto:{best['auto'] * 1e6:.1f}" if auto else ""))
        if not agree:
            raise RuntimeError(f"a variant disagrees with the default at {dtype} {M}x{N}x{K}")
        del A, B, C, ref
    f.close()


def library_choices(rows, cu=256):
    """What the built library selects for each row's shape, in both modes
    (host-only queries, no GPU needed): the network (the default) and the
    measured table (LB_SELECTOR=table)."""
    import bit_integer_gemm_amd as lb
    lb.load()
    old = os.environ.pop("LB_SELECTOR", None)
    try:
        for r in rows:
            r["network"] = list(lb.lb_select_variant(DTYPES[r["dtype"]], r["M"], r["N"], r["K"], cu))
        os.environ["LB_SELECTOR"] = "table"
        for r in rows:
            r["table"] = list(lb.lb_select_variant(DTYPES[r["dtype"]], r["M"], r["N"], r["K"], cu))
    finally:
        os.environ.pop("LB_SELECTOR", None)
        if old is not None:
            os.environ["LB_SELECTOR"] = old
    return rows


def score_heldout(paths, eps=EPS, default=DEFAULT, query_library=True):
    """Scores of the selection on held-out timings: violations (selected more
    than eps slower than the default), top-2 (the fastest is among the two
    predicted), top-1 within eps, selected / fastest time, and the speedups
    over the default and over the best single fixed variant (chosen on these
    shapes, so that comparison favours the fixed variant).  With
    query_library the choices are what the built library selects now (network
    and table); otherwise the ones recorded with the timings."""
    rows = [json.loads(line) for p in paths for line in open(p)]
    if not rows:
        return {}
    if query_library:
        library_choices(rows)
    else:
        for r in rows:
            r["network"] = r.get("network", r.get("mlp"))

    def gm(xs):
        return math.exp(sum(math.log(x) for x in xs) / len(xs))
    out = {"shapes": len(rows), "eps": eps, "default_variant": default}
    fixed = min(range(9), key=lambda v: gm([r["sec"][v] / min(r["sec"]) for r in rows]))
    out["best_fixed_variant"] = fixed
    for who in ("network", "table"):
        t_sel = [r["sec"][r[who][0]] for r in rows]
        best = [min(r["sec"]) for r in rows]
        fastest = [min(range(9), key=lambda v: (r["sec"][v], v)) for r in rows]
        viol = [(r["M"], r["N"], r["K"], r[who][0], round(r["sec"][r[who][0]] / r["sec"][default], 3))
                for r in rows if r["sec"][r[who][0]] > (1 + eps) * r["sec"][default]]
        out[who] = {
            "violations_slower_than_default": len(viol), "violation_shapes": viol,
            "top2_accuracy": sum(1 for r, b in zip(rows, fastest) if b in r[who][:2]) / len(rows),
            "top1_within_eps": sum(1 for ts, b in zip(t_sel, best) if ts <= (1 + eps) * b) / len(rows),
            "selected_over_fastest_time": {"geomean": gm([ts / b for ts, b in zip(t_sel, best)]),
                                           "worst": max(ts / b for ts, b in zip(t_sel, best))},
            "speedup_vs_default": {"geomean": gm([r["sec"][default] / ts for r, ts in zip(rows, t_sel)]),
                                   "min": min(r["sec"][default] / ts for r, ts in zip(rows, t_sel)),
                                   "max": max(r["sec"][default] / ts for r, ts in zip(rows, t_sel))},
            "speedup_vs_best_fixed": {"geomean": gm([r["sec"][fixed] / ts for r, ts in zip(rows, t_sel)]),
                                      "min": min(r["sec"][fixed] / ts for r, ts in zip(rows, t_sel))},
        }
    out["all_variants_agree"] = all(r["agree"] for r in rows)
    if any(r.get("auto_sec") is None for r in rows):
        return out
    # the automatic path (recorded with the library the timings were taken
    # with: its choice, plus any two-launch split or K bands)
    sp = [r["sec"][default] / r["auto_sec"] for r in rows]
    sp_sel = [r["sec"][r["network"][0]] / r["auto_sec"] for r in rows]
    out["automatic_path"] = {
        "speedup_vs_default": {"geomean": gm(sp), "min": min(sp), "max": max(sp)},
        "speedup_vs_selected_variant": {"geomean": gm(sp_sel), "min": min(sp_sel), "max": max(sp_sel)},
        "slower_than_default": [(r["M"], r["N"], r["K"], round(x, 3)) for r, x in zip(rows, sp)
                                if x < 1 / (1 + eps)]}
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--dtype", choices=sorted(DTYPES), default="s8")
    r.add_argument("--out", required=True)
    r.add_argument("--M", type=int, nargs="*")
    r.add_argument("--N", type=int, nargs="*")
    r.add_argument("--K", type=int, nargs="*")
    r.add_argument("--no-check", action="store_true")
    t = sub.add_parser("table")
    t.add_argument("files", nargs="+")
    t.add_argument("--write", action="store_true")
    e = sub.add_parser("evaluate")
    e.add_argument("files", nargs="+", help="timing runs made with the compiled table")
    e.add_argument("--json", help="write the report here")
    h = sub.add_parser("heldout")
    h.add_argument("--dtype", choices=sorted(DTYPES), default="s8")
    h.add_argument("--out", required=True)
    h.add_argument("--set", choices=("heldout", "train", "grid"), default="heldout",
                   help="held-out shapes (two passes plus the automatic path), or the "
                        "training shapes / the grid (one pass, variants only)")
    sh = sub.add_parser("score-heldout")
    sh.add_argument("files", nargs="+")
    sh.add_argument("--json", help="write the report here")
    a = ap.parse_args(argv)
    if a.cmd == "heldout":
        t0 = time.time()
        if a.set == "heldout":
            run_heldout(a.dtype, a.out, log=lambda s: print(s, flush=True))
        else:
            shapes = train_shapes(a.dtype) if a.set == "train" else grid_shapes(a.dtype)
            run_heldout(a.dtype, a.out, shapes=shapes, passes=1, auto=False,
                        log=lambda s: print(s, flush=True))
        print(f"[heldout] done in {time.time() - t0:.1f} s", flush=True)
    elif a.cmd == "score-heldout":
        rep = score_heldout(a.files)
        txt = json.dumps(rep, indent=1)
        print(txt)
        if a.json:
            with open(a.json, "w") as f:
                f.write(txt + "\n")
    elif a.cmd == "run":
        t0 = time.time()
        run_sweep(a.dtype, a.out, a.M, a.N, a.K, check=not a.no_check,
                  log=lambda s: print(s, flush=True))
        print(f"[sweep] done in {time.time() - t0:.1f} s", flush=True)
    elif a.cmd == "evaluate":
        rep = evaluate(None, a.files)
        txt = json.dumps(rep, indent=1)
        print(txt)
        if a.json:
            with open(a.json, "w") as f:
                f.write(txt + "\n")
    else:
        lab = labels(load_records(a.files))
        n_def = sum(1 for (b, _, _) in lab.values() if b == DEFAULT)
        print(f"{len(lab)} shapes labelled; default kept on {n_def}")
        if a.write:
            write_table(lab)
            print(f"wrote {TABLE}")


if __name__ == "__main__":
    main()
