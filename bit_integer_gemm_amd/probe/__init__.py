"""Measurements behind design decisions (a tool; not part of the GEMM library).

1. Matrix-instruction issue rates on gfx950.  Times the int8 16x16x64 MFMA and the scaled 16x16x128 MFMA with FP8 e4m3,
FP6 e3m2 and FP4 e2m1 operands, each wave issuing 16 independent accumulator
chains, at 1, 2 and 4 waves per SIMD; operands hold realistic bits (uniform
int8 bytes; random e3m2 codes; one bit plane per FP4 nibble, as the 1-bit GEMM
feeds it).  These rates decide which matrix instruction a low-bit operand is
worth converting to.

2. MFMA throughput with independent vector instructions between the MFMAs
(does the vector ALU run beside the matrix core, or take its issue slots?).

3. Output-store bandwidth when all workgroups store at once, when only one
XCD's do, and when one in eight of every XCD's do (256 KiB each, the int32
tile of a 256 x 256 GEMM tile), to tell a per-XCD limit from a chip-wide one.

4. Cycles per MFMA slot (s_memtime, per wave) of one wave per SIMD issuing V
vector instructions (a masking AND, a 64-bit shift) or s_nop 1 after each of
its own MFMAs: how many unpack instructions fit between a wave's MFMAs.

5. Cycles per MFMA of waves that also issue direct global->LDS copies between
their MFMAs (one wave per SIMD; copies in all four waves or in one): the cost
of a copy to its wave, and where the CU's copy path saturates.

6. The 1-bit GEMM on the vector ALUs (AND + popcount-add per pair of 32-bit
words) at 4096 x 4096 x 8192 bits, against the vector ALUs' peak and against
the library's 1-bit GEMM on the same operands (identical results required).

  python -m bit_integer_gemm_amd.probe          # prints one JSON object
"""
from __future__ import annotations

import ctypes
import json
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "probe.hip")
LIB = os.path.join(HERE, "libprobe.so")
KINDS = {"int8_16x16x64": (0, 2 * 16 * 16 * 64), "fp8_e4m3_16x16x128": (1, 2 * 16 * 16 * 128),
         "fp6_e3m2_16x16x128": (2, 2 * 16 * 16 * 128), "fp4_e2m1_16x16x128": (3, 2 * 16 * 16 * 128)}


def build() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {SRC}:\n{r.stderr[-4000:]}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def measure(target_ms: float = 8.0) -> dict:
    import torch
    lib = ctypes.CDLL(LIB)
    lib.mfma_rate_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.mfma_rate_run.restype = ctypes.c_float
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"cu": cu, "rates": {}}
    for name, (kind, ops) in KINDS.items():
        for wps in (1, 2, 4):
            blocks = cu * wps          # 4 waves per workgroup = one per SIMD
            buf = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            iters = 256
            for _ in range(2):     # the first launch also loads the code object
                ms = lib.mfma_rate_run(kind, blocks, iters, ctypes.c_void_p(buf.data_ptr()))
            if ms < 0:
                raise RuntimeError(f"probe launch failed ({ms})")
            iters = max(64, int(iters * target_ms / max(ms, 1e-3)))
            best = min(lib.mfma_rate_run(kind, blocks, iters, ctypes.c_void_p(buf.data_ptr()))
                       for _ in range(3))
            n_inst = iters * 16 * wps            # per SIMD
            out["rates"][f"{name}/waves_per_simd={wps}"] = {
                "ns_per_instruction_per_simd": round(best * 1e6 / n_inst, 3),
                "tops": round(ops * n_inst * 4 * cu / (best / 1e3) / 1e12, 1),
                "iters": iters, "ms": round(best, 3)}
            print(f"[probe] {name} waves/SIMD {wps}: {best * 1e6 / n_inst:.2f} ns per instruction per SIMD",
                  flush=True)
    return out


def measure_mix(target_ms: float = 8.0) -> dict:
    """ns per int8 MFMA per SIMD with V = 0..4 independent VALU instructions
    after each, at 1 and 2 waves per SIMD."""
    import torch
    lib = ctypes.CDLL(LIB)
    lib.mix_rate_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.mix_rate_run.restype = ctypes.c_float
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    out = {}
    for wps in (1, 2):
        blocks = cu * wps
        buf = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        for v in range(5):
            iters = 256
            for _ in range(2):
                ms = lib.mix_rate_run(v, blocks, iters, ctypes.c_void_p(buf.data_ptr()))
            if ms < 0:
                raise RuntimeError(f"mix probe failed ({ms})")
            iters = max(64, int(iters * target_ms / max(ms, 1e-3)))
            best = min(lib.mix_rate_run(v, blocks, iters, ctypes.c_void_p(buf.data_ptr())) for _ in range(3))
            ns = best * 1e6 / (iters * 16 * wps)
            out[f"waves_per_simd={wps}/valu_per_mfma={v}"] = {"ns_per_mfma_per_simd": round(ns, 3)}
            print(f"[probe] mix: {wps} wave(s)/SIMD, {v} VALU per MFMA: {ns:.2f} ns per MFMA per SIMD", flush=True)
    return out


def measure_stores(chunk_bytes: int = 256 << 10, reps: int = 5) -> dict:
    """GB/s of the store probe: all 2048 workgroups (8 per CU) storing, those of
    one XCD, and one in eight of every XCD's."""
    import torch
    lib = ctypes.CDLL(LIB)
    lib.store_rate_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.store_rate_run.restype = ctypes.c_float
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = cu * 8
    buf = torch.empty(blocks * chunk_bytes, dtype=torch.uint8, device="cuda")
    out = {}
    for mode, name, share in ((0, "all workgroups", 1.0), (1, "one XCD's workgroups", 1 / 8),
                              (2, "one in eight of every XCD's workgroups", 1 / 8)):
        ms = min(lib.store_rate_run(blocks, chunk_bytes, mode, ctypes.c_void_p(buf.data_ptr()))
                 for _ in range(reps))
        if ms < 0:
            raise RuntimeError(f"store probe failed ({ms})")
        nbytes = blocks * chunk_bytes * share
        out[name] = {"bytes": int(nbytes), "us": round(ms * 1e3, 2), "GB_per_s": round(nbytes / (ms / 1e3) / 1e9, 1)}
        print(f"[probe] stores, {name}: {nbytes / 2**20:.0f} MiB in {ms * 1e3:.1f} us", flush=True)
    return out


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def measure_slots(iters: int = 1000) -> dict:
    """Cycles per MFMA slot of one wave per SIMD with V other instructions
    after each MFMA (median over the waves)."""
    import torch
    lib = ctypes.CDLL(LIB)
    lib.slot_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.slot_run.restype = ctypes.c_int
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    cyc = torch.zeros(cu * 4, dtype=torch.int32, device="cuda")
    buf = torch.empty(cu * 256, dtype=torch.float32, device="cuda")
    names = {0: "v_and_b32 (SGPR mask)", 1: "v_lshlrev_b64", 2: "s_nop 1"}
    out = {}
    base = None
    for op, v in ((0, 0), (0, 1), (0, 2), (0, 3), (0, 4), (0, 8), (1, 1), (1, 2), (2, 1), (2, 2)):
        for _ in range(2):
            if lib.slot_run(op, v, cu, iters, ctypes.c_void_p(cyc.data_ptr()), ctypes.c_void_p(buf.data_ptr())) != 0:
                raise RuntimeError("slot probe failed")
        c = _median([x & 0xFFFFFFFF for x in cyc.cpu().tolist()]) / (16 * iters)
        if v == 0:
            base = c
        key = "none" if v == 0 else f"{names[op]} x{v}"
        out[key] = {"cycles_per_mfma_slot": round(c, 2), "extra_cycles": round(c - base, 2)}
        print(f"[probe] slots: {key}: {c:.2f} cycles per MFMA slot", flush=True)
    return out


def measure_copies(iters: int = 500) -> dict:
    """Cycles per MFMA of one wave per SIMD issuing copies between its MFMAs:
    (MFMAs per copy group, copies per group) x (all waves copy, wave 0 only)."""
    import torch
    lib = ctypes.CDLL(LIB)
    lib.copy_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                             ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.copy_run.restype = ctypes.c_int
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    n = 2 << 20
    src = torch.randint(-128, 128, (n + (128 << 10),), dtype=torch.int8, device="cuda")
    cyc = torch.zeros(cu * 4, dtype=torch.int32, device="cuda")
    buf = torch.empty(cu * 256, dtype=torch.float32, device="cuda")
    out = {}
    for _ in range(2):   # mode 0: no wave copies (the MFMA-only baseline)
        if lib.copy_run(8, 1, ctypes.c_void_p(src.data_ptr()), n - 1, 0, cu, iters,
                        ctypes.c_void_p(cyc.data_ptr()), ctypes.c_void_p(buf.data_ptr())) != 0:
            raise RuntimeError("copy probe failed")
    base = _median([x & 0xFFFFFFFF for x in cyc.cpu().tolist()]) / (32 * iters)
    out["no copies"] = {"cycles_per_mfma_wave0": round(base, 2), "copies_per_mfma": 0.0}
    print(f"[probe] copies: none: {base:.2f} cycles per MFMA", flush=True)
    for cpm, burst in ((16, 1), (8, 1), (4, 1), (2, 1), (8, 2), (16, 4), (32, 8)):
        for mode, who in ((1, "all waves"), (2, "wave 0 only")):
            for _ in range(2):
                if lib.copy_run(cpm, burst, ctypes.c_void_p(src.data_ptr()), n - 1, mode, cu, iters,
                                ctypes.c_void_p(cyc.data_ptr()), ctypes.c_void_p(buf.data_ptr())) != 0:
                    raise RuntimeError("copy probe failed")
            w = [x & 0xFFFFFFFF for x in cyc.cpu().tolist()]
            c0 = _median(w[0::4]) / (32 * iters)
            key = f"{burst} copies per {cpm} MFMAs, {who}"
            per_copy = (c0 - base) * cpm / burst
            out[key] = {"cycles_per_mfma_wave0": round(c0, 2), "copies_per_mfma": burst / cpm,
                        "cycles_per_copy": round(per_copy, 1)}
            print(f"[probe] copies: {key}: wave 0 {c0:.2f} cycles per MFMA, {per_copy:.1f} per copy", flush=True)
    return out


VALU_B1_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 2 * 64 / 1e12   # and + popcount-add per 32 bit-MACs


def valu_b1(A, B, C, reps: int = 1) -> float:
    """C = popcount(A AND B) over K bits on the vector ALUs (A: M x K/32, B: N x
    K/32 int32 tensors holding the bit words, C: M x N int32); milliseconds for
    `reps` launches."""
    lib = ctypes.CDLL(LIB)
    lib.valu_b1_run.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_int]
    lib.valu_b1_run.restype = ctypes.c_float
    M, kw = A.shape
    N = B.shape[0]
    ms = lib.valu_b1_run(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, 32 * kw, reps)
    if ms < 0:
        raise RuntimeError(f"valu_b1_run failed ({ms})")
    return ms


def measure_valu_b1(M: int = 4096, N: int = 4096, K: int = 8192) -> dict:
    """The vector-ALU popcount 1-bit GEMM against the library's 1-bit GEMM
    (automatic choice: the FP4 matrix-core route) on the same operands; the
    two results must be identical."""
    import torch
    import bit_integer_gemm_amd as lb
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    A = torch.randint(-2**31, 2**31 - 1, (M, K // 32), dtype=torch.int32, device="cuda", generator=g)
    B = torch.randint(-2**31, 2**31 - 1, (N, K // 32), dtype=torch.int32, device="cuda", generator=g)
    Cv = torch.empty((M, N), dtype=torch.int32, device="cuda")
    Cl = torch.empty_like(Cv)
    valu_b1(A, B, Cv)
    lb.lb_gemm_b1(A, B, Cl)
    torch.cuda.synchronize()
    if not torch.equal(Cv, Cl):
        raise RuntimeError("the vector-ALU 1-bit GEMM and the library disagree")
    ops = 2.0 * M * N * K
    reps = 20
    valu_b1(A, B, Cv, 3)
    t_valu = min(valu_b1(A, B, Cv, reps) for _ in range(3)) / reps * 1e-3
    for _ in range(10):
        lb.lb_gemm_b1(A, B, Cl)
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            lb.lb_gemm_b1(A, B, Cl)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps * 1e-3
        best = t if best is None else min(best, t)
    out = {"shape": [M, N, K], "valu_us": round(t_valu * 1e6, 2), "valu_tops": round(ops / t_valu / 1e12, 1),
           "valu_frac_of_valu_peak": round(ops / t_valu / 1e12 / VALU_B1_PEAK_TOPS, 3),
           "library_us": round(best * 1e6, 2), "library_tops": round(ops / best / 1e12, 1),
           "library_speedup": round(t_valu / best, 2), "identical": True}
    print(f"[probe] 1-bit on the vector ALUs: {out['valu_us']} us, {out['valu_tops']} TOP/s "
          f"({out['valu_frac_of_valu_peak']:.0%} of {VALU_B1_PEAK_TOPS:.1f}); library {out['library_us']} us "
          f"({out['library_speedup']}x)", flush=True)
    return out


def main():
    if not os.path.exists(LIB):
        sys.exit(f"{LIB} not built: run __graft_entry__.build() or bit_integer_gemm_amd.probe.build()")
    print(json.dumps({"mfma": measure(), "mix": measure_mix(), "stores": measure_stores(),
                      "slots": measure_slots(), "copies": measure_copies(), "valu_b1": measure_valu_b1()}))
