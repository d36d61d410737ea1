#!/usr/bin/env python3
"""Benchmark of the tiled GEMM C = act(A·B) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5a|c3|c2|c5b|c1|c4|mx1|mx2|mx3]
                    [--no-cpu-baseline] [--no-secondary] [--copy-calibration]

A step is one launch of the whole hot path (global->LDS tile copies, the
pipelined MFMA K loop and the fused epilogue) over one batch of seeded synthetic
inputs already resident in HBM.  The headline workload is the 8192^3 fp16 GEMM
(fp32 accumulate, fp16 out); the 4096^3 ReLU GEMM, the memory-bound skinny
16x16384x8192 case, the small 1024^3, 1000x1500x777 bf16 and 256^3 cases and the
8192^3 block-scaled MXFP8 GEMM are reported alongside in "secondary".  Operand sets are
rotated so that the inputs of consecutive launches are not the same buffers
(keeps the ~256 MB Infinity Cache from serving repeat reads).

Timing: W untimed launches, then exactly K launches between a barrier +
device synchronisation on both sides, bracketed by HIP events recorded on the
stream the kernels run on.  Rank 0 prints one JSON line.  The secondary
workloads warm up for at least 100 ms of launches besides (their kernels are
short, and the clock settles only after tens of milliseconds of load).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s (fp16, fp32 acc) and % of MFMA peak; skinny: HBM GB/s %"
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6,     # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
               "e4m3": 5033.2, "e5m2": 5033.2}    # FP8 (block-scaled): twice that
PEAK_HBM_GBS = 8000.0
# Sources of each kernel family, keyed by the plan's variant number (tlg.h).
KERNEL_SOURCES = {
    1: ["gemm_tile.hpp", "tlg_device.hpp"],
    2: ["gemm_tile.hpp", "tlg_device.hpp"],
    5: ["gemm_tile.hpp", "tlg_device.hpp"],
    3: ["gemm_skinny.hip", "gemm_lds.hpp", "tlg_device.hpp"],
    6: ["gemm_lds.hpp", "gemm_lds_f16.hip", "gemm_lds_bf16.hip", "tlg_device.hpp"],
    7: ["gemm_lds.hpp", "gemm_lds_f16.hip", "gemm_lds_bf16.hip", "tlg_device.hpp"],
    8: ["gemm_lds.hpp", "gemm_lds_f16.hip", "gemm_lds_bf16.hip", "tlg_device.hpp"],
    10: ["gemm_lds.hpp", "gemm_lds_f16.hip", "gemm_lds_bf16.hip", "tlg_device.hpp"],
    9: ["gemm_mx.hpp", "gemm_mx.hip", "gemm_lds.hpp", "tlg_device.hpp"],
    "attn": ["attn_fwd.hpp", "attn_fwd.hip", "gemm_lds.hpp", "tlg_device.hpp"],
    "w4": ["gemm_w4.hip", "gemm_lds.hpp", "tlg_device.hpp"],
    "sp": ["gemm_sp.hip", "gemm_lds.hpp", "tlg_device.hpp"],
}
ATTN_VARIANT = "attn"
W4_VARIANT = "w4"
SP_VARIANT = "sp"


def kernel_hash(variant: int) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[variant]:
        with open(os.path.join(ROOT, "tiled_dense_gemm_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_constant(name: str) -> int:
    """A launch constant of the kernels, read from their internal header (for labels)."""
    import re
    with open(os.path.join(ROOT, "tiled_dense_gemm_02_amd", "csrc", "tlg_internal.h")) as fh:
        m = re.search(rf"constexpr int {name} = (\d+);", fh.read())
    if not m:
        raise RuntimeError(f"{name} not found in tlg_internal.h")
    return int(m.group(1))


def stored_traffic(workload: str, variant: int):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_hash") != kernel_hash(variant):
        return None
    return rec.get("traffic_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # ~40 ms of launches: the clock settles only after tens of ms of MFMA load
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="c5a", help="c1..c5b, a block-scaled workload mx1..mx3, "
                    "an attention workload fa1..fa4, a dequant GEMM workload w4a..w4c, "
                    "or a 2:4 sparse GEMM workload sp1..sp3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also launch one 1 GiB device copy (FETCH/WRITE counter calibration)")
    return ap.parse_args()


def measure(case, steps, warmup, rotate_bytes=1 << 30, log=None, min_warm_ms=0.0):
    """Time `steps` launches of `case` after `warmup` untimed ones (and, with
    min_warm_ms > 0, after as many more as make up that much GPU time: the clock
    and power management settle only after tens of milliseconds of load, which a
    fixed count of a short kernel does not reach).  Returns a dict with the timing
    and the plan."""
    import torch
    import tiled_dense_gemm_02_amd as tlg
    import tlg_workloads as W

    dev = torch.device("cuda:0")
    A, B, _ = W.make_inputs(case)
    plan = tlg.Gemm(case.M, case.N, case.K, A.dtype, {"f16": torch.float16, "bf16": torch.bfloat16,
                                                        "f32": torch.float32}[case.c],
                    transpose_A=bool(case.transpose_A), transpose_B=bool(case.transpose_B),
                    epilogue="relu" if case.relu else "none")
    set_bytes = (A.numel() + B.numel()) * 2
    nsets = max(1, min(8, math.ceil(rotate_bytes / max(set_bytes, 1))))
    Ad = [A.to(dev) for _ in range(nsets)]
    Bd = [B.to(dev) for _ in range(nsets)]
    C = torch.empty((case.M, case.N), dtype=plan_out_dtype(case), device=dev)
    stream = torch.cuda.current_stream(dev)
    # One checked launch through the tensor interface, then the raw-pointer form (the
    # library's own argument checks still run on every call; the Python-side tensor
    # checks would otherwise cost as much as a small kernel).
    plan.run(Ad[0], Bd[0], C, stream)
    ptrs = [(Ad[i].data_ptr(), Bd[i].data_ptr()) for i in range(nsets)]
    c_ptr, sh = C.data_ptr(), stream.cuda_stream
    status = 0
    for i in range(warmup):
        status |= plan.run_ptrs(ptrs[i % nsets][0], ptrs[i % nsets][1], c_ptr, sh)
    torch.cuda.synchronize()
    if min_warm_ms > 0:
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        for i in range(20):
            status |= plan.run_ptrs(ptrs[i % nsets][0], ptrs[i % nsets][1], c_ptr, sh)
        w1.record(stream)
        torch.cuda.synchronize()
        per = max(w0.elapsed_time(w1) / 20, 1e-3)
        for i in range(int(math.ceil(max(0.0, min_warm_ms - 20 * per) / per))):
            status |= plan.run_ptrs(ptrs[i % nsets][0], ptrs[i % nsets][1], c_ptr, sh)
        torch.cuda.synchronize()
    if log:
        log(f"[bench] {case.name}: {plan.describe()} sets={nsets}")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        status |= plan.run_ptrs(ptrs[i % nsets][0], ptrs[i % nsets][1], c_ptr, sh)
    end.record(stream)
    torch.cuda.synchronize()
    if status != 0:
        raise RuntimeError(f"tlg_gemm_run failed during the timed launches (status {status})")
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    return {"ms": ms, "wall_s": wall, "plan": plan, "C": C, "A": A, "B": B, "nsets": nsets}


def measure_mx(case, steps, warmup, rotate_bytes=1 << 30, log=None, min_warm_ms=0.0):
    """measure() for a block-scaled FP8 workload (tlg_gemm_run_mx)."""
    import torch
    import tiled_dense_gemm_02_amd as tlg
    import tlg_workloads as W

    dev = torch.device("cuda:0")
    A, SA, B, SB, _ = W.make_mx_inputs(case)
    plan = tlg.Gemm(case.M, case.N, case.K, case.fmt, plan_out_dtype(case), transpose_B=True,
                    epilogue="relu" if case.relu else "none")
    nsets = max(1, min(8, math.ceil(rotate_bytes / max(A.numel() + B.numel(), 1))))
    sets = [(A.to(dev), SA.to(dev), B.to(dev), SB.to(dev)) for _ in range(nsets)]
    C = torch.empty((case.M, case.N), dtype=plan_out_dtype(case), device=dev)
    stream = torch.cuda.current_stream(dev)
    plan.run_mx(*sets[0][:2], *sets[0][2:], C, stream)
    ptrs = [tuple(t.data_ptr() for t in st) for st in sets]
    c_ptr, sh = C.data_ptr(), stream.cuda_stream
    status = 0

    def launch(i):
        a, sa, b, sb = ptrs[i % nsets]
        return plan.run_mx_ptrs(a, sa, b, sb, c_ptr, sh)

    for i in range(warmup):
        status |= launch(i)
    torch.cuda.synchronize()
    if min_warm_ms > 0:
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        for i in range(20):
            status |= launch(i)
        w1.record(stream)
        torch.cuda.synchronize()
        per = max(w0.elapsed_time(w1) / 20, 1e-3)
        for i in range(int(math.ceil(max(0.0, min_warm_ms - 20 * per) / per))):
            status |= launch(i)
        torch.cuda.synchronize()
    if log:
        log(f"[bench] {case.name}: {plan.describe()} sets={nsets}")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        status |= launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    if status != 0:
        raise RuntimeError(f"tlg_gemm_run_mx failed during the timed launches (status {status})")
    return {"ms": start.elapsed_time(end) / steps, "wall_s": time.perf_counter() - t0, "plan": plan, "C": C,
            "nsets": nsets}


def measure_attn(case, steps, warmup, rotate_bytes=1 << 30, log=None, min_warm_ms=0.0):
    """measure() for an attention-forward workload (tlg_attn_fwd)."""
    import torch
    import tiled_dense_gemm_02_amd as tlg
    import tlg_workloads as W

    dev = torch.device("cuda:0")
    q, k, v = W.make_attn_inputs(case)
    nsets = max(1, min(8, math.ceil(rotate_bytes / max(3 * q.numel() * 2, 1))))
    sets = [tuple(x.to(dev) for x in (q, k, v)) for _ in range(nsets)]
    O = torch.empty_like(sets[0][0])
    stream = torch.cuda.current_stream(dev)
    tlg.attention(*sets[0], O, causal=bool(case.causal), scale=case.scale, stream=stream)
    ptrs = [tuple(t.data_ptr() for t in st) for st in sets]
    o_ptr, sh = O.data_ptr(), stream.cuda_stream
    sc = case.softmax_scale
    status = 0

    def launch(i):
        qp, kp, vp = ptrs[i % nsets]
        return tlg.attention_ptrs(qp, kp, vp, o_ptr, case.B, case.S, case.H, case.D, q.dtype, case.causal, sc, sh)

    for i in range(warmup):
        status |= launch(i)
    torch.cuda.synchronize()
    if min_warm_ms > 0:
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        for i in range(20):
            status |= launch(i)
        w1.record(stream)
        torch.cuda.synchronize()
        per = max(w0.elapsed_time(w1) / 20, 1e-3)
        for i in range(int(math.ceil(max(0.0, min_warm_ms - 20 * per) / per))):
            status |= launch(i)
        torch.cuda.synchronize()
    if log:
        log(f"[bench] {case.name}: attention B={case.B} S={case.S} H={case.H} D={case.D} causal={case.causal} "
            f"sets={nsets}")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        status |= launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    if status != 0:
        raise RuntimeError(f"tlg_attn_fwd failed during the timed launches (status {status})")
    return {"ms": start.elapsed_time(end) / steps, "wall_s": time.perf_counter() - t0, "C": O, "nsets": nsets,
            "describe": f"attn_fwd block=128x64 threads=256 dim={case.D} causal={case.causal} dtype={case.dtype}"}


def measure_w4(case, steps, warmup, rotate_bytes=1 << 30, log=None, min_warm_ms=0.0):
    """measure() for a 4-bit dequant GEMM workload (tlg_gemm_w4)."""
    import torch
    import tiled_dense_gemm_02_amd as tlg
    import tlg_workloads as W

    dev = torch.device("cuda:0")
    A, Wq, S, Z, _ = W.make_w4_inputs(case)
    set_bytes = Wq.numel() + S.numel() * 2 + Z.numel() + A.numel() * 2
    nsets = max(1, min(16, math.ceil(rotate_bytes / max(set_bytes, 1))))
    sets = [tuple(t.to(dev) for t in (A, Wq, S, Z)) for _ in range(nsets)]
    C = torch.empty((case.M, case.N), dtype=plan_out_dtype(case), device=dev)
    stream = torch.cuda.current_stream(dev)
    tlg.gemm_w4(*sets[0], C, group=case.G, epilogue="relu" if case.relu else "none", stream=stream)
    ptrs = [tuple(t.data_ptr() for t in st) for st in sets]
    c_ptr, sh = C.data_ptr(), stream.cuda_stream
    status = 0

    def launch(i):
        a, w, sc, z = ptrs[i % nsets]
        return tlg.gemm_w4_ptrs(a, w, sc, z, c_ptr, case.M, case.N, case.K, case.G, A.dtype, C.dtype, case.relu, sh)

    for i in range(warmup):
        status |= launch(i)
    torch.cuda.synchronize()
    if min_warm_ms > 0:
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        for i in range(20):
            status |= launch(i)
        w1.record(stream)
        torch.cuda.synchronize()
        per = max(w0.elapsed_time(w1) / 20, 1e-3)
        for i in range(int(math.ceil(max(0.0, min_warm_ms - 20 * per) / per))):
            status |= launch(i)
        torch.cuda.synchronize()
    if log:
        log(f"[bench] {case.name}: w4 M={case.M} N={case.N} K={case.K} G={case.G} sets={nsets}")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        status |= launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    if status != 0:
        raise RuntimeError(f"tlg_gemm_w4 failed during the timed launches (status {status})")
    return {"ms": start.elapsed_time(end) / steps, "wall_s": time.perf_counter() - t0, "C": C, "nsets": nsets,
            "describe": f"gemm_w4 block=16x64x512 threads={kernel_constant('kW4Threads')} group={case.G} "
                        f"{case.ab}->{case.c}"}


def cpu_baseline_w4(case, C_gpu, rows):
    """cpu_baseline() for a dequant GEMM workload: the oracle on the first `rows` output rows."""
    import numpy as np
    import tlg_workloads as W
    from oracle import build_oracle, oracle as O
    if not os.path.exists(O.LIB_PATH):
        build_oracle.build()
    A, Wq, S, Z, _ = W.make_w4_inputs(case)
    t0 = time.perf_counter()
    o = O.w4gemm(case.M, case.N, case.K, case.G, W.bits16(A), Wq.numpy(), W.bits16(S), Z.numpy(), dtype=case.ab,
                 relu=case.relu, rows=(0, rows))
    dt = time.perf_counter() - t0
    sample_bytes = case.N * case.K // 2 + 3 * case.N * (case.K // case.G) + 2 * rows * case.K
    gpu = C_gpu[:rows].float().cpu().numpy().astype(np.float64)
    rel = 2.0 ** -8 if case.c == "bf16" else 2.0 ** -10
    wmax = 15.0 * float(S.float().abs().max())
    ok = bool((np.abs(gpu - o) <= rel * np.abs(o) + 1e-4 * np.sqrt(case.K) * wmax).all())
    return {"value": sample_bytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {rows} of {case.M} output rows of {case.name} (all weights dequantized once, "
                      f"{2.0 * rows * case.N * case.K / 1e9:.1f} GFLOP, fp64 loops, {dt:.1f} s)",
            "seconds": dt, "sample_matches_gpu": ok}


def bench_w4(args, case, log):
    """The JSON line of a dequant GEMM workload: HBM-bound (one read of the packed weights,
    scales, zero points and A, one write of C)."""
    r = measure_w4(case, args.steps, args.warmup, log=log, min_warm_ms=100.0)
    ms = r["ms"]
    gbs = case.algorithmic_bytes / (ms * 1e-3) / 1e9
    tflops = case.flops / (ms * 1e-3) / 1e12
    roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "traffic": stored_traffic(args.workload, W4_VARIANT), "kernel": "gemm_w4",
            "per_launch": {"flops": case.flops, "algorithmic_bytes": case.algorithmic_bytes, "avg_kernel_ms": ms}}
    out = {"metric": "dequant GEMM GB/s (4-bit weights, fp32 accumulate) and % of HBM peak", "value": gbs,
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": f"u4/{case.ab}",
           "data": "synthetic (seeded, see tlg_workloads.py)",
           "config": {"workload": f"{case.name}: {case.note}", "M": case.M, "N": case.N, "K": case.K,
                      "group": case.G, "ab_dtype": case.ab, "c_dtype": case.c, "plan": r["describe"],
                      "operand_sets_rotated": r["nsets"], "TFLOP/s": tflops},
           "roofline": roof}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_w4(case, r["C"], {"w4a": 16, "w4b": 5, "w4c": 8}[case.name])
    return out


def measure_sp(case, steps, warmup, rotate_bytes=1 << 30, log=None, min_warm_ms=0.0):
    """measure() for a 2:4 structured-sparse GEMM workload (tlg_gemm_sp)."""
    import torch
    import tiled_dense_gemm_02_amd as tlg
    import tlg_workloads as W

    dev = torch.device("cuda:0")
    A, Wv, Wm, _ = W.make_sp_inputs(case)
    set_bytes = A.numel() * 2 + Wv.numel() * 2 + Wm.numel()
    nsets = max(1, min(8, math.ceil(rotate_bytes / max(set_bytes, 1))))
    sets = [tuple(t.to(dev) for t in (A, Wv, Wm)) for _ in range(nsets)]
    C = torch.empty((case.M, case.N), dtype=plan_out_dtype(case), device=dev)
    stream = torch.cuda.current_stream(dev)
    tlg.gemm_sp(*sets[0], C, epilogue="relu" if case.relu else "none", stream=stream)
    ptrs = [tuple(t.data_ptr() for t in st) for st in sets]
    c_ptr, sh = C.data_ptr(), stream.cuda_stream
    status = 0

    def launch(i):
        a, wv, wm = ptrs[i % nsets]
        return tlg.gemm_sp_ptrs(a, wv, wm, c_ptr, case.M, case.N, case.K, A.dtype, C.dtype, case.relu, sh)

    for i in range(warmup):
        status |= launch(i)
    torch.cuda.synchronize()
    if min_warm_ms > 0:
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        for i in range(20):
            status |= launch(i)
        w1.record(stream)
        torch.cuda.synchronize()
        per = max(w0.elapsed_time(w1) / 20, 1e-3)
        for i in range(int(math.ceil(max(0.0, min_warm_ms - 20 * per) / per))):
            status |= launch(i)
        torch.cuda.synchronize()
    if log:
        log(f"[bench] {case.name}: sp M={case.M} N={case.N} K={case.K} sets={nsets}")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        status |= launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    if status != 0:
        raise RuntimeError(f"tlg_gemm_sp failed during the timed launches (status {status})")
    return {"ms": start.elapsed_time(end) / steps, "wall_s": time.perf_counter() - t0, "C": C, "nsets": nsets,
            "describe": f"gemm_sp block=256x256x64 threads=512 {case.ab}->{case.c}"}


def bench_sp(args, case, log):
    """The JSON line of a 2:4 sparse GEMM workload.  FLOPs count the stored (nonzero)
    weights only (M*N*K), priced against the dense MFMA peak of the operand dtype, which
    is the same fraction as the instruction's dense-equivalent rate against its own peak."""
    r = measure_sp(case, args.steps, args.warmup, log=log, min_warm_ms=100.0)
    ms = r["ms"]
    tflops = case.flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[case.ab]
    roof = {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s", "frac": tflops / peak,
            "traffic": stored_traffic(args.workload, SP_VARIANT), "kernel": "gemm_sp",
            "per_launch": {"flops": case.flops, "algorithmic_bytes": case.algorithmic_bytes, "avg_kernel_ms": ms}}
    out = {"metric": "2:4 sparse GEMM TFLOP/s of stored-weight multiply-adds (fp32 accumulate) and % of dense MFMA peak",
           "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": case.ab,
           "data": "synthetic (seeded, see tlg_workloads.py)",
           "config": {"workload": f"{case.name}: {case.note}", "M": case.M, "N": case.N, "K": case.K,
                      "ab_dtype": case.ab, "c_dtype": case.c, "plan": r["describe"],
                      "operand_sets_rotated": r["nsets"], "dense_equivalent_TFLOP/s": 2 * tflops},
           "roofline": roof}
    if not args.no_cpu_baseline:
        import numpy as np
        import tlg_workloads as W
        from oracle import build_oracle, oracle as O
        if not os.path.exists(O.LIB_PATH):
            build_oracle.build()
        rows = {"sp1": 256, "sp2": 1000, "sp3": 64}[case.name]
        A, Wv, Wm, _ = W.make_sp_inputs(case)
        t0 = time.perf_counter()
        o = O.spgemm(case.M, case.N, case.K, W.bits16(A), W.bits16(Wv), Wm.numpy(), dtype=case.ab, relu=case.relu,
                     rows=(0, rows))
        dt = time.perf_counter() - t0
        gpu = r["C"][:rows].float().cpu().numpy().astype(np.float64)
        ok = bool((np.abs(gpu - o) <= O.tolerance(o, case.K, case.c)).all())
        flops = float(rows) * case.N * case.K
        out["cpu_baseline"] = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {rows} of {case.M} output rows of {case.name} "
                                         f"({flops / 1e9:.1f} GFLOP of stored-weight multiply-adds, fp64 loops, {dt:.1f} s)",
                               "seconds": dt, "sample_matches_gpu": ok}
    return out


def plan_out_dtype(case):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[case.c]


def cpu_baseline(case, C_gpu, rows):
    """Time the oracle (as it stands) on the first `rows` output rows; check those rows
    against the GPU output as a side effect."""
    import numpy as np
    import tlg_workloads as W
    from oracle import build_oracle, oracle as O
    if not os.path.exists(O.LIB_PATH):
        build_oracle.build()
    A, B, _ = W.make_inputs(case)
    nthreads = min(os.cpu_count() or 1, 16)
    t0 = time.perf_counter()
    o = O.gemm(case.M, case.N, case.K, W.bits16(A), W.bits16(B), ab=case.ab, c=case.c,
               transpose_A=case.transpose_A, transpose_B=case.transpose_B, relu=case.relu,
               rows=(0, rows), nthreads=nthreads)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * case.N * case.K
    gpu = C_gpu[:rows].float().cpu().numpy().astype(np.float64)
    tol = O.tolerance(o, case.K, case.c)
    ok = bool((np.abs(gpu - o) <= tol).all())
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": f"first {rows} of {case.M} output rows of {case.name} "
                      f"({flops / 1e9:.1f} GFLOP, fp64 triple loop, {dt:.1f} s)",
            "seconds": dt, "sample_matches_gpu": ok}


def cpu_baseline_mx(case, C_gpu, rows):
    """cpu_baseline() for a block-scaled FP8 workload (the MX oracle)."""
    import numpy as np
    import tlg_workloads as W
    from oracle import build_oracle, oracle as O
    if not os.path.exists(O.LIB_PATH):
        build_oracle.build()
    A, SA, B, SB, _ = W.make_mx_inputs(case)
    nthreads = min(os.cpu_count() or 1, 16)
    t0 = time.perf_counter()
    o = O.mxgemm(case.M, case.N, case.K, A.numpy(), SA.numpy(), B.numpy(), SB.numpy(), fmt_a=case.fmt,
                 fmt_b=case.fmt, c=case.c, relu=case.relu, rows=(0, rows), nthreads=nthreads)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * case.N * case.K
    gpu = C_gpu[:rows].float().cpu().numpy().astype(np.float64)
    ok = bool((np.abs(gpu - o) <= O.tolerance(o, case.K, case.c)).all())
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": f"first {rows} of {case.M} output rows of {case.name} "
                      f"({flops / 1e9:.1f} GFLOP, fp64 triple loop, {dt:.1f} s)",
            "seconds": dt, "sample_matches_gpu": ok}


def cpu_baseline_attn(case, O_gpu, positions):
    """cpu_baseline() for an attention workload: the attention oracle on the last
    `positions` query positions of every (batch, head)."""
    import numpy as np
    import tlg_workloads as W
    from oracle import build_oracle, oracle as O
    if not os.path.exists(O.LIB_PATH):
        build_oracle.build()
    q, k, v = W.make_attn_inputs(case)
    nthreads = min(os.cpu_count() or 1, 16)
    i0 = case.S - positions
    t0 = time.perf_counter()
    o = O.attn(case.B, case.S, case.H, case.D, W.bits16(q), W.bits16(k), W.bits16(v), dtype=case.dtype,
               causal=case.causal, scale=case.softmax_scale, rows=(i0, case.S), nthreads=nthreads)
    dt = time.perf_counter() - t0
    keys = sum(i + 1 for i in range(i0, case.S)) if case.causal else positions * case.S
    flops = 4.0 * case.D * keys * case.B * case.H
    gpu = O_gpu[:, i0:].float().cpu().numpy().astype(np.float64)
    ok = bool((np.abs(gpu - o) <= O.attn_tolerance(o, float(v.float().abs().max()), case.dtype)).all())
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": f"last {positions} of {case.S} query positions of every batch and head of {case.name} "
                      f"({flops / 1e9:.1f} GFLOP, fp64 loops, {dt:.1f} s)",
            "seconds": dt, "sample_matches_gpu": ok}


def bench_attn(args, case, log):
    """The JSON line of an attention-forward workload (MFMA-bound: both products run on
    the matrix cores; the algorithmic work is 4 * dim FLOPs per allowed query-key pair)."""
    r = measure_attn(case, args.steps, args.warmup, log=log, min_warm_ms=100.0)
    ms = r["ms"]
    tflops = case.flops / (ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": tflops, "peak": PEAK_TFLOPS[case.dtype], "unit": "TFLOP/s",
            "frac": tflops / PEAK_TFLOPS[case.dtype], "traffic": stored_traffic(args.workload, ATTN_VARIANT),
            "kernel": "attn_fwd", "per_launch": {"flops": case.flops, "algorithmic_bytes": case.algorithmic_bytes,
                                                 "avg_kernel_ms": ms}}
    out = {"metric": "attention forward TFLOP/s (fp16, fp32 accumulate) and % of MFMA peak", "value": tflops,
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": case.dtype,
           "data": "synthetic (seeded, see tlg_workloads.py)",
           "config": {"workload": f"{case.name}: {case.note}", "batch": case.B, "seq": case.S, "heads": case.H,
                      "dim": case.D, "causal": case.causal, "plan": r["describe"], "operand_sets_rotated": r["nsets"]},
           "roofline": roof}
    if not args.no_cpu_baseline:
        positions = {"fa1": 1024, "fa2": 777, "fa3": 32, "fa4": 64}[case.name]
        out["cpu_baseline"] = cpu_baseline_attn(case, r["C"], positions)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              f"the sharding across GPUs is not built", file=sys.stderr)
        sys.exit(2)
    import torch
    import tlg_workloads as W

    def log(m):
        print(m, file=sys.stderr, flush=True)

    if args.copy_calibration:
        x = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")   # 1 GiB
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 1 GiB read + 1 GiB write done")
        del x, y

    if args.workload in W.SP_CONFIGS:
        print(json.dumps(bench_sp(args, W.SP_CONFIGS[args.workload], log)), flush=True)
        return
    if args.workload in W.W4_CONFIGS:
        print(json.dumps(bench_w4(args, W.W4_CONFIGS[args.workload], log)), flush=True)
        return
    if args.workload in W.ATTN_CONFIGS:
        print(json.dumps(bench_attn(args, W.ATTN_CONFIGS[args.workload], log)), flush=True)
        return
    is_mx = args.workload in W.MX_CONFIGS
    case = W.MX_CONFIGS[args.workload] if is_mx else W.CONFIGS[args.workload]
    r = (measure_mx if is_mx else measure)(case, args.steps, args.warmup, log=log)
    plan = r["plan"]
    info = plan.info
    kind = "skinny" if info.variant == 3 else "tile"   # HBM-bound vs MFMA-bound kernel
    ab = case.fmt if is_mx else case.ab
    ms = r["ms"]
    tflops = case.flops / (ms * 1e-3) / 1e12
    gbs = case.algorithmic_bytes / (ms * 1e-3) / 1e9
    if kind == "skinny":
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS}
        value, unit = gbs, "GB/s"
    else:
        roof = {"bound": "mfma", "achieved": tflops, "peak": PEAK_TFLOPS[ab], "unit": "TFLOP/s",
                "frac": tflops / PEAK_TFLOPS[ab]}
        value, unit = tflops, "TFLOP/s"
    roof["traffic"] = stored_traffic(args.workload, info.variant)
    roof["kernel"] = plan.describe().split()[0]
    roof["per_launch"] = {"flops": case.flops, "algorithmic_bytes": case.algorithmic_bytes,
                          "avg_kernel_ms": ms}

    out = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": ab, "data": "synthetic (seeded, see tlg_workloads.py)",
           "config": {"workload": f"{case.name}: {case.note}", "M": case.M, "N": case.N, "K": case.K,
                      "ab_dtype": ab, "c_dtype": case.c, "transpose_A": 0 if is_mx else case.transpose_A,
                      "transpose_B": 1 if is_mx else case.transpose_B, "epilogue": "relu" if case.relu else "none",
                      "plan": plan.describe(), "operand_sets_rotated": r["nsets"]},
           "roofline": roof}

    if not args.no_secondary:
        sec = []
        for name in ("c3", "c5b", "c2", "c4", "c1", "mx3", "fa3", "w4a", "sp3"):
            if name == args.workload:
                continue
            sec_mx, sec_attn, sec_w4 = name in W.MX_CONFIGS, name in W.ATTN_CONFIGS, name in W.W4_CONFIGS
            sec_sp = name in W.SP_CONFIGS
            c2 = (W.MX_CONFIGS[name] if sec_mx else W.ATTN_CONFIGS[name] if sec_attn else
                  W.W4_CONFIGS[name] if sec_w4 else W.SP_CONFIGS[name] if sec_sp else W.CONFIGS[name])
            fn = (measure_mx if sec_mx else measure_attn if sec_attn else measure_w4 if sec_w4 else
                  measure_sp if sec_sp else measure)
            rr = fn(c2, max(10, args.steps // 2), 40, log=log, min_warm_ms=100.0)
            t = rr["ms"] * 1e-3
            entry = {"workload": name, "ms": rr["ms"], "TFLOP/s": c2.flops / t / 1e12,
                     "GB/s": c2.algorithmic_bytes / t / 1e9,
                     "plan": rr["describe"] if (sec_attn or sec_w4 or sec_sp) else rr["plan"].describe()}
            entry["mfma_frac"] = entry["TFLOP/s"] / PEAK_TFLOPS[c2.fmt if sec_mx else c2.dtype if sec_attn else c2.ab]
            entry["hbm_frac"] = entry["GB/s"] / PEAK_HBM_GBS
            sec.append(entry)
            del rr
        out["secondary"] = sec

    if not args.no_cpu_baseline:
        # a bounded sample (~10 s of the oracle on 16 host threads)
        rows = {"c5a": 4096, "c3": 4096, "c2": 1024, "c1": 256, "c4": 1000, "c5b": 16, "mx1": 256, "mx2": 1000,
                "mx3": 2048}[args.workload]
        cb = (cpu_baseline_mx if is_mx else cpu_baseline)(case, r["C"], rows)
        out["cpu_baseline"] = cb
        if unit == "GB/s":
            cb["value_gbs"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
