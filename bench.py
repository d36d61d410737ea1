#!/usr/bin/env python3
"""Benchmark of the tiled GEMM C = act(A·B) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-secondary] [--copy-calibration]

A step is one launch of the whole hot path (global->LDS tile copies, the
pipelined MFMA K loop and the fused epilogue) over one batch of seeded synthetic
inputs already resident in HBM.  The headline workload is the 8192^3 fp16 GEMM
(fp32 accumulate, fp16 out); the 4096^3 ReLU GEMM, the memory-bound skinny
16x16384x8192 case, the small 1024^3, 1000x1500x777 bf16 and 256^3 cases, and one
configuration each of the block-scaled, attention, dequant and sparse kernels are
reported alongside in "secondary".  Operand sets are rotated so that consecutive
launches do not read the same buffers (keeps the ~256 MB Infinity Cache from
serving repeat reads).

Timing, the same rule for every workload: W untimed launches, then more until at
least 100 ms of GPU time has passed (power management and the shader clock settle
only after tens of milliseconds of load), then exactly K launches between device
synchronisations, with a HIP event recorded on the launch stream before every
launch and after the last one.  The mean is the headline; min / median / p90
come from a second pass in which each launch has its own pair of events.  For the
three target workloads the shader clock and socket power are sampled from a
thread of this process through the amdsmi library (started before the first GPU
call), over 3 s of further launches of the same workload right after the
timed ones (the driver refreshes the readings about once a second).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s (fp16, fp32 acc) and % of MFMA peak; skinny: HBM GB/s %"
# Dense peaks of MI355X (AMD's published figures, no sparsity).
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6,     # 256 CU x 4096 FLOP/clk x 2.4 GHz
               "e4m3": 5033.2, "e5m2": 5033.2,    # FP8: twice that
               "e2m1": 10066.3}                   # FP4: four times
FLOP_PER_CLK_CU = {"f16": 4096, "bf16": 4096, "e4m3": 8192, "e5m2": 8192, "e2m1": 16384}
PEAK_HBM_GBS = 8000.0
WARM_MS = 100.0
# The metrics table refreshes about once a second, so the clock window spans
# 3 s of launches (about three fresh readings); it is taken for the three target
# workloads only.
CLOCK_MS = 3000.0
CLOCK_WORKLOADS = ("c5a", "c3", "c5b")
WARM_RULE = (f"W untimed launches, then more until >= {WARM_MS:.0f} ms of GPU time, then K timed launches "
             "between two HIP events on the launch stream (the mean); then K launches each between its own "
             f"event pair (min/median/p90); then {CLOCK_MS:.0f} ms more launches while the clock is sampled "
             f"(workloads {', '.join(CLOCK_WORKLOADS)}); secondary workloads time max(K/2, 10) launches or "
             "at least 20 ms of them")
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
    13: ["gemm_lds.hpp", "gemm_lds32.hip", "tlg_device.hpp"],
    9: ["gemm_mx.hpp", "gemm_mx.hip", "gemm_lds.hpp", "tlg_device.hpp"],
    "attn": ["attn_fwd.hpp", "attn_fwd.hip", "gemm_lds.hpp", "tlg_device.hpp"],
    "w4": ["gemm_w4.hip", "gemm_lds.hpp", "tlg_device.hpp"],
    "sp": ["gemm_sp.hip", "gemm_lds.hpp", "tlg_device.hpp"],
}
ATTN_VARIANT = "attn"
W4_VARIANT = "w4"
SP_VARIANT = "sp"


def _code_only(text: str) -> str:
    """A C/C++ source without its comments and blank lines, so that the hash below
    follows the code and not the wording of its comments (no kernel source has a
    comment marker inside a string literal)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_hash(variant) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[variant]:
        with open(os.path.join(ROOT, "tiled_dense_gemm_02_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def kernel_constant(name: str) -> int:
    """A launch constant of the kernels, read from their internal header (for labels)."""
    import re
    with open(os.path.join(ROOT, "tiled_dense_gemm_02_amd", "csrc", "tlg_internal.h")) as fh:
        m = re.search(rf"constexpr int {name} = (\d+);", fh.read())
    if not m:
        raise RuntimeError(f"{name} not found in tlg_internal.h")
    return int(m.group(1))


def stored_traffic(workload: str, variant):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_hash") != kernel_hash(variant):
        return None
    return rec.get("traffic_bytes_per_launch")


# ---------------------------------------------------------------------------- clock, device, host
class ClockSampler:
    """Shader clock and socket power of the GPU, sampled every few milliseconds from a
    thread of this process through the amdsmi library (the driver's gpu_metrics table).
    Started before the first GPU call; no child process."""

    def __init__(self, period_s: float = 0.004):
        self.samples = []          # (perf_counter time, mean shader clock over the XCDs in MHz, socket W)
        self.error = None
        self.bdfs = []
        self._handles = []
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            self._smi = amdsmi
            self._handles = amdsmi.amdsmi_get_processor_handles()
            if not self._handles:
                raise RuntimeError("amdsmi found no GPU")
            self.bdfs = [amdsmi.amdsmi_get_gpu_device_bdf(h) for h in self._handles]
            self._h = self._handles[0]
            self._period = period_s
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        except Exception as e:   # no amdsmi, no permission: the clock fields stay null
            self.error = f"{type(e).__name__}: {e}"

    def select(self, bdf: str):
        """Sample the GPU with this PCI address (the HIP device the bench runs on)."""
        for h, b in zip(self._handles, self.bdfs):
            if str(b).lower() == bdf.lower():
                self._h = h

    def _one(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0]
        clk = sum(clks) / len(clks) if clks else m.get("current_gfxclk")
        pw = m.get("current_socket_power")
        return (m.get("firmware_timestamp"), clk if isinstance(clk, (int, float)) else None,
                pw if isinstance(pw, (int, float)) else None)

    def _run(self):
        # The driver refreshes the metrics table about once a second (measured on
        # MI355X): only samples with a new firmware timestamp are kept.
        last = None
        while not self._stop.is_set():
            try:
                stamp, clk, pw = self._one()
                if stamp != last:
                    last = stamp
                    self.samples.append((time.perf_counter(), clk, pw))
            except Exception as e:
                self.error = f"{type(e).__name__}: {e}"
                return
            time.sleep(self._period)

    def max_sclk_mhz(self):
        try:
            info = self._smi.amdsmi_get_clock_info(self._h, self._smi.AmdSmiClkType.GFX)
            return info.get("max_clk")
        except Exception:
            return None

    def window(self, t0: float, t1: float):
        """Mean (and range) of the samples taken between t0 and t1."""
        s = [x for x in self.samples if t0 <= x[0] <= t1]
        clk = [x[1] for x in s if x[1] is not None]
        pw = [x[2] for x in s if x[2] is not None]
        if not clk:
            return {"samples": len(s), "sclk_mhz": None, "error": self.error}
        return {"samples": len(s), "sclk_mhz": sum(clk) / len(clk), "sclk_mhz_min": min(clk),
                "sclk_mhz_max": max(clk), "socket_w": (sum(pw) / len(pw)) if pw else None,
                "socket_w_max": max(pw) if pw else None}

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=1.0)


def host_facts():
    """Versions and host CPU, read from files (no child process, no GPU call)."""
    facts = {"python": sys.version.split()[0]}
    try:
        facts["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        facts["rocm"] = None
    try:
        v = {}
        for line in open("/opt/rocm/share/hip/version"):
            if "=" in line and not line.startswith("#"):
                k, x = line.strip().split("=", 1)
                v[k] = x
        facts["hip"] = (f"{v['HIP_VERSION_MAJOR']}.{v['HIP_VERSION_MINOR']}.{v['HIP_VERSION_PATCH']}-"
                        f"{v['HIP_VERSION_GITHASH']}")
    except (OSError, KeyError):
        facts["hip"] = None
    try:
        facts["clang_major"] = sorted(os.listdir("/opt/rocm/lib/llvm/lib/clang"))[-1]
    except OSError:
        facts["clang_major"] = None
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    facts["cpu_model"] = model
    facts["nproc"] = os.cpu_count()
    facts["cpu_affinity"] = len(os.sched_getaffinity(0))
    facts["omp_num_threads"] = os.environ.get("OMP_NUM_THREADS")
    return facts


def cpu_threads() -> int:
    """Host threads for the CPU baseline: every core this process may run on, capped by
    OMP_NUM_THREADS when the machine sets it (the host's share per GPU)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def device_facts(sampler: ClockSampler):
    import ctypes
    import torch
    props = torch.cuda.get_device_properties(0)
    facts = {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
             "hbm_gib": round(props.total_memory / 2 ** 30, 1), "hip_runtime": torch.version.hip,
             "torch": torch.__version__}
    bdf = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}.0"
    facts["pci"] = bdf
    sampler.select(bdf)
    try:
        # hipDeviceGetAttribute(&v, hipDeviceAttributeClockRate, 0): the peak shader clock in kHz
        # (hipDeviceAttributeClockRate is entry 5 of hipDeviceAttribute_t in hip_runtime_api.h).
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:
            facts["max_sclk_mhz"] = v.value / 1000.0
    except OSError:
        pass
    facts["max_sclk_mhz_smi"] = sampler.max_sclk_mhz()
    facts["clock_sampler_error"] = sampler.error
    return facts


# ---------------------------------------------------------------------------- timing
def timed_launches(launch, stream, steps, warmup, sampler=None, sample_clock=True, min_timed_ms=0.0):
    """The one timing rule (see the module docstring).  launch(i) enqueues launch i and
    returns its status.

    1. warm-up: `warmup` launches, then more until WARM_MS of GPU time;
    2. the timed run: `steps` launches between two HIP events on the launch stream
       (the headline mean);
    3. the per-launch distribution: the same number of launches again, each between its
       own pair of events (min / median / p90; an event pair adds a few microseconds,
       which matters only for the smallest kernels);
    4. the clock: launches go on for CLOCK_MS more while the sampler reads the shader
       clock and socket power (the driver's metrics table refreshes too slowly for the
       few milliseconds of a short timed run); the samples of the timed run itself are
       reported beside them."""
    import torch
    warm_ms = WARM_MS
    status = 0
    for i in range(warmup):
        status |= launch(i)
    torch.cuda.synchronize()
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for i in range(20):
        status |= launch(i)
    w1.record(stream)
    torch.cuda.synchronize()
    per = max(w0.elapsed_time(w1) / 20, 1e-3)
    for i in range(int(math.ceil(max(0.0, warm_ms - 20 * per) / per))):
        status |= launch(i)
    if min_timed_ms > 0:      # secondary workloads: at least this much timed GPU work
        steps = max(steps, int(math.ceil(min_timed_ms / per)))
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        status |= launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # per-launch distribution
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        status |= launch(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    # clock window
    clock = None
    if sample_clock and sampler is not None and sampler.error is None and CLOCK_MS > 0:
        n = int(math.ceil(CLOCK_MS / per))
        c0 = time.perf_counter()
        for i in range(n):
            status |= launch(i)
            if i % 64 == 63:
                torch.cuda.synchronize()   # keep the queue short so the window is the launches' own
        torch.cuda.synchronize()
        c1 = time.perf_counter()
        clock = sampler.window(c0, c1)
        clock["window_ms"] = (c1 - c0) * 1e3
        # The timed run itself is not sampled: it is shorter than the ~1 s refresh of the
        # driver's metrics, so a reading taken during it describes the time before it.
    if status != 0:
        raise RuntimeError(f"a launch failed during the timed run (status {status})")
    each = sorted(a.elapsed_time(b) for a, b in evs)

    def q(f):
        return each[min(len(each) - 1, int(f * (len(each) - 1) + 0.5))]

    mean = start.elapsed_time(end) / steps
    r = {"ms": mean, "wall_s": t1 - t0, "steps": steps,
         "per_launch_ms": {"mean": mean, "min": each[0], "median": q(0.5), "p90": q(0.9), "max": each[-1]}}
    if sampler is not None:
        r["clock"] = clock if clock is not None else {"sclk_mhz": None, "error": sampler.error,
                                                      "note": None if sampler.error else "not sampled"}
    return r


def _rotation(set_bytes, rotate_bytes=1 << 30, cap=8):
    return max(1, min(cap, math.ceil(rotate_bytes / max(set_bytes, 1))))


def plan_out_dtype(case):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[case.c]


def measure(case, steps, warmup, sampler=None, log=None, variant="auto", min_timed_ms=0.0):
    """Time the 16-bit GEMM of `case` through a plan (tlg_gemm_create / tlg_gemm_run)."""
    import torch
    import tiled_dense_gemm_02_amd as tlg
    import tlg_workloads as W

    dev = torch.device("cuda:0")
    A, B, _ = W.make_inputs(case)
    plan = tlg.Gemm(case.M, case.N, case.K, A.dtype, plan_out_dtype(case), transpose_A=bool(case.transpose_A),
                    transpose_B=bool(case.transpose_B), epilogue="relu" if case.relu else "none", variant=variant)
    nsets = _rotation((A.numel() + B.numel()) * 2)
    Ad = [A.to(dev) for _ in range(nsets)]
    Bd = [B.to(dev) for _ in range(nsets)]
    C = torch.empty((case.M, case.N), dtype=plan_out_dtype(case), device=dev)
    stream = torch.cuda.current_stream(dev)
    # One checked launch through the tensor interface, then the raw-pointer form (the
    # library's own argument checks still run on every call).
    plan.run(Ad[0], Bd[0], C, stream)
    ptrs = [(Ad[i].data_ptr(), Bd[i].data_ptr()) for i in range(nsets)]
    c_ptr, sh = C.data_ptr(), stream.cuda_stream
    if log:
        log(f"[bench] {case.name}: {plan.describe()} sets={nsets}")
    r = timed_launches(lambda i: plan.run_ptrs(ptrs[i % nsets][0], ptrs[i % nsets][1], c_ptr, sh), stream, steps,
                       warmup, sampler, sample_clock=case.name in CLOCK_WORKLOADS,
                       min_timed_ms=min_timed_ms)
    r.update({"plan": plan, "describe": plan.describe(), "C": C, "nsets": nsets})
    return r


def measure_mx(case, steps, warmup, sampler=None, log=None, min_timed_ms=0.0):
    """Time a block-scaled workload (tlg_gemm_run_mx)."""
    import torch
    import tiled_dense_gemm_02_amd as tlg
    import tlg_workloads as W

    dev = torch.device("cuda:0")
    A, SA, B, SB, _ = W.make_mx_inputs(case)
    plan = tlg.Gemm(case.M, case.N, case.K, case.fmt, plan_out_dtype(case), transpose_B=True,
                    epilogue="relu" if case.relu else "none")
    nsets = _rotation(A.numel() + B.numel())
    sets = [(A.to(dev), SA.to(dev), B.to(dev), SB.to(dev)) for _ in range(nsets)]
    C = torch.empty((case.M, case.N), dtype=plan_out_dtype(case), device=dev)
    stream = torch.cuda.current_stream(dev)
    plan.run_mx(*sets[0][:2], *sets[0][2:], C, stream)
    ptrs = [tuple(t.data_ptr() for t in st) for st in sets]
    c_ptr, sh = C.data_ptr(), stream.cuda_stream

    def launch(i):
        a, sa, b, sb = ptrs[i % nsets]
        return plan.run_mx_ptrs(a, sa, b, sb, c_ptr, sh)

    if log:
        log(f"[bench] {case.name}: {plan.describe()} sets={nsets}")
    r = timed_launches(launch, stream, steps, warmup, sampler, sample_clock=False, min_timed_ms=min_timed_ms)
    r.update({"plan": plan, "describe": plan.describe(), "C": C, "nsets": nsets})
    return r


def measure_attn(case, steps, warmup, sampler=None, log=None, min_timed_ms=0.0):
    """Time an attention-forward workload (tlg_attn_fwd)."""
    import torch
    import tiled_dense_gemm_02_amd as tlg
    import tlg_workloads as W

    dev = torch.device("cuda:0")
    q, k, v = W.make_attn_inputs(case)
    nsets = _rotation(3 * q.numel() * 2)
    sets = [tuple(x.to(dev) for x in (q, k, v)) for _ in range(nsets)]
    O = torch.empty_like(sets[0][0])
    stream = torch.cuda.current_stream(dev)
    tlg.attention(*sets[0], O, causal=bool(case.causal), scale=case.scale, stream=stream)
    ptrs = [tuple(t.data_ptr() for t in st) for st in sets]
    o_ptr, sh = O.data_ptr(), stream.cuda_stream
    sc = case.softmax_scale

    def launch(i):
        qp, kp, vp = ptrs[i % nsets]
        return tlg.attention_ptrs(qp, kp, vp, o_ptr, case.B, case.S, case.H, case.D, q.dtype, case.causal, sc, sh)

    if log:
        log(f"[bench] {case.name}: attention B={case.B} S={case.S} H={case.H} D={case.D} causal={case.causal} "
            f"sets={nsets}")
    r = timed_launches(launch, stream, steps, warmup, sampler, sample_clock=False, min_timed_ms=min_timed_ms)
    r.update({"C": O, "nsets": nsets,
              "describe": f"attn_fwd block={tlg.attention_query_block(case.B, case.S, case.H, case.D, case.causal)}x64 threads=256 "
                          f"dim={case.D} causal={case.causal} dtype={case.dtype}"})
    return r


def measure_w4(case, steps, warmup, sampler=None, log=None, min_timed_ms=0.0):
    """Time a 4-bit dequant GEMM workload (tlg_gemm_w4)."""
    import torch
    import tiled_dense_gemm_02_amd as tlg
    import tlg_workloads as W

    dev = torch.device("cuda:0")
    A, Wq, S, Z, _ = W.make_w4_inputs(case)
    nsets = _rotation(Wq.numel() + S.numel() * 2 + Z.numel() + A.numel() * 2, cap=16)
    sets = [tuple(t.to(dev) for t in (A, Wq, S, Z)) for _ in range(nsets)]
    C = torch.empty((case.M, case.N), dtype=plan_out_dtype(case), device=dev)
    stream = torch.cuda.current_stream(dev)
    tlg.gemm_w4(*sets[0], C, group=case.G, epilogue="relu" if case.relu else "none", stream=stream)
    ptrs = [tuple(t.data_ptr() for t in st) for st in sets]
    c_ptr, sh = C.data_ptr(), stream.cuda_stream

    def launch(i):
        a, w, sc, z = ptrs[i % nsets]
        return tlg.gemm_w4_ptrs(a, w, sc, z, c_ptr, case.M, case.N, case.K, case.G, A.dtype, C.dtype, case.relu, sh)

    if log:
        log(f"[bench] {case.name}: w4 M={case.M} N={case.N} K={case.K} G={case.G} sets={nsets}")
    r = timed_launches(launch, stream, steps, warmup, sampler, sample_clock=False, min_timed_ms=min_timed_ms)
    r.update({"C": C, "nsets": nsets,
              "describe": f"gemm_w4 block=16x64x512 threads={kernel_constant('kW4Threads')} group={case.G} "
                          f"{case.ab}->{case.c}"})
    return r


def measure_sp(case, steps, warmup, sampler=None, log=None, min_timed_ms=0.0):
    """Time a 2:4 structured-sparse GEMM workload (tlg_gemm_sp)."""
    import torch
    import tiled_dense_gemm_02_amd as tlg
    import tlg_workloads as W

    dev = torch.device("cuda:0")
    A, Wv, Wm, _ = W.make_sp_inputs(case)
    nsets = _rotation(A.numel() * 2 + Wv.numel() * 2 + Wm.numel())
    sets = [tuple(t.to(dev) for t in (A, Wv, Wm)) for _ in range(nsets)]
    C = torch.empty((case.M, case.N), dtype=plan_out_dtype(case), device=dev)
    stream = torch.cuda.current_stream(dev)
    tlg.gemm_sp(*sets[0], C, epilogue="relu" if case.relu else "none", stream=stream)
    ptrs = [tuple(t.data_ptr() for t in st) for st in sets]
    c_ptr, sh = C.data_ptr(), stream.cuda_stream

    def launch(i):
        a, wv, wm = ptrs[i % nsets]
        return tlg.gemm_sp_ptrs(a, wv, wm, c_ptr, case.M, case.N, case.K, A.dtype, C.dtype, case.relu, sh)

    if log:
        log(f"[bench] {case.name}: sp M={case.M} N={case.N} K={case.K} sets={nsets}")
    r = timed_launches(launch, stream, steps, warmup, sampler, sample_clock=False, min_timed_ms=min_timed_ms)
    r.update({"C": C, "nsets": nsets, "describe": f"gemm_sp block=256x256x64 threads=512 {case.ab}->{case.c}"})
    return r


# ---------------------------------------------------------------------------- the oracle, timed
def _oracle():
    from oracle import build_oracle, oracle as O
    if not os.path.exists(O.LIB_PATH):
        build_oracle.build()
    return O


def _cpu_record(value, unit, nthreads, sample, dt, ok):
    return {"value": value, "unit": unit, "cores": nthreads, "kind": "oracle", "sample": sample, "seconds": dt,
            "sample_matches_gpu": ok}


def cpu_baseline(case, C_gpu, rows):
    """Time the oracle (as it stands) on the first `rows` output rows on the host's
    threads; check those rows against the GPU output as a side effect."""
    import numpy as np
    import tlg_workloads as W
    O = _oracle()
    A, B, _ = W.make_inputs(case)
    nthreads = cpu_threads()
    t0 = time.perf_counter()
    o = O.gemm(case.M, case.N, case.K, W.bits16(A), W.bits16(B), ab=case.ab, c=case.c,
               transpose_A=case.transpose_A, transpose_B=case.transpose_B, relu=case.relu,
               rows=(0, rows), nthreads=nthreads)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * case.N * case.K
    gpu = C_gpu[:rows].float().cpu().numpy().astype(np.float64)
    ok = bool((np.abs(gpu - o) <= O.tolerance(o, case.K, case.c)).all())
    return _cpu_record(flops / dt / 1e12, "TFLOP/s", nthreads,
                       f"first {rows} of {case.M} output rows of {case.name} ({flops / 1e9:.1f} GFLOP, "
                       f"fp64 triple loop, {dt:.1f} s)", dt, ok)


def cpu_baseline_mx(case, C_gpu, rows):
    import numpy as np
    import tlg_workloads as W
    O = _oracle()
    A, SA, B, SB, _ = W.make_mx_inputs(case)
    nthreads = cpu_threads()
    t0 = time.perf_counter()
    o = O.mxgemm(case.M, case.N, case.K, A.numpy(), SA.numpy(), B.numpy(), SB.numpy(), fmt_a=case.fmt,
                 fmt_b=case.fmt, c=case.c, relu=case.relu, rows=(0, rows), nthreads=nthreads)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * case.N * case.K
    gpu = C_gpu[:rows].float().cpu().numpy().astype(np.float64)
    ok = bool((np.abs(gpu - o) <= O.tolerance(o, case.K, case.c)).all())
    return _cpu_record(flops / dt / 1e12, "TFLOP/s", nthreads,
                       f"first {rows} of {case.M} output rows of {case.name} ({flops / 1e9:.1f} GFLOP, "
                       f"fp64 triple loop, {dt:.1f} s)", dt, ok)


def cpu_baseline_attn(case, O_gpu, positions):
    import numpy as np
    import tlg_workloads as W
    O = _oracle()
    q, k, v = W.make_attn_inputs(case)
    nthreads = cpu_threads()
    i0 = case.S - positions
    t0 = time.perf_counter()
    o = O.attn(case.B, case.S, case.H, case.D, W.bits16(q), W.bits16(k), W.bits16(v), dtype=case.dtype,
               causal=case.causal, scale=case.softmax_scale, rows=(i0, case.S), nthreads=nthreads)
    dt = time.perf_counter() - t0
    keys = sum(i + 1 for i in range(i0, case.S)) if case.causal else positions * case.S
    flops = 4.0 * case.D * keys * case.B * case.H
    gpu = O_gpu[:, i0:].float().cpu().numpy().astype(np.float64)
    ok = bool((np.abs(gpu - o) <= O.attn_tolerance(o, float(v.float().abs().max()), case.dtype)).all())
    return _cpu_record(flops / dt / 1e12, "TFLOP/s", nthreads,
                       f"last {positions} of {case.S} query positions of every batch and head of {case.name} "
                       f"({flops / 1e9:.1f} GFLOP, fp64 loops, {dt:.1f} s)", dt, ok)


def cpu_baseline_w4(case, C_gpu, rows):
    import numpy as np
    import tlg_workloads as W
    O = _oracle()
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
    return _cpu_record(sample_bytes / dt / 1e9, "GB/s", 1,
                       f"first {rows} of {case.M} output rows of {case.name} (all weights dequantized once, "
                       f"{2.0 * rows * case.N * case.K / 1e9:.1f} GFLOP, fp64 loops, single-threaded routine, "
                       f"{dt:.1f} s)", dt, ok)


def cpu_baseline_sp(case, C_gpu, rows):
    import numpy as np
    import tlg_workloads as W
    O = _oracle()
    A, Wv, Wm, _ = W.make_sp_inputs(case)
    nthreads = cpu_threads()
    t0 = time.perf_counter()
    o = O.spgemm(case.M, case.N, case.K, W.bits16(A), W.bits16(Wv), Wm.numpy(), dtype=case.ab, relu=case.relu,
                 rows=(0, rows), nthreads=nthreads)
    dt = time.perf_counter() - t0
    gpu = C_gpu[:rows].float().cpu().numpy().astype(np.float64)
    ok = bool((np.abs(gpu - o) <= O.tolerance(o, case.K, case.c)).all())
    flops = float(rows) * case.N * case.K
    return _cpu_record(flops / dt / 1e12, "TFLOP/s", nthreads,
                       f"first {rows} of {case.M} output rows of {case.name} ({flops / 1e9:.1f} GFLOP of "
                       f"stored-weight multiply-adds, fp64 loops, {dt:.1f} s)", dt, ok)


# ---------------------------------------------------------------------------- lines
def clock_fields(r, dev, dtype_key, tflops):
    """Per-launch distribution, the measured clock of the timed window, and the fraction
    of the matrix-core peak at that clock."""
    clk = r.get("clock") or {}
    out = {"per_launch_ms": r["per_launch_ms"], "clock": clk}
    mhz = clk.get("sclk_mhz")
    if mhz and tflops is not None and dtype_key in FLOP_PER_CLK_CU:
        peak = dev["cus"] * FLOP_PER_CLK_CU[dtype_key] * mhz * 1e6 / 1e12
        out["peak_at_measured_clock_tflops"] = peak
        out["frac_of_peak_at_measured_clock"] = tflops / peak
    return out


def gemm_line(args, case, is_mx, sampler, dev, log):
    r = (measure_mx if is_mx else measure)(case, args.steps, args.warmup, sampler, log)
    plan = r["plan"]
    info = plan.info
    hbm_bound = info.variant == 3                    # the skinny kernel streams B once
    ab = case.fmt if is_mx else case.ab
    ms = r["ms"]
    tflops = case.flops / (ms * 1e-3) / 1e12
    gbs = case.algorithmic_bytes / (ms * 1e-3) / 1e9
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS}
        value, unit = gbs, "GB/s"
    else:
        roof = {"bound": "mfma", "achieved": tflops, "peak": PEAK_TFLOPS[ab], "unit": "TFLOP/s",
                "frac": tflops / PEAK_TFLOPS[ab]}
        value, unit = tflops, "TFLOP/s"
    roof["traffic"] = stored_traffic(args.workload, info.variant)
    roof["kernel"] = plan.describe().split()[0]
    roof["per_launch"] = {"flops": case.flops, "algorithmic_bytes": case.algorithmic_bytes, "avg_kernel_ms": ms}
    out = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": ab, "data": "synthetic (seeded, see tlg_workloads.py)",
           "config": {"workload": f"{case.name}: {case.note}", "M": case.M, "N": case.N, "K": case.K,
                      "ab_dtype": ab, "c_dtype": case.c, "transpose_A": 0 if is_mx else case.transpose_A,
                      "transpose_B": 1 if is_mx else case.transpose_B, "epilogue": "relu" if case.relu else "none",
                      "plan": plan.describe(), "operand_sets_rotated": r["nsets"]},
           "roofline": roof, "timing": clock_fields(r, dev, ab, None if hbm_bound else tflops)}
    return out, r


def attn_line(args, case, sampler, dev, log):
    r = measure_attn(case, args.steps, args.warmup, sampler, log)
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
           "roofline": roof, "timing": clock_fields(r, dev, case.dtype, tflops)}
    if not args.no_cpu_baseline:
        positions = {"fa1": 1024, "fa2": 777, "fa3": 32, "fa4": 64}[case.name]
        out["cpu_baseline"] = cpu_baseline_attn(case, r["C"], positions)
    return out


def w4_line(args, case, sampler, dev, log):
    r = measure_w4(case, args.steps, args.warmup, sampler, log)
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
           "roofline": roof, "timing": clock_fields(r, dev, case.ab, None)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_w4(case, r["C"], {"w4a": 16, "w4b": 5, "w4c": 8}[case.name])
    return out


def sp_line(args, case, sampler, dev, log):
    """FLOPs count the stored (nonzero) weights only (M*N*K), priced against the dense MFMA
    peak of the operand dtype (the same fraction as the instruction's dense-equivalent
    rate against its own peak)."""
    r = measure_sp(case, args.steps, args.warmup, sampler, log)
    ms = r["ms"]
    tflops = case.flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[case.ab]
    roof = {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s", "frac": tflops / peak,
            "traffic": stored_traffic(args.workload, SP_VARIANT), "kernel": "gemm_sp",
            "per_launch": {"flops": case.flops, "algorithmic_bytes": case.algorithmic_bytes, "avg_kernel_ms": ms}}
    out = {"metric": "2:4 sparse GEMM TFLOP/s of stored-weight multiply-adds (fp32 accumulate) and % of dense "
                     "MFMA peak",
           "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": case.ab,
           "data": "synthetic (seeded, see tlg_workloads.py)",
           "config": {"workload": f"{case.name}: {case.note}", "M": case.M, "N": case.N, "K": case.K,
                      "ab_dtype": case.ab, "c_dtype": case.c, "plan": r["describe"],
                      "operand_sets_rotated": r["nsets"], "dense_equivalent_TFLOP/s": 2 * tflops},
           "roofline": roof, "timing": clock_fields(r, dev, case.ab, tflops)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_sp(case, r["C"], {"sp1": 256, "sp2": 1000, "sp3": 64}[case.name])
    return out


SECONDARY_MIN_MS = 20.0   # timed GPU work per secondary workload, at least


def secondary_entry(name, args, sampler, dev, log):
    import tlg_workloads as W
    steps, mt = max(10, args.steps // 2), SECONDARY_MIN_MS
    if name in W.MX_CONFIGS:
        c = W.MX_CONFIGS[name]
        rr, dt = measure_mx(c, steps, args.warmup, sampler, log, min_timed_ms=mt), c.fmt
    elif name in W.ATTN_CONFIGS:
        c = W.ATTN_CONFIGS[name]
        rr, dt = measure_attn(c, steps, args.warmup, sampler, log, min_timed_ms=mt), c.dtype
    elif name in W.W4_CONFIGS:
        c = W.W4_CONFIGS[name]
        rr, dt = measure_w4(c, steps, args.warmup, sampler, log, min_timed_ms=mt), c.ab
    elif name in W.SP_CONFIGS:
        c = W.SP_CONFIGS[name]
        rr, dt = measure_sp(c, steps, args.warmup, sampler, log, min_timed_ms=mt), c.ab
    else:
        c = W.CONFIGS[name]
        rr, dt = measure(c, steps, args.warmup, sampler, log, min_timed_ms=mt), c.ab
    t = rr["ms"] * 1e-3
    tflops = c.flops / t / 1e12
    gbs = c.algorithmic_bytes / t / 1e9
    entry = {"workload": name, "ms": rr["ms"], "timed_launches": rr["steps"], "TFLOP/s": tflops, "GB/s": gbs,
             "plan": rr["describe"],
             "mfma_frac": tflops / PEAK_TFLOPS[dt], "hbm_frac": gbs / PEAK_HBM_GBS}
    entry.update(clock_fields(rr, dev, dt, tflops))
    return entry


SECONDARY = ("c3", "c5b", "c2", "c4", "c1", "mx3", "mx6", "fa3", "fa1", "w4a", "sp3")
# Oracle sample sizes: about 10 s of the oracle on 16 host threads.
CPU_ROWS = {"c5a": 4096, "c3": 4096, "c2": 1024, "c1": 256, "c4": 1000, "c5b": 16, "mx1": 256, "mx2": 1000,
            "mx3": 2048, "mx4": 256, "mx5": 1000, "mx6": 2048}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="c5a", help="c1..c5b, a block-scaled workload mx1..mx3, "
                    "an attention workload fa1..fa4, a dequant GEMM workload w4a..w4c, "
                    "or a 2:4 sparse GEMM workload sp1..sp3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also launch one 1 GiB device copy (FETCH/WRITE counter calibration)")
    ap.add_argument("--warm-ms", type=float, default=WARM_MS,
                    help="GPU time of warm-up launches after the W counted ones (0 for counter runs, "
                         "which only need the launches to happen)")
    ap.add_argument("--no-clock", action="store_true", help="skip the clock-sampling window (counter runs)")
    return ap.parse_args()


def main():
    global WARM_MS, WARM_RULE, CLOCK_MS
    args = parse()
    if args.warm_ms != WARM_MS:
        WARM_MS = args.warm_ms
        WARM_RULE = WARM_RULE.replace(">= 100 ms", f">= {WARM_MS:g} ms")
    if args.no_clock:
        WARM_RULE = WARM_RULE.split(f"; then {CLOCK_MS:.0f} ms")[0]
        CLOCK_MS = 0.0
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              f"the sharding across GPUs is not built", file=sys.stderr)
        sys.exit(2)

    def log(m):
        print(m, file=sys.stderr, flush=True)

    # Host facts and the clock sampler come before the first GPU call.
    host = host_facts()
    sampler = ClockSampler()
    import torch
    import tlg_workloads as W
    try:
        dev = device_facts(sampler)
        if args.copy_calibration:
            x = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")   # 1 GiB
            y = torch.empty_like(x)
            y.copy_(x)
            torch.cuda.synchronize()
            log("[bench] copy calibration: 1 GiB read + 1 GiB write done")
            del x, y

        name = args.workload
        if name in W.SP_CONFIGS:
            out = sp_line(args, W.SP_CONFIGS[name], sampler, dev, log)
        elif name in W.W4_CONFIGS:
            out = w4_line(args, W.W4_CONFIGS[name], sampler, dev, log)
        elif name in W.ATTN_CONFIGS:
            out = attn_line(args, W.ATTN_CONFIGS[name], sampler, dev, log)
        else:
            is_mx = name in W.MX_CONFIGS
            case = W.MX_CONFIGS[name] if is_mx else W.CONFIGS[name]
            out, r = gemm_line(args, case, is_mx, sampler, dev, log)
            if not args.no_secondary:
                out["secondary"] = [secondary_entry(s, args, sampler, dev, log) for s in SECONDARY if s != name]
            if not args.no_cpu_baseline:
                out["cpu_baseline"] = (cpu_baseline_mx if is_mx else cpu_baseline)(case, r["C"], CPU_ROWS[name])
        out["timing_rule"] = WARM_RULE
        out["device"] = dev
        out["host"] = host
    finally:
        sampler.stop()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
