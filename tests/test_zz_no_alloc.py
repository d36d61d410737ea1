"""GPU test of tlg_gemm_run_noalloc (the entry point that allocates nothing): through the
C-ABI, against the plan + run pair of tlg_gemm_create / tlg_gemm_run on the same inputs,
which runs the same kernel, so the outputs must be bit-identical; and against the oracle
within the tolerance |gpu - o| <= 2^-10 |o| + 1e-4 sqrt(K).  Two calls in a row, the second
smaller, both with a split-K choice (the calls share the library's static scratch), then
shapes whose automatic plan needs no scratch; and the same calls captured into a graph and
replayed."""
from __future__ import annotations

import ctypes

import pytest
import torch

import tlg_workloads as W
from parity import assert_within_tolerance, log, oracle_full, out_values

pytestmark = pytest.mark.gpu


def _pair(case):
    import tiled_dense_gemm_02_amd as tlg
    lib = tlg.load_library()
    dev = torch.device("cuda:0")
    A, B, _ = W.make_inputs(case)
    Ad, Bd = A.to(dev), B.to(dev)
    T = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    C1 = torch.full((case.M, case.N), 7.0, dtype=T[case.c], device=dev)
    C2 = torch.full((case.M, case.N), -3.0, dtype=T[case.c], device=dev)
    plan = tlg.Gemm(case.M, case.N, case.K, T[case.ab], T[case.c], transpose_A=bool(case.transpose_A),
                    transpose_B=bool(case.transpose_B), epilogue="relu" if case.relu else "none")
    log(f"[case] noalloc {case.name}: {plan.describe()}")
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.tlg_gemm_run_noalloc(case.M, case.N, case.K, tlg._code(T[case.ab]), tlg._code(T[case.c]),
                                  case.transpose_A, case.transpose_B, 1, case.relu, Ad.data_ptr(), Bd.data_ptr(),
                                  C1.data_ptr(), ctypes.c_void_p(stream))
    assert st == 0, tlg.status_name(st)
    plan.run(Ad, Bd, C2)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.uint8), C2.view(torch.uint8)), "noalloc result differs from the plan's"
    o = oracle_full(case, A, B, None)
    assert_within_tolerance(out_values(C1), o, case, "tlg_gemm_run_noalloc")
    return plan


def test_noalloc_split_k_twice_second_smaller():
    first = W.GemmCase("noalloc-1024x1024x4096", 1024, 1024, 4096, relu=1, seed=4301)
    second = W.GemmCase("noalloc-520x300x3100", 520, 300, 3100, ab="bf16", c="f32", transpose_B=1, seed=4302)
    p1 = _pair(first)
    assert p1.info.splits == 4
    p2 = _pair(second)
    assert p2.info.splits > 1 and p2.info.workspace_bytes < p1.info.workspace_bytes
    # and the first again after the smaller one (the counters came back to zero)
    _pair(first)


def test_noalloc_skinny_split_twice_second_smaller():
    """The skinny kernel's K ranges keep their partial tiles and counters in the same
    static scratch."""
    first = W.GemmCase("noalloc-16x4096x8192", 16, 4096, 8192, transpose_B=1, seed=4303)
    second = W.GemmCase("noalloc-9x2048x4096", 9, 2048, 4096, c="f32", transpose_B=1, relu=1, seed=4304)
    p1 = _pair(first)
    assert p1.info.variant == 3 and p1.info.splits == 4
    p2 = _pair(second)
    assert p2.info.variant == 3 and p2.info.splits > 1 and p2.info.workspace_bytes < p1.info.workspace_bytes
    _pair(first)


def test_noalloc_without_scratch():
    for case in (W.CONFIGS["c1"], W.CONFIGS["c4"], W.CONFIGS["c5b"].with_(N=2048, K=1024)):
        plan = _pair(case)
        assert plan.info.splits == 1


def test_noalloc_under_graph_capture():
    """Callers under HIP graph capture: a split-K and a skinny-split call captured once
    into a graph (after one eager call on the device, which sets up the static scratch),
    replayed four times with C cleared, and other eager calls that use the same scratch,
    between the replays.  Every replay must equal the eager result bit for bit."""
    import tiled_dense_gemm_02_amd as tlg
    dev = torch.device("cuda:0")
    T = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    cases = [W.GemmCase("graph-1024x1024x4096", 1024, 1024, 4096, relu=1, seed=4311),
             W.GemmCase("graph-16x4096x8192", 16, 4096, 8192, c="f32", transpose_B=1, seed=4312)]
    runs = []
    for case in cases:
        A, B, _ = W.make_inputs(case)
        Ad, Bd = A.to(dev), B.to(dev)
        kw = dict(transpose_B=bool(case.transpose_B), epilogue="relu" if case.relu else "none")
        ref = torch.empty((case.M, case.N), dtype=T[case.c], device=dev)
        tlg.gemm_noalloc(Ad, Bd, ref, **kw)
        torch.cuda.synchronize()
        runs.append((case, Ad, Bd, kw, ref, torch.empty_like(ref)))
    side = torch.cuda.Stream(dev)
    graph = torch.cuda.CUDAGraph()
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for case, Ad, Bd, kw, ref, out in runs:       # warm-up on the capture stream
            tlg.gemm_noalloc(Ad, Bd, out, **kw)
    torch.cuda.synchronize()
    log("[case] noalloc graph: capturing " + ", ".join(r[0].name for r in runs))
    with torch.cuda.graph(graph, stream=side):
        for case, Ad, Bd, kw, ref, out in runs:
            tlg.gemm_noalloc(Ad, Bd, out, **kw)
    for rep in range(4):
        for _, _, _, _, _, out in runs:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for case, _, _, _, ref, out in runs:
            assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8)), f"replay {rep} of {case.name} differs"
        # eager calls between the replays, on the same scratch (the other shape's plan)
        for case, Ad, Bd, kw, ref, out in runs[::-1]:
            scratch_user = torch.empty_like(ref)
            tlg.gemm_noalloc(Ad, Bd, scratch_user, **kw)
            torch.cuda.synchronize()
            assert torch.equal(scratch_user.view(torch.uint8), ref.view(torch.uint8))
        log(f"    replay {rep}: bit-identical to the eager result")
