"""GPU test of tlg_gemm_run_noalloc (the entry point that allocates nothing): through the
C-ABI, against the plan + run pair of tlg_gemm_create / tlg_gemm_run on the same inputs,
which runs the same kernel, so the outputs must be bit-identical; and against the oracle
within the tolerance |gpu - o| <= 2^-10 |o| + 1e-4 sqrt(K).  Two calls in a row, the second
smaller, both with a split-K choice (the calls share the library's static scratch), then
shapes whose automatic plan needs no scratch."""
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
