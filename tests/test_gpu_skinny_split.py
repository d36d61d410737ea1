"""GPU parity of the skinny kernel's wider instances (32 x 64 and 64 x 32 outputs per
workgroup for 16 < M <= 64) and of its K split over several workgroups per column block
(grids of fewer than 256 blocks of 16 x 64 outputs: each workgroup streams a range of K
stages and the last one of a block to finish sums the fp32 partial tiles in K-range
order).  Every output is compared with the oracle: within the tolerance on N(0,1)/sqrt(K)
and uniform inputs, exactly on small integers (a range read twice or lost fails), with
guard bands around C, accumulating onto C, over two row blocks, and over four runs of one
plan (the per-block counters must come back to zero; repeats are bit-identical).  Shapes
include the decode shape's share of one GPU when its columns are split over 2, 4 or 8."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import tlg_workloads as W
from parity import assert_exact, assert_within_tolerance, log, oracle_full, out_values, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import tiled_dense_gemm_02_amd as tlg
    tlg.load_library()
    yield


def _check(case, exact=False, guard=1024, variant="auto", want_splits=None):
    log(f"[case] skinny-split {case.name} M={case.M} N={case.N} K={case.K} ab={case.ab} c={case.c} "
        f"relu={case.relu} clear={case.clear_accum} dist={case.dist}")
    A, B, C_in = W.make_inputs(case)
    C, plan, buf, g = run_gpu(case, A, B, C_in, variant=variant, guard=guard)
    log(f"    plan: {plan.describe()}")
    assert plan.info.variant == 3
    if want_splits is not None:
        assert plan.info.splits == want_splits
    if guard:
        raw = buf.view(torch.uint8).cpu()
        esz = 4 if case.c == "f32" else 2
        assert bool((raw[:g * esz] == 0x5A).all()) and bool((raw[(g + case.M * case.N) * esz:] == 0x5A).all()), \
            "store outside C"
    gpu = out_values(C)
    o = oracle_full(case, A, B, C_in)
    if exact:
        assert_exact(gpu, o, case, plan.describe())
    else:
        err = assert_within_tolerance(gpu, o, case, plan.describe())
        log(f"    max|err| = {err:.3e}")
    return plan


# (M, N, K, splits the plan must choose)
_SHARDS = [(16, 8192, 8192, 2), (16, 4096, 8192, 4), (16, 2048, 8192, 8)]


@pytest.mark.parametrize("M,N,K,splits", _SHARDS)
def test_decode_shares(M, N, K, splits):
    """16 x 16384 x 8192 with its columns split over 2, 4 and 8 GPUs."""
    case = W.GemmCase(f"share-{N}", M, N, K, transpose_B=1, dist="uniform", seed=5100 + N)
    _check(case, want_splits=splits)


@pytest.mark.parametrize("M,N,K", [(16, 2048, 8192), (13, 4000, 8200), (16, 640, 3000), (1, 136, 4096)])
def test_small_integers_exact(M, N, K):
    """Ragged rows and columns, a last stage of 8 elements (K = 8200), ranges of 3-4 stages."""
    case = W.GemmCase(f"int-{M}x{N}x{K}", M, N, K, c="f32", transpose_B=1, relu=1, dist="smallint",
                      seed=5200 + K)
    plan = _check(case, exact=True)
    assert plan.info.splits > 1


@pytest.mark.parametrize("c", ["f16", "f32", "bf16"])
def test_accumulate_onto_c(c):
    case = W.GemmCase(f"accum-{c}", 16, 2048, 4096, ab="bf16" if c == "bf16" else "f16", c=c, transpose_B=1,
                      clear_accum=0, relu=int(c == "f32"), dist="normal", seed=5300)
    plan = _check(case)
    assert plan.info.splits > 1


def test_two_row_blocks_forced():
    """M = 80 through the forced skinny variant: two row blocks of 64, each with its own ranges."""
    case = W.GemmCase("rows80", 80, 1024, 4096, transpose_B=1, dist="normal", seed=5400)
    plan = _check(case, variant="skinny")
    assert plan.info.splits > 1


def test_plan_reused_counters_return_to_zero():
    import tiled_dense_gemm_02_amd as tlg
    dev = torch.device("cuda:0")
    M, N, K = 16, 4096, 8192
    cases = [W.GemmCase(f"reuse-{i}", M, N, K, transpose_B=1, dist="normal", seed=5500 + i) for i in range(2)]
    inputs = [W.make_inputs(c) for c in cases]
    plan = tlg.Gemm(M, N, K, torch.float16, torch.float16, transpose_B=True)
    assert plan.info.splits == 4 and plan.info.workspace_bytes > 0
    outs = []
    for rep in range(4):
        A, B, _ = inputs[rep % 2]
        C = torch.empty((M, N), dtype=torch.float16, device=dev)
        plan.run(A.to(dev), B.to(dev), C)
        torch.cuda.synchronize()
        outs.append(C.view(torch.int16).cpu())
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[3])
    for i, case in enumerate(cases):
        A, B, _ = inputs[i]
        assert_within_tolerance(out_values(outs[i].view(torch.float16)), oracle_full(case, A, B, None), case,
                                "plan reuse")


# ---------------------------------------------------------------- 17 <= M <= 64 (and more rows forced)
@pytest.mark.parametrize("M,N,K", [(17, 1000, 1040), (24, 16384, 8192), (32, 4000, 8200), (48, 2048, 4096),
                                   (64, 16384, 8192), (64, 999, 3000)])
def test_wider_row_blocks_exact(M, N, K):
    """32 rows (M <= 32) and 64 rows (M <= 64, 32 columns per block) of A per workgroup:
    exact on small integers, ragged rows, columns and K, split and unsplit plans."""
    case = W.GemmCase(f"rows-{M}x{N}x{K}", M, N, K, c="f32", transpose_B=1, relu=M % 2, dist="smallint",
                      seed=5600 + M)
    plan = _check(case, exact=True)
    assert plan.info.block_m == (32 if M <= 32 else 64)


@pytest.mark.parametrize("M,c", [(40, "f16"), (100, "bf16")])
def test_wider_row_blocks_tolerance(M, c):
    """M = 100 through the forced skinny variant: two row blocks of 64."""
    case = W.GemmCase(f"rows-{M}-{c}", M, 3000, 4096, ab="bf16" if c == "bf16" else "f16", c=c, transpose_B=1,
                      dist="normal", seed=5700 + M)
    _check(case, variant="skinny")


def test_wider_row_blocks_accumulate():
    case = W.GemmCase("rows-accum", 56, 2048, 8192, c="f16", transpose_B=1, clear_accum=0, relu=1, dist="normal",
                      seed=5800)
    plan = _check(case)
    assert plan.info.block_m == 64 and plan.info.splits > 1
