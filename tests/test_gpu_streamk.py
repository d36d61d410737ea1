"""GPU parity of the persistent stream-K schedules (tile256dma_streamk,
tile128dma_streamk) against the oracle: the small-grid workloads with the scheduler
forced, grids with whole waves plus a shared tail, ragged shapes in every layout,
accumulation onto C, K = 0, small-integer exactness, and one plan run several times
in a row (its per-tile counters must come back to zero after every launch, and each
tile must be finished exactly once: any tile finished twice with clear_accum = 0, or
never, shows up as a wrong value).  Tolerance |gpu - o| <= 2^-10 |o| + 1e-4 sqrt(K)
(2^-8 for bf16 output); exact for small integers."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import tlg_workloads as W
from parity import assert_exact, assert_within_tolerance, log, oracle_full, out_values, run_gpu

pytestmark = pytest.mark.gpu

SK256, SK128 = "tile256dma_streamk", "tile128dma_streamk"


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import tiled_dense_gemm_02_amd as tlg
    tlg.load_library()
    yield


def _check(case, variant, exact=False, guard=1024):
    log(f"[case] {case.name} M={case.M} N={case.N} K={case.K} ab={case.ab} c={case.c} tA={case.transpose_A} "
        f"tB={case.transpose_B} relu={case.relu} clear={case.clear_accum} dist={case.dist} variant={variant}")
    A, B, C_in = W.make_inputs(case)
    C, plan, buf, g = run_gpu(case, A, B, C_in, variant=variant, guard=guard)
    log(f"    {plan.describe()}")
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
        assert_within_tolerance(gpu, o, case, plan.describe())
    return plan


def test_config2_streamk_forced():
    plan = _check(W.CONFIGS["c2"], SK128)
    assert plan.info.dp_tiles == 0 and plan.info.sk_tiles == 64 and plan.info.grid == 256
    plan = _check(W.CONFIGS["c2"], SK256)
    assert plan.info.sk_tiles == 16


def test_config4_streamk_forced():
    plan = _check(W.CONFIGS["c4"], SK128, guard=4096)
    assert plan.info.sk_tiles == 96
    _check(W.CONFIGS["c4"], SK256, guard=4096)


def test_whole_waves_plus_shared_tail():
    """8192 x 4608 x 1024: 576 tiles of 256 x 256 -> 256 whole, 320 shared."""
    case = W.GemmCase("sk-8192x4608x1024", 8192, 4608, 1024, relu=1, dist="normal", seed=4401)
    plan = _check(case, SK256, guard=4096)
    assert (plan.info.dp_tiles, plan.info.sk_tiles) == (256, 320)


def test_ragged_large_exact():
    """306 tiles of 256 x 256 (one wave plus a tail, all shared), K = 4100: exact."""
    case = W.GemmCase("sk-4600x4350x4100", 4600, 4350, 4100, c="f32", transpose_B=1, dist="smallint", seed=4402)
    plan = _check(case, SK256, exact=True, guard=4096)
    assert (plan.info.dp_tiles, plan.info.sk_tiles) == (0, 306)


@pytest.mark.parametrize("variant", [SK256, SK128])
@pytest.mark.parametrize("tA,tB", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_ragged_sweep_layouts(variant, tA, tB):
    rng = np.random.default_rng(4500 + 10 * tA + tB + (0 if variant == SK256 else 100))
    for it in range(5):
        M, N, K = (int(x) for x in rng.choice([1, 17, 64, 129, 257, 300, 520], 3))
        K = int(rng.choice([1, 63, 65, 200, 777, 1500]))
        r8 = lambda x: (x + 7) // 8 * 8
        M = r8(M) if tA else M
        N = N if tB else r8(N)
        ab = "f16" if it % 2 == 0 else "bf16"
        c = ["f16", "f32", "bf16"][it % 3]
        case = W.GemmCase(f"sk-ragged{it}", M, N, K, ab=ab, c=c, transpose_A=tA, transpose_B=tB, relu=it % 2,
                          seed=4600 + it)
        _check(case, variant)


@pytest.mark.parametrize("variant", [SK256, SK128])
@pytest.mark.parametrize("ab", ["f16", "bf16"])
def test_small_integers_exact(variant, ab):
    case = W.GemmCase("sk-int", 520, 392, 1000, ab=ab, c="f32", transpose_B=1, dist="smallint", relu=1, seed=4700)
    _check(case, variant, exact=True)


@pytest.mark.parametrize("variant", [SK256, SK128])
def test_accumulate_onto_c_and_k0(variant):
    """clear_accum = 0: the elected segment adds C's prior value once."""
    for c in ("f16", "f32"):
        case = W.GemmCase(f"sk-accum-{c}", 300, 264, 1536, c=c, clear_accum=0, relu=1, seed=4800)
        _check(case, variant)
    case = W.GemmCase("sk-k0", 70, 96, 0, c="f32", clear_accum=0, relu=1, seed=4801)
    plan = _check(case, variant)
    assert plan.info.sk_tiles == 0


@pytest.mark.parametrize("variant", [SK256, SK128])
def test_plan_reused_counters_return_to_zero(variant):
    """One plan, four runs on alternating inputs: each matches the oracle and repeats are
    bit-identical (a counter left non-zero would elect the wrong segment next time)."""
    import tiled_dense_gemm_02_amd as tlg
    M, N, K = 1000, 1100, 2000
    plan = tlg.Gemm(M, N, K, transpose_B=True, variant=variant)
    log(f"[case] stream-K reuse {plan.describe()}")
    outs = []
    for rep in range(4):
        case = W.GemmCase("sk-reuse", M, N, K, transpose_B=1, seed=4900 + rep % 2)
        A, B, _ = W.make_inputs(case)
        C = torch.empty((M, N), dtype=torch.float16, device="cuda")
        plan.run(A.cuda(), B.cuda(), C)
        torch.cuda.synchronize()
        assert_within_tolerance(out_values(C), oracle_full(case, A, B, None), case, plan.describe())
        outs.append(C.view(torch.int16).cpu())
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[3])
