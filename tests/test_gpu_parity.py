"""GPU parity: the HIP path (through the C-ABI binding) against the CPU oracle on the
same seeded inputs.  Tolerance |gpu - oracle| <= 2^-10 |oracle| + 1e-4 sqrt(K) for
inputs in [-1, 1]; exact (after the oracle's own rounding) for small-integer inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import tlg_workloads as W
from parity import (assert_exact, assert_within_tolerance, log, oracle_full, oracle_points, out_values,
                    run_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import tiled_dense_gemm_02_amd as tlg
    tlg.load_library()
    log(f"device: {torch.cuda.get_device_name(0)}")
    yield


def _full_check(case, variant="auto", guard=0, exact=False, a_offset=0, b_offset=0):
    log(f"[case] {case.name} M={case.M} N={case.N} K={case.K} ab={case.ab} c={case.c} "
        f"tA={case.transpose_A} tB={case.transpose_B} relu={case.relu} clear={case.clear_accum} "
        f"dist={case.dist} variant={variant} offsets={a_offset}/{b_offset}")
    A, B, C_in = W.make_inputs(case)
    C, plan, buf, g = run_gpu(case, A, B, C_in, variant=variant, guard=guard, a_offset=a_offset,
                              b_offset=b_offset)
    gpu = out_values(C)
    o = oracle_full(case, A, B, C_in)
    if exact:
        assert_exact(gpu, o, case, plan.describe())
    else:
        err = assert_within_tolerance(gpu, o, case, plan.describe())
        log(f"    max|err| = {err:.3e}  ({plan.describe()})")
    if guard:
        raw = buf.view(torch.uint8).cpu()
        esz = 4 if case.c == "f32" else 2
        head = raw[:g * esz]
        tail = raw[(g + case.M * case.N) * esz:]
        assert bool((head == 0x5A).all()) and bool((tail == 0x5A).all()), "store outside C"
    return plan


# ---------------------------------------------------------------- the five workloads
def test_config1_relu_256():
    _full_check(W.CONFIGS["c1"], guard=4096)


def test_config2_1024():
    plan = _full_check(W.CONFIGS["c2"])
    assert plan.info.block_m == 32 and plan.info.block_k == 128 and plan.info.k_tiles == 8   # 32x128 tiles, K in tiles of 128
    plan = _full_check(W.CONFIGS["c2"], variant="tile64dma")
    assert plan.info.block_m == 64 and plan.info.k_tiles == 8
    plan = _full_check(W.CONFIGS["c2"], variant="tile128dma")
    assert plan.info.k_tiles == 16          # 1024 / 64, the pages' K trip count
    plan = _full_check(W.CONFIGS["c2"], variant="tile128dma_sk")
    assert plan.info.splits == 4 and plan.info.k_tiles == 4   # K split in 4 ranges of 4 K tiles


def test_config4_ragged_bf16_bt_f32out():
    plan = _full_check(W.CONFIGS["c4"], guard=4096)
    assert plan.info.splits == 1
    plan = _full_check(W.CONFIGS["c4"], variant="tile128dma_sk", guard=4096)
    assert plan.info.splits == 2


def _sampled_check(case, count):
    log(f"[case] {case.name} sampled ({count} points) M={case.M} N={case.N} K={case.K}")
    A, B, C_in = W.make_inputs(case)
    C, plan, _, _ = run_gpu(case, A, B, C_in)
    ms, ns = W.sample_points(case.M, case.N, count)
    gpu = out_values(C)
    o = oracle_points(case, A, B, C_in, ms, ns)
    err = assert_within_tolerance(gpu[ms, ns], o, case, plan.describe())
    log(f"    max|err| = {err:.3e}  ({plan.describe()})")
    # properties that hold everywhere: finite, ReLU output non-negative
    assert np.isfinite(gpu).all()
    if case.relu:
        assert (gpu >= 0).all()
    return plan, gpu


def test_config3_relu_4096_sampled():
    plan, gpu = _sampled_check(W.CONFIGS["c3"], 4096)
    assert plan.info.variant == 6 and plan.info.grid == 256


def test_config5a_8192_sampled():
    plan, _ = _sampled_check(W.CONFIGS["c5a"], 4096)
    assert plan.info.grid == 1024


def test_config5b_skinny_full():
    plan = _full_check(W.CONFIGS["c5b"])
    assert plan.info.variant == 3


# ---------------------------------------------------------------- exactness
# The skinny kernel takes A stored [M,K] and B stored [N,K] only (tA=0, tB=1).
# The 64x128 and 32x128 direct-load kernels take A stored [M,K] only (tA=0).
def _layouts_of(v, layouts=((0, 0), (0, 1), (1, 0), (1, 1))):
    return [(tA, tB) for tA, tB in layouts
            if (v != "skinny" or (tA, tB) == (0, 1)) and (v not in ("tile64dma", "tile32dma") or tA == 0)]


_EXACT_CASES = [(v, tA, tB) for v in ["tile256", "tile256w8", "tile256dma", "tile128dma", "tile128dma_sk", "tile64dma",
                                      "tile32dma", "tile128", "skinny"]
                for tA, tB in _layouts_of(v)]


@pytest.mark.parametrize("variant,tA,tB", _EXACT_CASES)
@pytest.mark.parametrize("ab", ["f16", "bf16"])
def test_small_integers_exact(variant, ab, tA, tB):
    # 300 rows: ragged for the 128 tile; the 256 tile needs 128-bit loads, so with A
    # stored [K, M] its M must be a multiple of 8 (304)
    M = {"skinny": 16, "tile128": 300, "tile256": 304, "tile256w8": 304, "tile256dma": 304, "tile128dma": 304,
         "tile128dma_sk": 304, "tile64dma": 300, "tile32dma": 300}[variant]
    case = W.GemmCase("smallint", M, 264, 200, ab=ab, c="f32", transpose_A=tA, transpose_B=tB,
                      dist="smallint", seed=77, relu=1)
    _full_check(case, variant=variant, exact=True)


# ---------------------------------------------------------------- edges
RAGGED = [1, 15, 17, 31, 33, 64, 65, 127, 129, 257]


@pytest.mark.parametrize("variant,tA,tB", [(v, tA, tB) for v in ["tile128", "tile256", "tile256w8", "tile256dma",
                                                                   "tile128dma", "tile128dma_sk", "tile64dma",
                                                                   "tile32dma"]
                                           for tA, tB in _layouts_of(v)])
def test_ragged_sweep(variant, tA, tB):
    rng = np.random.default_rng(1000 + 10 * tA + tB + {"tile128": 0, "tile256": 100, "tile256w8": 200, "tile256dma": 300,
                                                       "tile128dma": 400, "tile128dma_sk": 500,
                                                       "tile64dma": 600, "tile32dma": 700}[variant])
    for it in range(6):
        M, N, K = (int(x) for x in rng.choice(RAGGED, 3))
        r8 = lambda x: (x + 7) // 8 * 8
        if variant in ("tile256", "tile256w8"):     # 128-bit register-staged loads: every extent % 8 == 0
            M, N, K = r8(M), r8(N), r8(K)
        elif variant in ("tile256dma", "tile128dma", "tile128dma_sk", "tile64dma", "tile32dma"):   # only M/N-contiguous rows need % 8 == 0
            M = r8(M) if tA else M
            N = N if tB else r8(N)
        ab = "f16" if it % 2 == 0 else "bf16"
        c = ["f16", "f32", "bf16"][it % 3]
        case = W.GemmCase(f"ragged{it}", M, N, K, ab=ab, c=c, transpose_A=tA, transpose_B=tB,
                          relu=it % 2, seed=500 + it)
        _full_check(case, variant=variant, guard=1024)


@pytest.mark.parametrize("variant,tA,tB", [(v, tA, tB) for v in ["tile256dma", "tile128dma", "tile128dma_sk", "tile64dma",
                                                                   "tile32dma"]
                                           for tA, tB in _layouts_of(v, ((0, 0), (0, 1), (1, 1)))])
def test_direct_loads_unaligned_k_and_base(variant, tA, tB):
    """K-contiguous operands at any K and at a base address 2 bytes off 16-byte alignment:
    unaligned 128-bit loads plus the trimmed K tail."""
    for it, K in enumerate((1, 7, 9, 63, 65, 200, 777)):
        M = 136 if tA else 130
        N = 77 if tB else 96
        case = W.GemmCase(f"unaligned-k{K}", M, N, K, ab="f16" if it % 2 == 0 else "bf16",
                          c=["f16", "f32"][it % 2], transpose_A=tA, transpose_B=tB, relu=it % 2,
                          seed=700 + it)
        _full_check(case, variant=variant, guard=1024, a_offset=0 if tA else 1, b_offset=1 if tB else 0)
    # small integers: exact
    case = W.GemmCase("unaligned-int", 130 if not tA else 136, 77 if tB else 96, 333, ab="bf16", c="f32",
                      transpose_A=tA, transpose_B=tB, dist="smallint", seed=790)
    _full_check(case, variant=variant, exact=True, a_offset=0 if tA else 1, b_offset=1 if tB else 0)


@pytest.mark.parametrize("M", [1, 8, 16, 17, 32])
def test_skinny_rows(M):
    case = W.GemmCase(f"skinny{M}", M, 1000, 520, transpose_B=1, seed=900 + M, relu=M % 2)
    plan = _full_check(case, variant="skinny", guard=1024)
    assert plan.info.variant == 3


def test_accumulate_onto_c():
    for variant, tB in (("tile128", 0), ("tile256", 0), ("tile256w8", 0), ("tile256dma", 0), ("tile256dma", 1),
                        ("tile128dma", 0), ("tile128dma", 1), ("tile128dma_sk", 0), ("tile128dma_sk", 1),
                        ("tile64dma", 0), ("tile64dma", 1), ("tile32dma", 0), ("tile32dma", 1),
                        ("skinny", 1)):
        for c in ("f16", "f32"):
            case = W.GemmCase(f"accum-{variant}-{c}", 16 if variant == "skinny" else 264, 200, 136,
                              c=c, transpose_B=tB, clear_accum=0, relu=1, seed=31)
            _full_check(case, variant=variant)


def test_empty_k_and_empty_output():
    case = W.GemmCase("k0", 70, 90, 0, c="f32", clear_accum=0, seed=5)
    _full_check(case)
    case = W.GemmCase("k0relu", 70, 90, 0, c="f16", relu=1, seed=6)
    _full_check(case)
    case = W.GemmCase("k0skinny", 16, 96, 0, c="f32", transpose_B=1, clear_accum=0, relu=1, seed=7)
    assert _full_check(case).info.variant == 3
    import tiled_dense_gemm_02_amd as tlg
    plan = tlg.Gemm(0, 5, 7)
    assert plan.info.variant == 4
    A = torch.empty((0, 7), dtype=torch.float16, device="cuda")
    B = torch.empty((7, 5), dtype=torch.float16, device="cuda")
    C = torch.empty((0, 5), dtype=torch.float16, device="cuda")
    plan.run(A, B, C)


def test_deterministic():
    case = W.CONFIGS["c2"].with_(name="determinism", relu=1)
    A, B, _ = W.make_inputs(case)
    C1, _, _, _ = run_gpu(case, A, B, None)
    C2, _, _, _ = run_gpu(case, A, B, None)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    case = W.CONFIGS["c5b"].with_(name="determinism-skinny", N=2048, K=4096)
    A, B, _ = W.make_inputs(case)
    C1, _, _, _ = run_gpu(case, A, B, None)
    C2, _, _, _ = run_gpu(case, A, B, None)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))


def test_split_k_plan_reused():
    """One split-K plan run on several inputs in a row (its per-tile counters return to
    zero after every launch), then on the same inputs again: each result within the
    tolerance, repeats bit-identical.  Range counts 2, 3, 4, 6 and 8, ragged last K tiles
    (K = 1000: the 16th K tile is 40 wide) and a last range shorter than the others
    (K = 3100: 49 K tiles in 5 ranges of 9 and one of 4, whose last K tile is 28 wide)."""
    import tiled_dense_gemm_02_amd as tlg
    for M, N, K, variant, splits in ((128, 384, 256, "tile128dma_sk", 2), (300, 264, 520, "tile128dma_sk", 3),
                                     (1024, 1024, 4096, "auto", 4), (1000, 600, 3100, "auto", 6),
                                     (200, 72, 1000, "tile128dma_sk", 8)):
        want = tlg.select(M, N, K, transpose_B=True, epilogue="relu", variant=variant)
        case = W.GemmCase(f"sk-{M}x{N}x{K}", M, N, K, transpose_B=1, relu=1, seed=1234)
        plan = tlg.Gemm(M, N, K, transpose_B=True, epilogue="relu", variant=variant)
        assert plan.info.variant == 8 and plan.info.splits == splits
        assert plan.info.as_dict() == want.as_dict()
        log(f"[case] split-K reuse {plan.describe()}")
        outs = []
        for rep in range(4):
            A, B, _ = W.make_inputs(case.with_(seed=1234 + rep % 2))
            C = torch.empty((M, N), dtype=torch.float16, device="cuda")
            plan.run(A.cuda(), B.cuda(), C)
            torch.cuda.synchronize()
            o = oracle_full(case, A, B, None)
            assert_within_tolerance(out_values(C), o, case, plan.describe())
            outs.append(C.view(torch.int16).cpu())
        assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[3])


@pytest.mark.parametrize("shape", [("c2", None), ("c4", None), ("longk", (1024, 1024, 8192))])
def test_autotuned_plan(shape):
    """tlg_gemm_tune: every candidate timed once, the fastest kept (its entry is the
    minimum of the report), its result within the tolerance, the choice cached."""
    import tiled_dense_gemm_02_amd as tlg
    name, mnk = shape
    case = W.CONFIGS[name] if mnk is None else W.CONFIGS["c2"].with_(name=name, M=mnk[0], N=mnk[1], K=mnk[2])
    A, B, _ = W.make_inputs(case)
    dt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    C = torch.empty((case.M, case.N), dtype=dt[case.c], device="cuda")
    Ad, Bd = A.cuda(), B.cuda()
    kw = dict(transpose_A=bool(case.transpose_A), transpose_B=bool(case.transpose_B),
              epilogue="relu" if case.relu else "none")
    plan, report = tlg.tune(Ad, Bd, C, iters=3, **kw)
    log(f"[case] tune {case.name}: chose {plan.describe()}")
    for v, sp, ms in report:
        log(f"    {v:14s} splits {sp}: {ms * 1e3:8.1f} us")
    assert len(report) >= 3
    best = min(report, key=lambda r: r[2])
    assert (tlg.VARIANTS[best[0]], best[1]) == (plan.info.variant, plan.info.splits)
    if case.M * case.N <= 1 << 21:
        o = oracle_full(case, A, B, None)
        C.fill_(0)
        plan.run(Ad, Bd, C)
        torch.cuda.synchronize()
        assert_within_tolerance(out_values(C), o, case, plan.describe())
    else:
        ms_, ns_ = W.sample_points(case.M, case.N, 2048)
        o = oracle_points(case, A, B, None, ms_, ns_)
        C.fill_(0)
        plan.run(Ad, Bd, C)
        torch.cuda.synchronize()
        assert_within_tolerance(out_values(C)[ms_, ns_], o, case, plan.describe())
    plan2, report2 = tlg.tune(Ad, Bd, C, iters=3, **kw)
    assert report2 == [] and plan2.info.as_dict() == plan.info.as_dict()


def test_zero_padding_invariant_on_gpu():
    """The ragged-K workload equals the same GEMM with K zero-padded to 832 = 13 * 64."""
    case = W.CONFIGS["c4"]
    A, B, _ = W.make_inputs(case)
    Kp = 832
    Ap = torch.zeros((case.M, Kp), dtype=A.dtype); Ap[:, :case.K] = A
    Bp = torch.zeros((case.N, Kp), dtype=B.dtype); Bp[:, :case.K] = B
    C1, _, _, _ = run_gpu(case, A, B, None)
    C2, _, _, _ = run_gpu(case.with_(K=Kp), Ap, Bp, None)
    assert torch.equal(C1, C2)


@pytest.mark.parametrize("shape", [(520, 392, 1000, 0, 1), (300, 264, 777, 0, 0), (1024, 1024, 1024, 0, 0),
                                   (264, 136, 640, 1, 1)])
def test_ring_depths_and_tilings_bit_identical(shape):
    """The direct-load kernels with a 2-slot ring of 64-wide K tiles (256x256 tiles), a
    4-slot ring of 64-wide K tiles (128x128), a 3-slot ring of 128-wide K tiles (64x128)
    and a 4-slot ring of 128-wide K tiles (32x128) all form every output's fp32 sum from the same MFMA
    16x16x32 steps in ascending K: their results must be bit-identical (a dropped,
    repeated or reordered K tile in any ring shows up here)."""
    M, N, K, tA, tB = shape
    case = W.GemmCase(f"ringsweep-{M}x{N}x{K}", M, N, K, transpose_A=tA, transpose_B=tB, relu=1, seed=4950)
    A, B, _ = W.make_inputs(case)
    variants = ["tile256dma", "tile128dma"] + ([] if tA else ["tile64dma", "tile32dma"])
    outs = {}
    for v in variants:
        C, plan, _, _ = run_gpu(case, A, B, None, variant=v)
        outs[v] = C.view(torch.int16).cpu()
        log(f"[case] {case.name} {plan.describe()}")
    ref = outs[variants[0]]
    for v in variants[1:]:
        assert torch.equal(outs[v], ref), f"{v} differs from {variants[0]}"
    assert_within_tolerance(out_values(C), oracle_full(case, A, B, None), case, "ring sweep")
