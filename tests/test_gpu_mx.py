"""GPU parity of the block-scaled FP8 GEMM (tlg_gemm_run_mx) against the CPU MX oracle
on the same seeded bytes.  Tolerance |gpu - oracle| <= 2^-10 |oracle| + 1e-4 sqrt(K)
(the products of FP8 elements and power-of-two scales are exact in fp32, so only the
fp32 accumulation and the output rounding separate the two); exact after the oracle's
own rounding for small-integer elements."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import tlg_workloads as W
from oracle import oracle as O
from parity import assert_exact, assert_within_tolerance, log, out_values

pytestmark = pytest.mark.gpu

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import tiled_dense_gemm_02_amd as tlg
    tlg.load_library()
    yield


def _np(x):
    return None if x is None else x.numpy()


def _run(case: W.MxCase, A, SA, B, SB, C_in, guard=0):
    import tiled_dense_gemm_02_amd as tlg
    dev = torch.device("cuda:0")
    plan = tlg.Gemm(case.M, case.N, case.K, case.fmt, _TORCH[case.c], transpose_B=True,
                    clear_accum=bool(case.clear_accum), epilogue="relu" if case.relu else "none")
    n = case.M * case.N
    if guard:
        buf = torch.empty(guard + n + guard, dtype=_TORCH[case.c], device=dev)
        buf.view(torch.uint8).fill_(0x5A)
        C = buf[guard:guard + n].view(case.M, case.N)
    else:
        buf, C = None, torch.empty((case.M, case.N), dtype=_TORCH[case.c], device=dev)
    if not case.clear_accum:
        C.copy_(C_in.to(dev))
    plan.run_mx(A.to(dev), SA.to(dev), B.to(dev), SB.to(dev), C)
    torch.cuda.synchronize()
    if guard:
        raw = buf.view(torch.uint8).cpu()
        esz = 4 if case.c == "f32" else 2
        assert bool((raw[:guard * esz] == 0x5A).all()) and bool((raw[(guard + n) * esz:] == 0x5A).all()), \
            "store outside C"
    return C, plan


def _oracle(case, A, SA, B, SB, C_in, rows=None):
    cin = None if case.clear_accum else W.raw_bits(C_in)
    return O.mxgemm(case.M, case.N, case.K, _np(A), _np(SA), _np(B), _np(SB), fmt_a=case.fmt, fmt_b=case.fmt,
                    c=case.c, clear_accum=case.clear_accum, relu=case.relu, C_in_bits=cin, rows=rows)


def _full_check(case, guard=0, exact=False):
    log(f"[case] {case.name} M={case.M} N={case.N} K={case.K} fmt={case.fmt} c={case.c} relu={case.relu} "
        f"clear={case.clear_accum} dist={case.dist}")
    A, SA, B, SB, C_in = W.make_mx_inputs(case)
    C, plan = _run(case, A, SA, B, SB, C_in, guard=guard)
    gpu = out_values(C)
    o = _oracle(case, A, SA, B, SB, C_in)
    if exact:
        assert_exact(gpu, o, case, plan.describe())
    else:
        err = assert_within_tolerance(gpu, o, case, plan.describe())
        log(f"    max|err| = {err:.3e}  ({plan.describe()})")
    return plan


def test_mx1_relu_256():
    plan = _full_check(W.MX_CONFIGS["mx1"], guard=4096)
    assert plan.info.variant == 9 and plan.info.k_tiles == 2


def test_mx2_ragged_e5m2_f32out():
    _full_check(W.MX_CONFIGS["mx2"], guard=4096)


def test_mx3_8192_sampled():
    case = W.MX_CONFIGS["mx3"]
    log(f"[case] {case.name} sampled")
    A, SA, B, SB, _ = W.make_mx_inputs(case)
    C, plan = _run(case, A, SA, B, SB, None)
    ms, ns = W.sample_points(case.M, case.N, 2048)
    o = O.mxgemm_points(case.M, case.N, case.K, _np(A), _np(SA), _np(B), _np(SB), ms, ns, fmt_a=case.fmt,
                        fmt_b=case.fmt, c=case.c)
    gpu = out_values(C)
    err = assert_within_tolerance(gpu[ms, ns], o, case, plan.describe())
    assert np.isfinite(gpu).all()
    log(f"    max|err| = {err:.3e}  ({plan.describe()})")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("c", ["f32", "f16"])
def test_mx_small_integers_exact(fmt, c):
    case = W.MxCase("mx-smallint", 300, 264, 384, fmt=fmt, c=c, relu=1, dist="smallint", seed=77)
    _full_check(case, exact=True, guard=1024)


@pytest.mark.parametrize("shape", [(1, 1, 128), (17, 33, 128), (255, 257, 256), (256, 256, 0), (513, 130, 640)])
def test_mx_edges(shape):
    M, N, K = shape
    for it, (fmt, c, relu) in enumerate((("e4m3", "bf16", 1), ("e5m2", "f16", 0))):
        case = W.MxCase(f"mx-edge{M}x{N}x{K}", M, N, K, fmt=fmt, c=c, relu=relu, dist="uniform", seed=600 + it)
        if K == 0:
            case = case.with_(clear_accum=0)
        _full_check(case, guard=1024)


def test_mx_accumulate_onto_c():
    for fmt, c in (("e4m3", "f16"), ("e5m2", "f32")):
        case = W.MxCase(f"mx-accum-{fmt}-{c}", 264, 200, 256, fmt=fmt, c=c, clear_accum=0, relu=1, seed=31)
        _full_check(case)


def test_mx_deterministic_and_plain_run_refused():
    import tiled_dense_gemm_02_amd as tlg
    case = W.MX_CONFIGS["mx1"].with_(name="mx-determinism", M=512, N=512, K=1024)
    A, SA, B, SB, _ = W.make_mx_inputs(case)
    C1, plan = _run(case, A, SA, B, SB, None)
    C2, _ = _run(case, A, SA, B, SB, None)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    Ad, Bd = A.cuda(), B.cuda()
    with pytest.raises(tlg.TlgError):
        plan.run(Ad.view(torch.float8_e4m3fn), Bd.view(torch.float8_e4m3fn), C1)   # scales are required


# ---------------------------------------------------------------- MXFP4 (E2M1 elements, two per byte)
def test_mxfp4_mx4_relu_256():
    plan = _full_check(W.MX_CONFIGS["mx4"], guard=4096)
    assert plan.info.variant == 9 and plan.info.block_k == 256 and plan.info.k_tiles == 1


def test_mxfp4_mx5_ragged_f32out():
    _full_check(W.MX_CONFIGS["mx5"], guard=4096)


def test_mxfp4_mx6_8192_sampled():
    case = W.MX_CONFIGS["mx6"]
    log(f"[case] {case.name} sampled")
    A, SA, B, SB, _ = W.make_mx_inputs(case)
    C, plan = _run(case, A, SA, B, SB, None)
    ms, ns = W.sample_points(case.M, case.N, 2048)
    o = O.mxgemm_points(case.M, case.N, case.K, _np(A), _np(SA), _np(B), _np(SB), ms, ns, fmt_a=case.fmt,
                        fmt_b=case.fmt, c=case.c)
    gpu = out_values(C)
    err = assert_within_tolerance(gpu[ms, ns], o, case, plan.describe())
    assert np.isfinite(gpu).all()
    log(f"    max|err| = {err:.3e}  ({plan.describe()})")


@pytest.mark.parametrize("K", [384, 512])
@pytest.mark.parametrize("c", ["f32", "f16"])
def test_mxfp4_small_integers_exact(K, c):
    """K = 384: the last K tile of 256 FP4 elements is half full (zero fill of the data
    and of the second scale plane)."""
    case = W.MxCase("mxfp4-smallint", 300, 264, K, fmt="e2m1", c=c, relu=1, dist="smallint", seed=78)
    _full_check(case, exact=True, guard=1024)


@pytest.mark.parametrize("shape", [(1, 1, 128), (17, 33, 128), (255, 257, 256), (256, 256, 0), (513, 130, 640)])
def test_mxfp4_edges(shape):
    M, N, K = shape
    for it, (c, relu) in enumerate((("bf16", 1), ("f16", 0))):
        case = W.MxCase(f"mxfp4-edge{M}x{N}x{K}", M, N, K, fmt="e2m1", c=c, relu=relu, dist="uniform", seed=610 + it)
        if K == 0:
            case = case.with_(clear_accum=0)
        _full_check(case, guard=1024)


def test_mxfp4_accumulate_onto_c():
    for c in ("f16", "f32"):
        case = W.MxCase(f"mxfp4-accum-{c}", 264, 200, 384, fmt="e2m1", c=c, clear_accum=0, relu=1, seed=32)
        _full_check(case)
