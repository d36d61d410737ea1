"""GPU parity of the 2:4 structured-sparse GEMM (tlg_gemm_sp) against the CPU oracle on the
same seeded bits: |gpu - o| <= 2^-10 |o| + 1e-4 sqrt(K) (2^-8 for bf16 output), exact for
small-integer cases."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import tlg_workloads as W
from oracle import oracle as O
from parity import log, out_values

pytestmark = pytest.mark.gpu
_T = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _run(case, A, Wv, Wm, guard=0):
    import tiled_dense_gemm_02_amd as tlg
    dev = _device()
    n = case.M * case.N
    if guard:
        buf = torch.empty(guard + n + guard, dtype=_T[case.c], device=dev)
        buf.view(torch.uint8).fill_(0x5A)
        C = buf[guard:guard + n].view(case.M, case.N)
    else:
        buf, C = None, torch.empty((case.M, case.N), dtype=_T[case.c], device=dev)
    tlg.gemm_sp(A.to(dev), Wv.to(dev), Wm.to(dev), C, epilogue="relu" if case.relu else "none")
    torch.cuda.synchronize()
    if guard:
        g = buf.view(torch.uint8)
        esz = buf.element_size()
        assert bool((g[:guard * esz] == 0x5A).all()) and bool((g[(guard + n) * esz:] == 0x5A).all()), "guard written"
    return C


def _check(case, gpu, o, exact=False):
    if exact:
        bad = gpu != O.rne_out(o.reshape(-1), case.c).reshape(o.shape)
    else:
        bad = ~(np.abs(gpu - o) <= O.tolerance(o, case.K, case.c))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{case.name}: {int(bad.sum())} of {bad.size} bad; first {idx.tolist()} "
                             f"gpu={gpu[bad][:5]} oracle={o[bad][:5]}")
    return float(np.abs(gpu - o).max()) if o.size else 0.0


def _full(case, guard=0, exact=False, inputs=None):
    log(f"[case] {case.name} M={case.M} N={case.N} K={case.K} {case.ab}->{case.c} relu={case.relu}")
    A, Wv, Wm, _ = inputs if inputs is not None else W.make_sp_inputs(case)
    C = _run(case, A, Wv, Wm, guard)
    o = O.spgemm(case.M, case.N, case.K, W.bits16(A), W.bits16(Wv), Wm.numpy(), dtype=case.ab, relu=case.relu)
    err = _check(case, out_values(C), o, exact)
    log(f"    max|err| = {err:.3e}")


def test_sp1_relu_256():
    _full(W.SP_CONFIGS["sp1"])


def test_sp2_ragged_bf16_f32out():
    _full(W.SP_CONFIGS["sp2"], guard=1024)


def test_sp3_8192_sampled():
    case = W.SP_CONFIGS["sp3"]
    log(f"[case] {case.name} sampled")
    A, Wv, Wm, _ = W.make_sp_inputs(case)
    C = out_values(_run(case, A, Wv, Wm))
    ms, ns = W.sample_points(case.M, case.N, 1024)
    o = O.spgemm_points(case.M, case.N, case.K, W.bits16(A), W.bits16(Wv), Wm.numpy(), ms, ns)
    err = _check(case, C[ms, ns], o)
    assert np.isfinite(C).all()
    log(f"    max|err| = {err:.3e}")


@pytest.mark.parametrize("ab", ["f16", "bf16"])
@pytest.mark.parametrize("c", ["f32", "f16"])
def test_small_integers_exact(ab, c):
    _full(W.SpCase(f"sp-smallint-{ab}-{c}", 300, 264, 384, ab=ab, c=c, relu=1, dist="smallint", seed=91),
          guard=512, exact=True)


@pytest.mark.parametrize("shape", [(1, 1, 64), (17, 33, 64), (255, 257, 128), (513, 130, 640), (40, 300, 0)],
                         ids=lambda s: "x".join(map(str, s)))
def test_edges(shape):
    M, N, K = shape
    for it, (ab, c, relu) in enumerate((("f16", "bf16", 1), ("bf16", "f16", 0))):
        _full(W.SpCase(f"sp-edge{M}x{N}x{K}", M, N, K, ab=ab, c=c, relu=relu, seed=900 + it), guard=512)


def test_repeated_positions_add():
    """Both stored values of a group at the same position (their sum is the weight there)."""
    case = W.SpCase("sp-repeat", 64, 96, 256, seed=95)
    A, Wv, _, _ = W.make_sp_inputs(case)
    rng = np.random.default_rng(96)
    pos = rng.integers(0, 4, size=(case.N, case.K // 2))
    Wm = torch.from_numpy(W.compress_24(pos))
    _full(case, inputs=(A, Wv, Wm, None))


def test_deterministic():
    case = W.SP_CONFIGS["sp2"].with_(name="sp-determinism", ab="f16", c="f16", M=512, N=512, K=1024)
    A, Wv, Wm, _ = W.make_sp_inputs(case)
    a = _run(case, A, Wv, Wm)
    b = _run(case, A, Wv, Wm)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_error_paths_enqueue_nothing():
    import tiled_dense_gemm_02_amd as tlg
    dev = _device()
    A = torch.zeros((64, 128), dtype=torch.float16, device=dev)
    Wv = torch.zeros((64, 64), dtype=torch.float16, device=dev)
    Wm = torch.zeros((64, 16), dtype=torch.uint8, device=dev)
    C = torch.full((64, 64), 7.0, dtype=torch.float16, device=dev)
    pa, pv, pm, pc = (t.data_ptr() for t in (A, Wv, Wm, C))
    f16 = torch.float16
    assert tlg.gemm_sp_ptrs(pa + 8, pv, pm, pc, 64, 64, 128, f16, f16) == -4     # A misaligned
    assert tlg.gemm_sp_ptrs(pa, pv, pm, pa, 64, 64, 128, f16, f16) == -1         # C overlaps A
    assert tlg.gemm_sp_ptrs(pa, pv, pm, pc, 64, 64, 96, f16, f16) == -2          # K % 64
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())
