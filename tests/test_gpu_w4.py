"""GPU parity of the 4-bit dequant GEMM (tlg_gemm_w4) against the CPU oracle on the same
seeded bits.  The dequantized weights are identical on both sides (a single rounding
of (q - z) * s), so only the fp32 accumulation and the output rounding separate them:
|gpu - o| <= 2^-10 |o| + 1e-4 sqrt(K) max|w| max|a| (2^-8 for bf16 output); exact for
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


def _run(case: W.W4Case, A, Wq, S, Z, guard: int = 0):
    import tiled_dense_gemm_02_amd as tlg
    dev = _device()
    n = case.M * case.N
    if guard:
        buf = torch.empty(guard + n + guard, dtype=_T[case.c], device=dev)
        buf.view(torch.uint8).fill_(0x5A)
        C = buf[guard:guard + n].view(case.M, case.N)
    else:
        buf, C = None, torch.empty((case.M, case.N), dtype=_T[case.c], device=dev)
    tlg.gemm_w4(A.to(dev), Wq.to(dev), S.to(dev), Z.to(dev), C, group=case.G,
                epilogue="relu" if case.relu else "none")
    torch.cuda.synchronize()
    if guard:
        g = buf.view(torch.uint8)
        esz = buf.element_size()
        assert bool((g[:guard * esz] == 0x5A).all()) and bool((g[(guard + n) * esz:] == 0x5A).all()), "guard written"
    return C


def _tol(case, o, A, wmax):
    rel = 2.0 ** -8 if case.c == "bf16" else 2.0 ** -10
    amax = float(A.float().abs().max()) if A.numel() else 0.0
    return rel * np.abs(o) + 1e-4 * np.sqrt(max(case.K, 1)) * max(wmax * amax, 1e-30)


def _check(case, gpu, o, A, wmax, exact=False):
    if exact:
        want = O.rne_out(o.reshape(-1), case.c).reshape(o.shape)
        bad = gpu != want
    else:
        bad = ~(np.abs(gpu - o) <= _tol(case, o, A, wmax))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{case.name}: {int(bad.sum())} of {bad.size} bad; first {idx.tolist()} "
                             f"gpu={gpu[bad][:5]} oracle={o[bad][:5]}")
    return float(np.abs(gpu - o).max()) if o.size else 0.0


def _full(case: W.W4Case, guard=0, exact=False):
    log(f"[case] {case.name} M={case.M} N={case.N} K={case.K} G={case.G} {case.ab}->{case.c} relu={case.relu}")
    A, Wq, S, Z, _ = W.make_w4_inputs(case)
    C = _run(case, A, Wq, S, Z, guard)
    o = O.w4gemm(case.M, case.N, case.K, case.G, W.bits16(A), Wq.numpy(), W.bits16(S), Z.numpy(), dtype=case.ab,
                 relu=case.relu)
    wmax = float(np.abs(O.w4_dequant(case.N, case.K, case.G, Wq.numpy(), W.bits16(S), Z.numpy(),
                                     dtype=case.ab)).max()) if case.K else 0.0
    err = _check(case, out_values(C), o, A, wmax, exact)
    log(f"    max|err| = {err:.3e}")


def test_w4b_ragged_bf16_f32out_relu():
    _full(W.W4_CONFIGS["w4b"], guard=1024)


def test_w4c_three_row_tiles_groups_of_32():
    _full(W.W4_CONFIGS["w4c"])


def test_w4a_decode_shape_sampled():
    case = W.W4_CONFIGS["w4a"]
    log(f"[case] {case.name} sampled")
    A, Wq, S, Z, _ = W.make_w4_inputs(case)
    C = out_values(_run(case, A, Wq, S, Z))
    ms, ns = W.sample_points(case.M, case.N, 512)
    o = O.w4gemm_points(case.M, case.N, case.K, case.G, W.bits16(A), Wq.numpy(), W.bits16(S), Z.numpy(), ms, ns)
    wmax = 15.0 * float(S.float().abs().max())
    err = _check(case, C[ms, ns], o, A, wmax)
    assert np.isfinite(C).all()
    log(f"    max|err| = {err:.3e}")


@pytest.mark.parametrize("ab", ["f16", "bf16"])
@pytest.mark.parametrize("c", ["f32", "f16"])
def test_small_integers_exact(ab, c):
    _full(W.W4Case(f"w4-smallint-{ab}-{c}", 19, 200, 1024, G=128, ab=ab, c=c, relu=1, dist="smallint", seed=71),
          guard=512, exact=True)


@pytest.mark.parametrize("ab", ["f16", "bf16"])
def test_w4a_small_integers_exact_full_size(ab):
    """The decode shape 16 x 16384 x 8192 in full, exactly, with a scale 2^-1..2^2 and a
    zero point 0..15 of its own for every row and group of 128: each weight is a multiple
    of 1/2 of magnitude at most 60 and A holds integers in [-4, 4], so every partial sum
    is a multiple of 1/2 below 2^21 (exact in fp32), and a scale or zero point read from
    the wrong row or group changes the result."""
    case = W.W4Case(f"w4a-int-groups-{ab}", 16, 16384, 8192, G=128, ab=ab, c="f32", dist="smallint_groups",
                    seed=7300 + (ab == "bf16"))
    log(f"[case] full-size {case.name} exact")
    A, Wq, S, Z, _ = W.make_w4_inputs(case)
    gpu = out_values(_run(case, A, Wq, S, Z))
    o = O.w4gemm(case.M, case.N, case.K, case.G, W.bits16(A), Wq.numpy(), W.bits16(S), Z.numpy(), dtype=case.ab)
    _check(case, gpu, o, A, 0.0, exact=True)


EDGES = [(1, 1, 32, 32), (1, 64, 32, 32), (16, 65, 64, 64), (17, 130, 544, 32), (3, 257, 1536, 256),
         (2, 129, 8160, 32), (4, 100, 0, 32)]


@pytest.mark.parametrize("shape", EDGES, ids=lambda s: "x".join(map(str, s)))
def test_edges(shape):
    M, N, K, G = shape
    for it, (ab, c, relu) in enumerate((("f16", "f16", 0), ("bf16", "bf16", 1))):
        _full(W.W4Case(f"w4-edge{M}x{N}x{K}g{G}", M, N, K, G=G, ab=ab, c=c, relu=relu, seed=800 + it), guard=256)


def test_deterministic():
    case = W.W4_CONFIGS["w4c"].with_(name="w4-determinism", M=16, N=2048, K=2048)
    A, Wq, S, Z, _ = W.make_w4_inputs(case)
    a = _run(case, A, Wq, S, Z)
    b = _run(case, A, Wq, S, Z)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_error_paths_enqueue_nothing():
    import tiled_dense_gemm_02_amd as tlg
    dev = _device()
    A = torch.zeros((16, 256), dtype=torch.float16, device=dev)
    Wq = torch.zeros((64, 128), dtype=torch.uint8, device=dev)
    S = torch.ones((64, 2), dtype=torch.float16, device=dev)
    Z = torch.zeros((64, 2), dtype=torch.uint8, device=dev)
    C = torch.full((16, 64), 7.0, dtype=torch.float16, device=dev)
    pa, pw, ps, pz, pc = (t.data_ptr() for t in (A, Wq, S, Z, C))
    f16 = torch.float16
    assert tlg.gemm_w4_ptrs(pa + 8, pw, ps, pz, pc, 16, 64, 256, 128, f16, f16) == -4     # A misaligned
    assert tlg.gemm_w4_ptrs(pa, pw, ps, pz, pa, 16, 64, 256, 128, f16, f16) == -1         # C overlaps A
    assert tlg.gemm_w4_ptrs(pa, pw, ps, pz, pc, 16, 64, 256, 96, f16, f16) == -1          # group 96
    assert tlg.gemm_w4_ptrs(pa, pw, ps, pz, pc, 16, 64, 256 * 257, 256, f16, f16) == -2   # K/G > 255
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())
