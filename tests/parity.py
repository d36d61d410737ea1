"""Shared helpers of the GPU parity tests: run a case through the C-ABI binding and
compare with the oracle on the same seeded bits."""
from __future__ import annotations

import sys

import numpy as np
import torch

import tlg_workloads as W
from oracle import oracle as O

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def out_values(C: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a device fp16/bf16/fp32 tensor (decoded by the oracle's decoder)."""
    Cc = C.detach().cpu().contiguous()
    if Cc.dtype == torch.float32:
        return Cc.numpy().astype(np.float64)
    code = "f16" if Cc.dtype == torch.float16 else "bf16"
    return O.decode(W.bits16(Cc), code).reshape(Cc.shape)


def _placed(X: torch.Tensor, offset: int, dev) -> torch.Tensor:
    """X on the device, starting `offset` elements into a fresh allocation (offset 1 gives a
    base address that is 2-byte but not 4-byte aligned)."""
    if not offset:
        return X.to(dev)
    buf = torch.zeros(offset + X.numel(), dtype=X.dtype, device=dev)
    view = buf[offset:offset + X.numel()].view(X.shape)
    view.copy_(X.to(dev))
    return view


def run_gpu(case: W.GemmCase, A: torch.Tensor, B: torch.Tensor, C_in: torch.Tensor | None,
            variant: str = "auto", guard: int = 0, a_offset: int = 0, b_offset: int = 0):
    """Run through tlg.Gemm; returns (C on device, plan).  With guard > 0, C lives inside a
    larger buffer whose guard bands must come back untouched (checked by the caller).
    a_offset / b_offset place A / B that many elements into their allocations."""
    import tiled_dense_gemm_02_amd as tlg
    dev = torch.device("cuda:0")
    plan = tlg.Gemm(case.M, case.N, case.K, _TORCH[case.ab], _TORCH[case.c],
                    transpose_A=bool(case.transpose_A), transpose_B=bool(case.transpose_B),
                    clear_accum=bool(case.clear_accum), epilogue="relu" if case.relu else "none",
                    variant=variant)
    Ad, Bd = _placed(A, a_offset, dev), _placed(B, b_offset, dev)
    n = case.M * case.N
    if guard:
        esz = 4 if case.c == "f32" else 2
        per_row = 256 // esz                        # keep C 256-byte aligned inside the buffer
        g = ((guard + per_row - 1) // per_row) * per_row
        buf = torch.empty(g + n + g, dtype=_TORCH[case.c], device=dev)
        buf.view(torch.uint8 if esz == 2 else torch.uint8).fill_(0x5A)
        C = buf[g:g + n].view(case.M, case.N)
    else:
        buf, g = None, 0
        C = torch.empty((case.M, case.N), dtype=_TORCH[case.c], device=dev)
    if not case.clear_accum:
        C.copy_(C_in.to(dev))
    plan.run(Ad, Bd, C)
    torch.cuda.synchronize()
    return C, plan, buf, g


def oracle_full(case: W.GemmCase, A, B, C_in):
    cin = None if case.clear_accum else W.raw_bits(C_in)
    return O.gemm(case.M, case.N, case.K, W.bits16(A), W.bits16(B), ab=case.ab, c=case.c,
                  transpose_A=case.transpose_A, transpose_B=case.transpose_B,
                  clear_accum=case.clear_accum, relu=case.relu, C_in_bits=cin)


def oracle_points(case: W.GemmCase, A, B, C_in, ms, ns):
    cin = None if case.clear_accum else W.raw_bits(C_in)
    return O.gemm_points(case.M, case.N, case.K, W.bits16(A), W.bits16(B), ms, ns, ab=case.ab,
                         c=case.c, transpose_A=case.transpose_A, transpose_B=case.transpose_B,
                         clear_accum=case.clear_accum, relu=case.relu, C_in_bits=cin)


def assert_within_tolerance(gpu: np.ndarray, o: np.ndarray, case: W.GemmCase, what: str = ""):
    """|gpu - o| <= 2^-10 |o| + 1e-4 sqrt(K) element by element (bf16 output: 2^-8)."""
    tol = O.tolerance(o, case.K, case.c)
    err = np.abs(gpu - o)
    bad = ~(err <= tol)                      # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what} {case.name}: {int(bad.sum())} of {bad.size} outside tolerance; "
                             f"first {idx.tolist()} gpu={gpu[bad][:5]} oracle={o[bad][:5]}")
    return float(err.max()) if err.size else 0.0


def assert_exact(gpu: np.ndarray, o: np.ndarray, case: W.GemmCase, what: str = ""):
    """gpu == rne_out(oracle) as values (for small-integer inputs)."""
    want = O.rne_out(o.reshape(-1), case.c).reshape(o.shape)
    bad = gpu != want
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what} {case.name}: {int(bad.sum())} inexact; first {idx.tolist()} "
                             f"gpu={gpu[bad][:5]} want={want[bad][:5]}")
