"""Pins of the 2:4 structured-sparse GEMM oracle: checks against things other than the
oracle itself (the generator's dense construction, a byte-level construction of the
metadata, exact integer products and the separately pinned 16-bit GEMM oracle).  Each
pin raises AssertionError."""
from __future__ import annotations

import numpy as np
import torch

import tlg_workloads as W

TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def pin_sp_expand_matches_generator(O):
    for dt in ("f16", "bf16"):
        case = W.SpCase("pin", 3, 11, 64, ab=dt, seed=7)
        _, Wv, Wm, dense = W.make_sp_inputs(case)
        got = O.sp_expand(11, 64, W.bits16(Wv), Wm.numpy(), dtype=dt)
        assert np.array_equal(got, dense), dt


def pin_sp_metadata_bytewise(O):
    """Group q's two positions written straight into byte q/2 (bits 4(q%2) and 4(q%2)+2)."""
    N, K = 1, 16
    vals = torch.tensor([[1.0, 2.0] * (K // 4)], dtype=torch.float16)
    for q in range(K // 4):
        for p0 in range(4):
            for p1 in range(4):
                Wm = np.zeros((N, K // 8), np.uint8)
                Wm[0, q // 2] = np.uint8((p0 | (p1 << 2)) << (4 * (q % 2)))
                got = O.sp_expand(N, K, W.bits16(vals), Wm)[0]
                want = np.zeros(K)
                for g in range(K // 4):            # every other group has positions 0, 0
                    if g == q:
                        want[4 * g + p0] += 1.0; want[4 * g + p1] += 2.0
                    else:
                        want[4 * g] += 3.0
                assert np.array_equal(got, want), (q, p0, p1)


def pin_sp_matches_16bit_oracle(O):
    """Distinct positions keep every dense weight an operand-type value: the pinned 16-bit
    oracle on the dense weights (B stored [N, K]) gives the same result."""
    for dt, relu in (("f16", 0), ("bf16", 1)):
        case = W.SpCase("pin", 9, 13, 128, ab=dt, relu=relu, seed=8)
        A, Wv, Wm, dense = W.make_sp_inputs(case)
        wbits = W.bits16(torch.as_tensor(dense).to(TDT[dt]))
        assert np.array_equal(torch.as_tensor(dense).to(TDT[dt]).double().numpy(), dense)
        ref = O.gemm(9, 13, 128, W.bits16(A), wbits, ab=dt, c="f32", transpose_B=1, relu=relu)
        got = O.spgemm(9, 13, 128, W.bits16(A), W.bits16(Wv), Wm.numpy(), dtype=dt, relu=relu)
        assert np.array_equal(ref, got), dt


def pin_sp_smallint_integer_matmul(O):
    case = W.SpCase("pin", 7, 10, 256, dist="smallint", seed=9)
    A, Wv, Wm, dense = W.make_sp_inputs(case)
    got = O.spgemm(7, 10, 256, W.bits16(A), W.bits16(Wv), Wm.numpy())
    want = A.double().numpy().astype(np.int64) @ dense.astype(np.int64).T
    assert np.array_equal(got, want.astype(np.float64))


def pin_sp_points_and_rows(O):
    case = W.SpCase("pin", 9, 33, 192, seed=10, relu=1)
    A, Wv, Wm, _ = W.make_sp_inputs(case)
    args = (W.bits16(A), W.bits16(Wv), Wm.numpy())
    full = O.spgemm(9, 33, 192, *args, relu=1)
    ms = np.array([0, 8, 3, 5]); ns = np.array([0, 32, 17, 2])
    assert np.array_equal(full[ms, ns], O.spgemm_points(9, 33, 192, *args, ms, ns, relu=1))
    assert np.array_equal(full[2:7], O.spgemm(9, 33, 192, *args, relu=1, rows=(2, 7)))


ALL_SP_PINS = [pin_sp_expand_matches_generator, pin_sp_metadata_bytewise, pin_sp_matches_16bit_oracle,
               pin_sp_smallint_integer_matmul, pin_sp_points_and_rows]
