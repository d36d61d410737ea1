"""Pins of the 4-bit dequant GEMM oracle: checks against things other than the oracle
itself (the generator's packer and torch's rounding, a byte-level construction of
the packed format, closed forms, exact integer products, and the separately pinned
16-bit GEMM oracle).  Each pin raises AssertionError."""
from __future__ import annotations

import numpy as np
import torch

import tlg_workloads as W

TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _rand(rng, N, K, G, dt, zmax=15):
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    z = rng.integers(0, zmax + 1, size=(N, K // G)).astype(np.uint8)
    s = torch.as_tensor(rng.uniform(0.01, 2.0, size=(N, K // G))).to(TDT[dt])
    return q, z, s


def _expected(q, z, s, G, dt):
    """(q - z) * s exactly in float64, rounded once to the operand type by torch."""
    zz = np.repeat(z.astype(np.float64), G, axis=1)
    ss = np.repeat(s.double().numpy(), G, axis=1)
    return torch.as_tensor((q.astype(np.float64) - zz) * ss).to(TDT[dt]).double().numpy()


def pin_w4_dequant_matches_packer_and_rounding(O):
    rng = np.random.default_rng(1)
    for N, K, G, dt in ((3, 64, 32, "f16"), (5, 256, 128, "bf16"), (2, 512, 64, "f16"), (4, 96, 32, "bf16")):
        q, z, s = _rand(rng, N, K, G, dt)
        got = O.w4_dequant(N, K, G, W.pack_w4(q), W.bits16(s), z, dtype=dt)
        assert np.array_equal(got, _expected(q, z, s, G, dt)), (N, K, G, dt)


def pin_w4_code_positions_bytewise(O):
    """One nonzero code at (n, k), written into the bytes directly from the format's
    statement (code k = 8w + j: byte 4w + shift/8, nibble shift%8), lands at (n, k)."""
    N, K, G = 2, 32, 32
    z = np.zeros((N, 1), np.uint8)
    s = torch.ones((N, 1), dtype=torch.float16)
    for n in range(N):
        for k in range(K):
            b = np.zeros((N, K // 2), np.uint8)
            j = k % 8
            shift = 4 * (j // 2) + (16 if j % 2 else 0)
            b[n, 4 * (k // 8) + shift // 8] = np.uint8(5 << (shift % 8))
            got = O.w4_dequant(N, K, G, b, W.bits16(s), z)
            want = np.zeros((N, K)); want[n, k] = 5.0
            assert np.array_equal(got, want), (n, k)


def pin_w4_codes_at_zero_point_give_zero(O):
    rng = np.random.default_rng(2)
    M, N, K, G = 3, 7, 128, 64
    z = rng.integers(0, 16, size=(N, K // G)).astype(np.uint8)
    q = np.repeat(z, G, axis=1)
    s = torch.as_tensor(rng.uniform(0.1, 3.0, size=(N, K // G))).half()
    A = torch.as_tensor(rng.uniform(-1, 1, size=(M, K))).half()
    out = O.w4gemm(M, N, K, G, W.bits16(A), W.pack_w4(q), W.bits16(s), z)
    assert np.array_equal(out, np.zeros((M, N)))


def pin_w4_smallint_integer_matmul(O):
    """Scales 1 and zero points 8: weights are the integers q - 8, so C is an integer product."""
    for dt in ("f16", "bf16"):
        case = W.W4Case("pin", 6, 9, 256, G=64, ab=dt, dist="smallint", seed=3)
        A, Wq, S, Z, q = W.make_w4_inputs(case)
        out = O.w4gemm(6, 9, 256, 64, W.bits16(A), Wq.numpy(), W.bits16(S), Z.numpy(), dtype=dt)
        want = A.double().numpy().astype(np.int64) @ (q.numpy().astype(np.int64) - 8).T
        assert np.array_equal(out, want.astype(np.float64)), dt


def pin_w4_rounds_ties_to_even(O):
    """(q - z) * s = 3 * (1 + 2^-10) lies halfway between two fp16 values; the weight is the even one."""
    s = torch.tensor([[1.0 + 2.0 ** -10]], dtype=torch.float16)
    q = np.zeros((1, 8), np.uint8); q[0, 0] = 3
    got = O.w4_dequant(1, 8, 8, W.pack_w4(q), W.bits16(s), np.zeros((1, 1), np.uint8))
    assert got[0, 0] == 3.0 + 2.0 ** -8, got[0, 0]


def pin_w4_matches_16bit_oracle(O):
    """The dequantized weights, as 16-bit values through the pinned GEMM oracle (B stored
    [N, K]), give the same result."""
    rng = np.random.default_rng(4)
    for M, N, K, G, dt, relu in ((5, 7, 128, 32, "f16", 0), (4, 3, 256, 128, "bf16", 1)):
        q, z, s = _rand(rng, N, K, G, dt)
        A = torch.as_tensor(rng.uniform(-1, 1, size=(M, K))).to(TDT[dt])
        w = O.w4_dequant(N, K, G, W.pack_w4(q), W.bits16(s), z, dtype=dt)
        wbits = W.bits16(torch.as_tensor(w).to(TDT[dt]))
        ref = O.gemm(M, N, K, W.bits16(A), wbits, ab=dt, c="f32", transpose_B=1, relu=relu)
        got = O.w4gemm(M, N, K, G, W.bits16(A), W.pack_w4(q), W.bits16(s), z, dtype=dt, relu=relu)
        assert np.array_equal(ref, got), (dt, relu)


def pin_w4_points_and_rows(O):
    case = W.W4Case("pin", 9, 33, 192, G=64, seed=5, relu=1)
    A, Wq, S, Z, _ = W.make_w4_inputs(case)
    args = (W.bits16(A), Wq.numpy(), W.bits16(S), Z.numpy())
    full = O.w4gemm(9, 33, 192, 64, *args, relu=1)
    ms = np.array([0, 8, 3, 5]); ns = np.array([0, 32, 17, 2])
    assert np.array_equal(full[ms, ns], O.w4gemm_points(9, 33, 192, 64, *args, ms, ns, relu=1))
    assert np.array_equal(full[2:7], O.w4gemm(9, 33, 192, 64, *args, relu=1, rows=(2, 7)))


ALL_W4_PINS = [pin_w4_dequant_matches_packer_and_rounding, pin_w4_code_positions_bytewise,
               pin_w4_codes_at_zero_point_give_zero, pin_w4_smallint_integer_matmul, pin_w4_rounds_ties_to_even,
               pin_w4_matches_16bit_oracle, pin_w4_points_and_rows]
