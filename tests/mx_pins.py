"""Pins of the block-scaled (MX) GEMM oracle: checks against things other than the
oracle itself (torch's FP8 / E8M0 conversions, exact rational sums, closed forms,
and the separately pinned 16-bit GEMM oracle).  Each pin raises AssertionError."""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

TORCH_FMT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2, "e8m0": torch.float8_e8m0fnu}


def torch_decode(bytes_, fmt) -> np.ndarray:
    """Element or scale values through torch's own FP8 / E8M0 conversions."""
    t = torch.as_tensor(np.ascontiguousarray(bytes_, dtype=np.uint8)).view(TORCH_FMT[fmt])
    return t.to(torch.float64).numpy()


def _rand_mx(rng, rows, K, fmt, lo=120, hi=135):
    """Random finite element bytes and scale bytes in [lo, hi]."""
    nan_free = [b for b in range(256) if np.isfinite(torch_decode([b], fmt)[0])]
    elems = rng.choice(np.asarray(nan_free, dtype=np.uint8), size=(rows, K))
    scales = rng.integers(lo, hi + 1, size=(rows, K // 32)).astype(np.uint8)
    return elems, scales


def _exact(elems, scales, fmt, r, k) -> Fraction:
    e = Fraction(float(torch_decode([elems[r, k]], fmt)[0]))
    return e * Fraction(2) ** (int(scales[r, k // 32]) - 127)


def pin_mx_decode_exhaustive(O):
    codes = np.arange(256, dtype=np.uint8)
    for fmt in ("e4m3", "e5m2", "e8m0"):
        mine = O.mx_decode(codes, fmt)
        ref = torch_decode(codes, fmt)
        assert np.array_equal(np.isnan(mine), np.isnan(ref)), fmt
        ok = ~np.isnan(ref)
        assert np.array_equal(mine[ok], ref[ok]), fmt
        # the sign of zero too
        assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok])), fmt


def pin_mx_fraction_bruteforce(O):
    rng = np.random.default_rng(11)
    for fmt_a, fmt_b, c, clear, relu in (("e4m3", "e4m3", "f16", 1, 0), ("e5m2", "e4m3", "f32", 0, 1),
                                         ("e4m3", "e5m2", "bf16", 1, 1)):
        M, N, K = 3, 2, 64
        A, SA = _rand_mx(rng, M, K, fmt_a)
        B, SB = _rand_mx(rng, N, K, fmt_b)
        Cin = None
        if not clear:
            Cin = rng.integers(0, 1 << 16, size=(M, N)).astype(np.uint32) & 0x3f7fffff   # finite fp32 bits
        out = O.mxgemm(M, N, K, A, SA, B, SB, fmt_a=fmt_a, fmt_b=fmt_b, c=c, clear_accum=clear, relu=relu,
                       C_in_bits=None if clear else (Cin if c == "f32" else Cin.astype(np.uint16)))
        for m in range(M):
            for n in range(N):
                s = Fraction(0)
                if not clear:
                    bits = int(Cin[m, n]) if c == "f32" else int(Cin[m, n]) & 0xffff
                    s = Fraction(float(O.decode(np.array([bits], np.uint32), c)[0]))
                for k in range(K):
                    s += _exact(A, SA, fmt_a, m, k) * _exact(B, SB, fmt_b, n, k)
                if relu:
                    s = max(s, Fraction(0))
                got = Fraction(float(out[m, n]))
                assert abs(got - s) <= abs(s) * Fraction(1, 2 ** 50), (fmt_a, fmt_b, m, n)


def pin_mx_block_scales_closed_form(O):
    """All elements 1.0: C[m,n] = 32 * sum_b 2^(SA[m,b]-127) * 2^(SB[n,b]-127)."""
    M, N, K = 4, 3, 256
    one = {"e4m3": 0x38, "e5m2": 0x3C}
    for fmt in ("e4m3", "e5m2"):
        A = np.full((M, K), one[fmt], np.uint8)
        B = np.full((N, K), one[fmt], np.uint8)
        SA = (120 + (np.arange(M)[:, None] * 3 + np.arange(K // 32)[None, :] * 5) % 13).astype(np.uint8)
        SB = (121 + (np.arange(N)[:, None] * 7 + np.arange(K // 32)[None, :]) % 11).astype(np.uint8)
        out = O.mxgemm(M, N, K, A, SA, B, SB, fmt_a=fmt, fmt_b=fmt, c="f32")
        want = 32.0 * np.exp2(SA.astype(np.float64)[:, None, :] + SB.astype(np.float64)[None, :, :] - 254).sum(2)
        assert np.array_equal(out, want), fmt


def pin_mx_smallint_integer_matmul(O):
    """Scales 127 (x1): the result is the integer matrix product, exactly."""
    rng = np.random.default_rng(12)
    M, N, K = 17, 9, 96
    for fmt in ("e4m3", "e5m2"):
        ia = rng.integers(-4, 5, size=(M, K))
        ib = rng.integers(-4, 5, size=(N, K))
        A = torch.as_tensor(ia, dtype=torch.float32).to(TORCH_FMT[fmt]).view(torch.uint8).numpy()
        B = torch.as_tensor(ib, dtype=torch.float32).to(TORCH_FMT[fmt]).view(torch.uint8).numpy()
        S1 = np.full((M, K // 32), 127, np.uint8)
        S2 = np.full((N, K // 32), 127, np.uint8)
        out = O.mxgemm(M, N, K, A, S1, B, S2, fmt_a=fmt, fmt_b=fmt, c="f32")
        assert np.array_equal(out, (ia @ ib.T).astype(np.float64)), fmt
        # one scale step up on A doubles everything
        out2 = O.mxgemm(M, N, K, A, S1 + 1, B, S2, fmt_a=fmt, fmt_b=fmt, c="f32")
        assert np.array_equal(out2, 2.0 * out), fmt


def pin_mx_matches_16bit_oracle(O):
    """MX operands whose scaled values are exact fp16 numbers give the same result as
    the 16-bit GEMM oracle on those numbers (B stored [N, K])."""
    rng = np.random.default_rng(13)
    M, N, K = 5, 7, 128
    for fmt in ("e4m3", "e5m2"):
        lo, hi = (120, 134) if fmt == "e4m3" else (124, 127)   # keeps E5M2 values inside fp16 range
        A, SA = _rand_mx(rng, M, K, fmt, lo, hi)
        B, SB = _rand_mx(rng, N, K, fmt, lo, hi)
        va = torch_decode(A, fmt) * np.exp2(np.repeat(SA.astype(np.float64), 32, axis=1) - 127)
        vb = torch_decode(B, fmt) * np.exp2(np.repeat(SB.astype(np.float64), 32, axis=1) - 127)
        ha = torch.as_tensor(va).to(torch.float16)
        hb = torch.as_tensor(vb).to(torch.float16)
        assert np.array_equal(ha.double().numpy(), va) and np.array_equal(hb.double().numpy(), vb), fmt
        bits_a = ha.view(torch.int16).numpy().view(np.uint16)
        bits_b = hb.view(torch.int16).numpy().view(np.uint16)
        ref = O.gemm(M, N, K, bits_a, bits_b, ab="f16", c="f32", transpose_B=1)
        got = O.mxgemm(M, N, K, A, SA, B, SB, fmt_a=fmt, fmt_b=fmt, c="f32")
        assert np.array_equal(ref, got), fmt


def pin_mx_points_and_rows(O):
    rng = np.random.default_rng(14)
    M, N, K = 33, 21, 160
    A, SA = _rand_mx(rng, M, K, "e4m3")
    B, SB = _rand_mx(rng, N, K, "e5m2")
    full = O.mxgemm(M, N, K, A, SA, B, SB, fmt_a="e4m3", fmt_b="e5m2", relu=1)
    ms = np.array([0, 32, 5, 17]); ns = np.array([0, 20, 13, 2])
    pts = O.mxgemm_points(M, N, K, A, SA, B, SB, ms, ns, fmt_a="e4m3", fmt_b="e5m2", relu=1)
    assert np.array_equal(full[ms, ns], pts)
    part = O.mxgemm(M, N, K, A, SA, B, SB, fmt_a="e4m3", fmt_b="e5m2", relu=1, rows=(10, 20), nthreads=3)
    assert np.array_equal(part, full[10:20])


ALL_MX_PINS = [pin_mx_decode_exhaustive, pin_mx_fraction_bruteforce, pin_mx_block_scales_closed_form,
               pin_mx_smallint_integer_matmul, pin_mx_matches_16bit_oracle, pin_mx_points_and_rows]
