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


# ---------------------------------------------------------------- MXFP4 (E2M1 elements, two per byte)
import os

_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "e2m1_values.txt")


def e2m1_table():
    """code -> value from the format's published value table (tests/golden/e2m1_values.txt)."""
    t = {}
    for line in open(_GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            c, v = line.split()
            t[int(c, 16)] = float(v)
    assert sorted(t) == list(range(16))
    return t


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """[rows, K] codes 0..15 -> [rows, K/2] bytes, element 2i in the low nibble of byte i."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def e2m1_as_e4m3_bits(codes: np.ndarray) -> np.ndarray:
    """The same values as E4M3 bytes, by moving the bit fields (E2M1 exponent field e > 0
    -> E4M3 exponent field e + 6, fraction bit -> the top fraction bit; the one
    subnormal magnitude 0.5 = 2^-1 -> exponent field 6)."""
    c = np.asarray(codes, dtype=np.uint8)
    sign = (c >> 3) & 1
    e = (c >> 1) & 3
    f = c & 1
    mag = np.where(e > 0, ((e + 6) << 3) | (f << 2), np.where(f == 1, 6 << 3, 0))
    return ((sign << 7) | mag).astype(np.uint8)


def pin_e2m1_decode_table(O):
    """All 16 codes against the published value table, and through torch's E4M3 decode
    of the same values moved into E4M3 bit fields."""
    codes = np.arange(16, dtype=np.uint8)
    mine = O.mx_decode(codes, "e2m1")
    t = e2m1_table()
    want = np.array([t[c] for c in range(16)])
    assert np.array_equal(mine, want) and np.array_equal(np.signbit(mine), np.signbit(want))
    via = torch_decode(e2m1_as_e4m3_bits(codes), "e4m3")
    assert np.array_equal(mine, via)


def _rand_e2m1(rng, rows, K, lo=120, hi=135):
    codes = rng.integers(0, 16, size=(rows, K)).astype(np.uint8)
    scales = rng.integers(lo, hi + 1, size=(rows, K // 32)).astype(np.uint8)
    return codes, scales


def pin_mxfp4_fraction_bruteforce(O):
    """Exact rational sums with element values from the published table, for E2M1 x E2M1
    and E2M1 x E4M3 operands, with and without accumulation and ReLU."""
    rng = np.random.default_rng(21)
    t = e2m1_table()
    for fmt_b, c, clear, relu in (("e2m1", "f32", 1, 0), ("e2m1", "f16", 0, 1), ("e4m3", "bf16", 1, 1)):
        M, N, K = 3, 4, 96
        ca, SA = _rand_e2m1(rng, M, K)
        if fmt_b == "e2m1":
            cb, SB = _rand_e2m1(rng, N, K)
            Bb = pack_e2m1(cb)
            bval = lambda n, k: Fraction(t[int(cb[n, k])])
        else:
            Bb, SB = _rand_mx(rng, N, K, "e4m3")
            bval = lambda n, k: Fraction(float(torch_decode([Bb[n, k]], "e4m3")[0]))
        Cin = None
        if not clear:
            Cin = (rng.integers(0, 1 << 14, size=(M, N)).astype(np.uint32) & 0x3bff)   # finite fp16 bits
        out = O.mxgemm(M, N, K, pack_e2m1(ca), SA, Bb, SB, fmt_a="e2m1", fmt_b=fmt_b, c=c, clear_accum=clear,
                       relu=relu, C_in_bits=None if clear else Cin.astype(np.uint16))
        for m in range(M):
            for n in range(N):
                s = Fraction(0)
                if not clear:
                    s = Fraction(float(O.decode(np.array([int(Cin[m, n])], np.uint32), c)[0]))
                for k in range(K):
                    a = Fraction(t[int(ca[m, k])]) * Fraction(2) ** (int(SA[m, k // 32]) - 127)
                    b = bval(n, k) * Fraction(2) ** (int(SB[n, k // 32]) - 127)
                    s += a * b
                if relu:
                    s = max(s, Fraction(0))
                assert abs(Fraction(float(out[m, n])) - s) <= abs(s) * Fraction(1, 2 ** 50), (fmt_b, m, n)


def pin_mxfp4_matches_e4m3_oracle(O):
    """Packed E2M1 operands give exactly the result of the E4M3 oracle on the same values
    stored one per byte (unpacked here, low nibble first, and moved into E4M3 fields)."""
    rng = np.random.default_rng(22)
    M, N, K = 9, 7, 256
    ca, SA = _rand_e2m1(rng, M, K)
    cb, SB = _rand_e2m1(rng, N, K)
    got = O.mxgemm(M, N, K, pack_e2m1(ca), SA, pack_e2m1(cb), SB, fmt_a="e2m1", fmt_b="e2m1", c="f32", relu=1)
    ref = O.mxgemm(M, N, K, e2m1_as_e4m3_bits(ca), SA, e2m1_as_e4m3_bits(cb), SB, fmt_a="e4m3", fmt_b="e4m3",
                   c="f32", relu=1)
    assert np.array_equal(got, ref)
    pts = O.mxgemm_points(M, N, K, pack_e2m1(ca), SA, pack_e2m1(cb), SB, np.array([0, 8, 3]), np.array([6, 0, 2]),
                          fmt_a="e2m1", fmt_b="e2m1", c="f32", relu=1)
    assert np.array_equal(pts, ref[[0, 8, 3], [6, 0, 2]])


def pin_mxfp4_closed_form(O):
    """All elements 1.0 (code 2, byte 0x22): C[m,n] = 32 * sum_b 2^(SA[m,b]-127) 2^(SB[n,b]-127);
    all elements 6.0 (code 7) on one side: six times that."""
    M, N, K = 3, 5, 128
    SA = (121 + (np.arange(M)[:, None] * 5 + np.arange(K // 32)[None, :] * 3) % 9).astype(np.uint8)
    SB = (124 + (np.arange(N)[:, None] * 2 + np.arange(K // 32)[None, :]) % 7).astype(np.uint8)
    ones = np.full((M, K // 2), 0x22, np.uint8)
    want = 32.0 * np.exp2(SA.astype(np.float64)[:, None, :] + SB.astype(np.float64)[None, :, :] - 254).sum(2)
    out = O.mxgemm(M, N, K, ones, SA, np.full((N, K // 2), 0x22, np.uint8), SB, fmt_a="e2m1", fmt_b="e2m1", c="f32")
    assert np.array_equal(out, want)
    out6 = O.mxgemm(M, N, K, np.full((M, K // 2), 0x77, np.uint8), SA, np.full((N, K // 2), 0x22, np.uint8), SB,
                    fmt_a="e2m1", fmt_b="e2m1", c="f32")
    assert np.array_equal(out6, 6.0 * want)


ALL_MX_PINS = [pin_mx_decode_exhaustive, pin_mx_fraction_bruteforce, pin_mx_block_scales_closed_form,
               pin_mx_smallint_integer_matmul, pin_mx_matches_16bit_oracle, pin_mx_points_and_rows,
               pin_e2m1_decode_table, pin_mxfp4_fraction_bruteforce, pin_mxfp4_matches_e4m3_oracle,
               pin_mxfp4_closed_form]
