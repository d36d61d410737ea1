"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes a loaded oracle and raises AssertionError when it
disagrees with:
  * hand-worked products and rounding cases (tests/golden/worked_gemm.json),
  * reference encodings of binary16 / bfloat16 / binary32 (tests/golden/format_values.txt),
  * numpy's and torch's own format conversions (exhaustive decode, RNE encode),
  * exact rational brute force (fractions.Fraction) on tiny shapes, with an
    independent decoder (struct 'e' for fp16, the binary32 layout for bf16),
  * integer matrix products (numpy int64) for small-integer inputs,
  * identity / permutation matrices, the ReLU closed form, the zero-padding
    invariant and the K = 0 empty sum.
The same functions run against deliberately broken copies of the oracle in
test_oracle.py to show that each plausible mistake is caught.
"""
from __future__ import annotations

import json
import os
import struct
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
def f16_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(x) -> np.ndarray:
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_of(x, dtype) -> np.ndarray:
    return f16_bits(x) if dtype == "f16" else bf16_bits(x)


def c_bits(x, dtype) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).view(np.uint32)
    return bits_of(x, dtype)


def frac_of_bits(b: int, dtype: str) -> Fraction:
    """Exact value of a 16-bit pattern through Python's own float formats."""
    if dtype == "f16":
        v = struct.unpack("<e", struct.pack("<H", int(b)))[0]
    else:
        v = struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]
    return Fraction(v)


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- golden files
def pin_worked_examples(O):
    data = json.load(open(os.path.join(GOLDEN, "worked_gemm.json")))
    for case in data["cases"]:
        M, N, K = case["M"], case["N"], case["K"]
        for dt in ("f16", "bf16"):
            A = bits_of(np.asarray(case["A"], dtype=np.float64).reshape(-1), dt)
            B = bits_of(np.asarray(case["B"], dtype=np.float64).reshape(-1), dt)
            cin = None
            if not case["clear_accum"]:
                cin = c_bits(np.asarray(case["C_in"], dtype=np.float64).reshape(-1), "f32")
            out = O.gemm(M, N, K, A, B, ab=dt, c="f32", transpose_A=case["transpose_A"],
                         transpose_B=case["transpose_B"], clear_accum=case["clear_accum"],
                         relu=case["relu"], C_in_bits=cin)
            want = np.asarray(case["C"], dtype=np.float64).reshape(M, N)
            assert np.array_equal(out, want), (case["name"], dt, out, want)
    for case in data["rounding"]["cases"]:
        dt = case["dtype"]
        A = bits_of(np.asarray(case["A"], dtype=np.float64).reshape(-1), dt)
        B = bits_of(np.asarray(case["B"], dtype=np.float64).reshape(-1), dt)
        o = O.gemm(1, 1, 2, A, B, ab=dt, c=dt)
        assert o[0, 0] == case["exact"], (case, o)
        enc = O.encode(o.reshape(-1), dt)
        assert int(enc[0]) == int(case["bits"], 16), (case, hex(int(enc[0])))
        assert O.rne_out(o.reshape(-1), dt)[0] == case["rounded"]


def pin_format_values(O):
    for line in open(os.path.join(GOLDEN, "format_values.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        dt, b, v = line.split()
        b = int(b, 16)
        v = float(v)
        got = O.decode(np.array([b], dtype=np.uint32), dt)[0]
        assert got == v and np.signbit(got) == np.signbit(v), (dt, hex(b), got, v)
        enc = int(O.encode(np.array([v]), dt)[0])
        assert enc == b, (dt, hex(b), hex(enc))


# ----------------------------------------------------------------- formats
def pin_decode_exhaustive(O):
    allb = np.arange(65536, dtype=np.uint32)
    ref16 = allb.astype(np.uint16).view(np.float16).astype(np.float64)
    got16 = O.decode(allb, "f16")
    nan = np.isnan(ref16)
    assert np.array_equal(np.isnan(got16), nan)
    assert np.array_equal(got16[~nan], ref16[~nan])
    assert np.array_equal(np.signbit(got16[~nan]), np.signbit(ref16[~nan]))
    with np.errstate(invalid="ignore"):
        refb = (allb << 16).view(np.float32).astype(np.float64)
    gotb = O.decode(allb, "bf16")
    nan = np.isnan(refb)
    assert np.array_equal(np.isnan(gotb), nan)
    assert np.array_equal(gotb[~nan], refb[~nan])
    assert np.array_equal(np.signbit(gotb[~nan]), np.signbit(refb[~nan]))
    r = _rng(11).integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    with np.errstate(invalid="ignore"):
        ref32 = r.view(np.float32).astype(np.float64)
    got32 = O.decode(r, "f32")
    nan = np.isnan(ref32)
    assert np.array_equal(got32[~nan], ref32[~nan])
    assert np.array_equal(np.isnan(got32), nan)


def _f16_test_values():
    rng = _rng(12)
    mag = np.exp2(rng.uniform(-30, 17, 200000))
    x = mag * rng.choice([-1.0, 1.0], mag.shape)
    # every midpoint between consecutive finite positive binary16 values (exact ties)
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2
    eps = np.abs(mids) * 2.0 ** -30
    extra = np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e10, 2.0 ** -25, 2.0 ** -26,
                      3 * 2.0 ** -26, 0.0, -0.0, 1.0, -1.0])
    return np.concatenate([x, mids, -mids, mids + eps, mids - eps, extra])


def pin_encode_f16(O):
    x = _f16_test_values()
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = O.encode(x, "f16")
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(x[i], hex(got[i]), hex(want[i])) for i in bad[:5]]
    assert int(O.encode(np.array([np.nan]), "f16")[0]) & 0x7C00 == 0x7C00


def pin_encode_bf16(O):
    rng = _rng(13)
    # float32-representable inputs, so torch's float32 -> bfloat16 cast (RNE) is the reference
    u = rng.integers(0, 2 ** 32, 300000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    # exact ties: bf16 patterns with an extra half-ulp bit set, including subnormals
    pats = np.arange(0, 0x7F80, dtype=np.uint32)
    ties = ((pats << 16) | 0x8000).view(np.float32)
    f = np.concatenate([f, ties, -ties, np.array([3.3961776e38, 3.39e38, 0.0, -0.0], np.float32)])
    want = torch.tensor(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.encode(f.astype(np.float64), "bf16")
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(f[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def pin_encode_f32(O):
    rng = _rng(14)
    mag = np.exp2(rng.uniform(-160, 130, 300000))
    x = mag * rng.choice([-1.0, 1.0], mag.shape)
    u = rng.integers(0, 0x7F800000, 50000, dtype=np.uint64).astype(np.uint32)
    fl = u.view(np.float32).astype(np.float64)
    nxt = (u + 1).view(np.float32).astype(np.float64)
    ties = (fl + nxt) / 2                      # exact binary32 midpoints
    x = np.concatenate([x, ties, -ties])
    with np.errstate(over="ignore"):
        want = x.astype(np.float32).view(np.uint32)
    got = O.encode(x, "f32")
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(x[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


# ----------------------------------------------------------------- the sum
def _rand_operands(rng, M, N, K, dt, tA, tB):
    a_shape = (K, M) if tA else (M, K)
    b_shape = (N, K) if tB else (K, N)
    A = bits_of(rng.uniform(-1, 1, a_shape).reshape(-1), dt)
    B = bits_of(rng.uniform(-1, 1, b_shape).reshape(-1), dt)
    return A, B


def pin_fraction_bruteforce(O):
    rng = _rng(21)
    shapes = [(1, 1, 1), (2, 3, 5), (3, 2, 8), (5, 8, 3), (8, 5, 17), (17, 3, 2), (3, 17, 8)]
    for (M, N, K) in shapes:
        for dt in ("f16", "bf16"):
            for tA in (0, 1):
                for tB in (0, 1):
                    relu = int(rng.integers(0, 2))
                    clear = int(rng.integers(0, 2))
                    A, B = _rand_operands(rng, M, N, K, dt, tA, tB)
                    cin = None if clear else c_bits(rng.uniform(-2, 2, M * N), "f32")
                    o = O.gemm(M, N, K, A, B, ab=dt, c="f32", transpose_A=tA, transpose_B=tB,
                               clear_accum=clear, relu=relu, C_in_bits=cin)
                    for m in range(M):
                        for n in range(N):
                            s = Fraction(0) if clear else Fraction(float(cin.view(np.float32)[m * N + n]))
                            absum = abs(s)
                            for k in range(K):
                                ai = (k * M + m) if tA else (m * K + k)
                                bi = (n * K + k) if tB else (k * N + n)
                                t = frac_of_bits(A[ai], dt) * frac_of_bits(B[bi], dt)
                                s += t
                                absum += abs(t)
                            if relu and s <= 0:
                                s = Fraction(0)
                            err = abs(Fraction(o[m, n]) - s)
                            assert err <= absum * Fraction(1, 2 ** 50), ((M, N, K, dt, tA, tB), m, n,
                                                                        float(s), o[m, n])
                            if relu:
                                assert o[m, n] >= 0 and not np.signbit(o[m, n])


def pin_small_integers(O):
    rng = _rng(22)
    for (M, N, K) in [(33, 47, 129), (64, 17, 200), (5, 130, 64), (1, 9, 1000)]:
        for dt in ("f16", "bf16"):
            for tA in (0, 1):
                for tB in (0, 1):
                    Ai = rng.integers(-4, 5, (M, K))
                    Bi = rng.integers(-4, 5, (K, N))
                    Cin = rng.integers(-50, 51, (M, N))
                    As = Ai.T.copy() if tA else Ai
                    Bs = Bi.T.copy() if tB else Bi
                    want = Ai @ Bi
                    o = O.gemm(M, N, K, bits_of(As.reshape(-1), dt), bits_of(Bs.reshape(-1), dt),
                               ab=dt, c="f32", transpose_A=tA, transpose_B=tB)
                    assert np.array_equal(o, want.astype(np.float64)), (M, N, K, dt, tA, tB)
                    o = O.gemm(M, N, K, bits_of(As.reshape(-1), dt), bits_of(Bs.reshape(-1), dt),
                               ab=dt, c="f32", transpose_A=tA, transpose_B=tB, clear_accum=0,
                               C_in_bits=c_bits(Cin.reshape(-1), "f32"), relu=1)
                    assert np.array_equal(o, np.maximum(want + Cin, 0).astype(np.float64))


def pin_identity_permutation(O):
    rng = _rng(23)
    n = 24
    eye = np.eye(n)
    perm = rng.permutation(n)
    P = eye[perm]
    for dt in ("f16", "bf16"):
        X = bits_of(rng.uniform(-1, 1, n * n), dt)
        Xv = O.decode(X, dt).reshape(n, n)
        I = bits_of(eye.reshape(-1), dt)
        assert np.array_equal(O.gemm(n, n, n, I, X, ab=dt, c="f32"), Xv)
        assert np.array_equal(O.gemm(n, n, n, X, I, ab=dt, c="f32"), Xv)
        Pb = bits_of(P.reshape(-1), dt)
        assert np.array_equal(O.gemm(n, n, n, Pb, X, ab=dt, c="f32"), Xv[perm])
        assert np.array_equal(O.gemm(n, n, n, X, Pb, ab=dt, c="f32"), Xv @ P)
        # X stored transposed, with the matching transpose flag, is the same operand X
        Xt = X.reshape(n, n).T.copy().reshape(-1)
        assert np.array_equal(O.gemm(n, n, n, Pb, Xt, ab=dt, c="f32", transpose_B=1), Xv[perm])
        assert np.array_equal(O.gemm(n, n, n, Xt, Pb, ab=dt, c="f32", transpose_A=1), Xv @ P)
        # ... while the flag alone reads the stored matrix transposed
        assert np.array_equal(O.gemm(n, n, n, Pb, X, ab=dt, c="f32", transpose_B=1), Xv.T[perm])


def pin_transpose_invariance(O):
    rng = _rng(24)
    M, N, K = 19, 23, 41
    for dt in ("f16", "bf16"):
        A = rng.uniform(-1, 1, (M, K))
        B = rng.uniform(-1, 1, (K, N))
        base = O.gemm(M, N, K, bits_of(A.reshape(-1), dt), bits_of(B.reshape(-1), dt), ab=dt)
        for tA in (0, 1):
            for tB in (0, 1):
                As = bits_of((A.T if tA else A).reshape(-1), dt)
                Bs = bits_of((B.T if tB else B).reshape(-1), dt)
                o = O.gemm(M, N, K, As, Bs, ab=dt, transpose_A=tA, transpose_B=tB)
                assert np.array_equal(o, base), (dt, tA, tB)
        # and against an independent float64 product of the decoded operands
        Ad = O.decode(bits_of(A.reshape(-1), dt), dt).reshape(M, K)
        Bd = O.decode(bits_of(B.reshape(-1), dt), dt).reshape(K, N)
        assert np.allclose(base, Ad @ Bd, rtol=0, atol=1e-12)


def pin_relu_closed_form(O):
    rng = _rng(25)
    M, N, K = 31, 29, 37
    A, B = _rand_operands(rng, M, N, K, "f16", 0, 0)
    plain = O.gemm(M, N, K, A, B)
    relu = O.gemm(M, N, K, A, B, relu=1)
    assert (plain < 0).any() and (plain > 0).any()
    assert np.array_equal(relu, np.where(plain > 0, plain, 0.0))
    assert not np.signbit(relu).any()


def pin_zero_padding(O):
    """Zero fill along K must not change the result (the ragged-K workload's invariant)."""
    rng = _rng(26)
    M, N, K, Kp = 37, 53, 77, 128
    for dt in ("f16", "bf16"):
        A = rng.uniform(-1, 1, (M, K))
        Bt = rng.uniform(-1, 1, (N, K))
        Ap = np.zeros((M, Kp)); Ap[:, :K] = A
        Btp = np.zeros((N, Kp)); Btp[:, :K] = Bt
        o = O.gemm(M, N, K, bits_of(A.reshape(-1), dt), bits_of(Bt.reshape(-1), dt), ab=dt,
                   c="f32", transpose_B=1)
        op = O.gemm(M, N, Kp, bits_of(Ap.reshape(-1), dt), bits_of(Btp.reshape(-1), dt), ab=dt,
                    c="f32", transpose_B=1)
        assert np.array_equal(o, op)
        # and it differs from the result with a dropped last K column (sanity of the invariant)
        o_short = O.gemm(M, N, K - 1, bits_of(A[:, :K - 1].reshape(-1), dt),
                         bits_of(Bt[:, :K - 1].reshape(-1), dt), ab=dt, c="f32", transpose_B=1)
        assert not np.array_equal(o, o_short)


def pin_points_and_rows(O):
    rng = _rng(27)
    M, N, K = 45, 38, 70
    for (tA, tB) in ((0, 0), (1, 1), (0, 1)):
        A, B = _rand_operands(rng, M, N, K, "bf16", tA, tB)
        cin = c_bits(rng.uniform(-1, 1, M * N), "f16")
        kw = dict(ab="bf16", c="f16", transpose_A=tA, transpose_B=tB, clear_accum=0,
                  C_in_bits=cin, relu=1)
        full = O.gemm(M, N, K, A, B, **kw)
        ms = rng.integers(0, M, 300)
        ns = rng.integers(0, N, 300)
        assert np.array_equal(O.gemm_points(M, N, K, A, B, ms, ns, **kw), full[ms, ns])
        assert np.array_equal(O.gemm(M, N, K, A, B, rows=(7, 30), nthreads=3, **kw), full[7:30])


def pin_empty_k(O):
    rng = _rng(28)
    M, N = 6, 5
    cin = rng.uniform(-1, 1, M * N)
    o = O.gemm(M, N, 0, np.zeros(0, np.uint16), np.zeros(0, np.uint16), c="f32",
               clear_accum=0, C_in_bits=c_bits(cin, "f32"))
    assert np.array_equal(o, cin.astype(np.float32).astype(np.float64).reshape(M, N))
    o = O.gemm(M, N, 0, np.zeros(0, np.uint16), np.zeros(0, np.uint16))
    assert np.array_equal(o, np.zeros((M, N)))


ALL_PINS = [pin_worked_examples, pin_format_values, pin_decode_exhaustive, pin_encode_f16,
            pin_encode_bf16, pin_encode_f32, pin_fraction_bruteforce, pin_small_integers,
            pin_identity_permutation, pin_transpose_invariance, pin_relu_closed_form,
            pin_zero_padding, pin_points_and_rows, pin_empty_k]
