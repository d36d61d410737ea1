"""CPU tests of the block-scaled (MX) GEMM oracle: its pins, its argument checks,
planted mistakes, and the seeded MX inputs."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest
import torch

import mx_pins
from oracle import oracle
from oracle.oracle import Oracle
import tlg_workloads as W

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "tlg_oracle.c")


@pytest.fixture(scope="module")
def O():
    return oracle.default()


@pytest.mark.parametrize("pin", mx_pins.ALL_MX_PINS, ids=lambda f: f.__name__)
def test_mx_pin(O, pin):
    pin(O)


def test_mx_rejects_bad_arguments(O):
    z = np.zeros(64, np.uint8)
    s = np.zeros(2, np.uint8)
    with pytest.raises(ValueError):
        O.mxgemm(1, 1, 48, z, s, z, s)              # K not a multiple of 32
    with pytest.raises(ValueError):
        O.mxgemm(1, 1, 32, z, s, z, s, clear_accum=0)
    with pytest.raises(KeyError):
        O.mxgemm(1, 1, 32, z, s, z, s, fmt_a="e3m2")
    with pytest.raises(ValueError):
        O.mxgemm_points(1, 1, 32, z, s, z, s, [1], [0])


MX_MUTANTS = {
    "block_of_16": ("* dec_e8m0(j->SA[m * KB + k / 32]);", "* dec_e8m0(j->SA[m * KB + k / 16]);"),
    "e4m3_exponent_bias": ("else v = ldexp((double)(8u + frac), (int)e - 7 - 3);",
                           "else v = ldexp((double)(8u + frac), (int)e - 8 - 3);"),
    "e4m3_subnormal": ("if (e == 0) v = ldexp((double)frac, 1 - 7 - 3);", "if (e == 0) v = ldexp((double)frac, -7 - 3);"),
    "scale_bias": ("return b == 255u ? NAN : ldexp(1.0, (int)b - 127);", "return b == 255u ? NAN : ldexp(1.0, (int)b - 128);"),
    "b_scaled_by_a_scales": ("* dec_e8m0(SB[n * KB + k / 32]);\n    int64_t rows",
                             "* dec_e8m0(SA[n * KB + k / 32]);\n    int64_t rows"),
    "e5m2_as_e4m3": ("case ORACLE_E5M2: return dec_e5m2(b);", "case ORACLE_E5M2: return dec_e4m3(b);"),
    "e2m1_high_nibble_first": ("return dec_e2m1((k & 1) ? byte >> 4 : byte & 15u);",
                               "return dec_e2m1((k & 1) ? byte & 15u : byte >> 4);"),
    "e2m1_exponent_bias": ("ldexp((double)(2u + frac), (int)e - 1 - 1);", "ldexp((double)(2u + frac), (int)e - 2 - 1);"),
    "e2m1_subnormal": ("e == 0 ? ldexp((double)frac, 1 - 1 - 1)", "e == 0 ? ldexp((double)frac, 1 - 1)"),
    "e2m1_row_stride_bytes": ("const uint32_t byte = X[r * (K / 2) + k / 2];", "const uint32_t byte = X[r * K + k / 2];"),
}


@pytest.mark.parametrize("name", sorted(MX_MUTANTS))
def test_mx_pins_catch_planted_mistake(tmp_path, name):
    src = open(ORACLE_SRC).read()
    old, new = MX_MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"mut_{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"libmut_{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", str(path),
                    "-o", str(so), "-lm", "-lpthread"], check=True)
    mut = Oracle(str(so))
    caught = False
    for pin in mx_pins.ALL_MX_PINS:
        try:
            pin(mut)
        except AssertionError:
            caught = True
            break
    assert caught, f"no pin caught the planted mistake {name}"


def test_mx_inputs_are_seeded_and_well_formed():
    case = W.MX_CONFIGS["mx1"]
    a1 = W.make_mx_inputs(case)
    a2 = W.make_mx_inputs(case)
    for x, y in zip(a1[:4], a2[:4]):
        assert torch.equal(x, y)
    A, SA, B, SB, C = a1
    assert A.dtype == torch.uint8 and A.shape == (256, 256) and SA.shape == (256, 8) and C is None
    va = A.view(torch.float8_e4m3fn).float()
    assert torch.isfinite(va).all() and float(va.abs().max()) <= 448.0
    # each block uses its scale: the largest element of a block lies in [2^8, 2^9]
    blk = va.abs().reshape(256, 8, 32).amax(2)
    assert float(blk.min()) >= 256.0
    m2 = W.MX_CONFIGS["mx2"]
    A, SA, B, SB, C = W.make_mx_inputs(m2)
    assert B.shape == (1500, 768) and SB.shape == (1500, 24)
    assert torch.isfinite(B.view(torch.float8_e5m2).float()).all()
    assert m2.algorithmic_bytes == (1000 + 1500) * 768 + (1000 + 1500) * 24 + 4 * 1000 * 1500


def test_mx_oracle_on_mx1_matches_sampled_bruteforce(O):
    """The 256^3 MXFP8 workload: full oracle vs exact rational sums at sampled points."""
    from fractions import Fraction
    case = W.MX_CONFIGS["mx1"]
    A, SA, B, SB, _ = (x.numpy() if x is not None else None for x in W.make_mx_inputs(case))
    full = O.mxgemm(case.M, case.N, case.K, A, SA, B, SB, relu=1)
    ms, ns = W.sample_points(case.M, case.N, 8)
    for m, n in zip(ms, ns):
        s = sum(mx_pins._exact(A, SA, "e4m3", m, k) * mx_pins._exact(B, SB, "e4m3", n, k) for k in range(case.K))
        s = max(s, Fraction(0))
        assert abs(Fraction(full[m, n]) - s) <= abs(s) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 60)
