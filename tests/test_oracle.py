"""CPU tests of the oracle: its pins, its argument checks, and that the pins catch planted mistakes."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest
import torch

import oracle_pins
from oracle import oracle
from oracle.oracle import Oracle
import tlg_workloads as W

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "tlg_oracle.c")


@pytest.fixture(scope="module")
def O():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(O, pin):
    pin(O)


def test_rejects_bad_arguments(O):
    z = np.zeros(4, np.uint16)
    with pytest.raises(ValueError):
        O.gemm(-1, 2, 2, z, z)
    with pytest.raises(ValueError):
        O.gemm(2, 2, 1, z, z, ab="f32")          # operands must be 16-bit
    with pytest.raises(ValueError):
        O.gemm(2, 2, 1, z, z, clear_accum=0)     # accumulating needs C_in
    with pytest.raises(ValueError):
        O.gemm_points(2, 2, 1, z, z, [2], [0])  # point outside C


# ------------------------------------------------------------------ planted mistakes
MUTANTS = {
    "drop_last_k": ("for (int64_t k = 0; k < j->K; ++k)\n                s += arow[k] * bc[k];",
                    "for (int64_t k = 0; k < j->K - 1; ++k)\n                s += arow[k] * bc[k];"),
    "b_index_swapped": ("transpose_B ? B[n * K + k] : B[k * N + n];\n            bcol",
                        "transpose_B ? B[k * N + n] : B[n * K + k];\n            bcol"),
    "a_index_swapped": ("j->tA ? j->A[k * j->M + m] : j->A[m * j->K + k]",
                        "j->tA ? j->A[m * j->K + k] : j->A[k * j->M + m]"),
    "relu_negative_zero": ("if (j->relu) s = (s > 0.0) ? s : 0.0;",
                           "if (j->relu) s = (s > 0.0) ? s : s * 0.0;"),
    "ties_away_from_zero": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    "subnormal_exponent": ("v = ldexp((double)frac, 1 - bias - p);", "v = ldexp((double)frac, -bias - p);"),
    "ignores_prior_c": ("double s = j->clear ? 0.0 : dec(j->cd, c_bits(j->C_in, j->cd, m * j->N + n));",
                        "double s = 0.0;"),
    "bf16_exponent_bits": ("case ORACLE_BF16: return dec_ieee(bits & 0xffffu, 7, 8);",
                           "case ORACLE_BF16: return dec_ieee(bits & 0xffffu, 8, 7);"),
}


def _build_mutant(tmp_path, name):
    src = open(ORACLE_SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"mut_{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"libmut_{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", str(path),
                    "-o", str(so), "-lm", "-lpthread"], check=True)
    return Oracle(str(so))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name):
    mut = _build_mutant(tmp_path, name)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mut)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught the planted mistake {name}"


# ------------------------------------------------------------------ seeded inputs
def test_inputs_are_seeded_and_shaped():
    c1 = W.CONFIGS["c1"]
    A1, B1, _ = W.make_inputs(c1)
    A2, B2, _ = W.make_inputs(c1)
    assert torch.equal(A1, A2) and torch.equal(B1, B2)
    assert A1.dtype == torch.float16 and A1.shape == (256, 256)
    assert float(A1.abs().max()) <= 1.0 and float(A1.min()) < -0.9 and float(A1.max()) > 0.9
    c4 = W.CONFIGS["c4"]
    A, B, _ = W.make_inputs(c4)
    assert A.shape == (1000, 777) and B.shape == (1500, 777) and B.dtype == torch.bfloat16
    # normal(0,1)/sqrt(K): sample std close to 1/sqrt(K)
    small = c4.with_(M=256, N=256, K=1024, ab="f16", c="f16", transpose_B=0, dist="normal")
    A, B, _ = W.make_inputs(small)
    std = float(A.float().std())
    assert abs(std * 32 - 1.0) < 0.02
    ints = small.with_(dist="smallint")
    A, B, _ = W.make_inputs(ints)
    vals = torch.unique(A.float())
    assert set(vals.tolist()) <= set(range(-4, 5))


def test_workload_table_matches_the_five_configs():
    C = W.CONFIGS
    assert (C["c1"].M, C["c1"].N, C["c1"].K, C["c1"].relu) == (256, 256, 256, 1)
    assert (C["c2"].M, C["c2"].relu) == (1024, 0)
    assert (C["c3"].M, C["c3"].relu, C["c3"].dist) == (4096, 1, "normal")
    assert (C["c4"].M, C["c4"].N, C["c4"].K, C["c4"].ab, C["c4"].c, C["c4"].transpose_B) == \
        (1000, 1500, 777, "bf16", "f32", 1)
    assert (C["c5a"].M, C["c5a"].dist) == (8192, "normal")
    assert (C["c5b"].M, C["c5b"].N, C["c5b"].K, C["c5b"].transpose_B) == (16, 16384, 8192, 1)
    # algorithmic bytes of the skinny case: 2*16*8192 + 2*8192*16384 + 2*16*16384
    assert C["c5b"].algorithmic_bytes == 269221888


def test_oracle_on_config1_matches_sampled_bruteforce(O):
    """The full 256^3 ReLU workload: full oracle vs exact rational sums at sampled points."""
    from fractions import Fraction
    case = W.CONFIGS["c1"]
    A, B, _ = W.make_inputs(case)
    Ab, Bb = W.bits16(A), W.bits16(B)
    full = O.gemm(case.M, case.N, case.K, Ab, Bb, relu=1)
    ms, ns = W.sample_points(case.M, case.N, 12)
    for m, n in zip(ms, ns):
        s = sum(oracle_pins.frac_of_bits(Ab[m * case.K + k], "f16") *
                oracle_pins.frac_of_bits(Bb[k * case.N + n], "f16") for k in range(case.K))
        s = max(s, Fraction(0))
        assert abs(Fraction(full[m, n]) - s) <= Fraction(1, 2 ** 40)
