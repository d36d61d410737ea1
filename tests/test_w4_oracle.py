"""CPU tests of the 4-bit dequant GEMM oracle: its pins, its argument checks, planted
mistakes, and the seeded inputs."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest
import torch

import w4_pins
from oracle import oracle
from oracle.oracle import Oracle
import tlg_workloads as W

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "tlg_oracle.c")


@pytest.fixture(scope="module")
def O():
    return oracle.default()


@pytest.mark.parametrize("pin", w4_pins.ALL_W4_PINS, ids=lambda f: f.__name__)
def test_w4_pin(O, pin):
    pin(O)


def test_w4_rejects_bad_arguments(O):
    z8 = np.zeros(64, np.uint8)
    s16 = np.zeros(4, np.uint16)
    a16 = np.zeros(64, np.uint16)
    with pytest.raises(ValueError):
        O.w4gemm(1, 1, 48, 32, a16, z8, s16, z8)            # K not a multiple of G
    with pytest.raises(ValueError):
        O.w4gemm(1, 1, 12, 4, a16, z8, s16, z8)             # K not a multiple of 8
    with pytest.raises(ValueError):
        O.w4gemm(1, 1, 32, 32, a16, z8, s16, z8, dtype="f32")
    with pytest.raises(ValueError):
        O.w4gemm_points(1, 1, 32, 32, a16, z8, s16, z8, [1], [0])


W4_MUTANTS = {
    "nibble_halves_swapped": ("const int shift = (j % 2 == 0) ? 4 * (j / 2) : 16 + 4 * (j / 2);",
                              "const int shift = (j % 2 == 0) ? 16 + 4 * (j / 2) : 4 * (j / 2);"),
    "zero_point_ignored": ("return dec(dt, enc(dt, (q - z) * s));", "return dec(dt, enc(dt, q * s + 0.0 * z));"),
    "no_rounding_of_weights": ("return dec(dt, enc(dt, (q - z) * s));", "return (q - z) * s;"),
    "group_index_halved": ("const double z = (double)Z[n * KG + k / G];",
                           "const double z = (double)Z[n * KG + (k / G) / 2];"),
    "scale_read_as_fp16": ("const double s = dec(dt, S[n * KG + k / G]);",
                           "const double s = dec(ORACLE_F16, S[n * KG + k / G]);"),
}


@pytest.mark.parametrize("name", sorted(W4_MUTANTS))
def test_w4_pins_catch_planted_mistake(tmp_path, name):
    src = open(ORACLE_SRC).read()
    old, new = W4_MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"mut_{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"libmut_{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", str(path),
                    "-o", str(so), "-lm", "-lpthread"], check=True)
    mut = Oracle(str(so))
    caught = False
    for pin in w4_pins.ALL_W4_PINS:
        try:
            pin(mut)
        except AssertionError:
            caught = True
            break
    assert caught, f"no pin caught the planted mistake {name}"


def test_w4_inputs_are_seeded_and_well_formed():
    case = W.W4_CONFIGS["w4b"]
    a, b = W.make_w4_inputs(case), W.make_w4_inputs(case)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    A, Wq, S, Z, q = a
    assert A.shape == (5, 768) and A.dtype == torch.bfloat16
    assert Wq.shape == (1000, 384) and Wq.dtype == torch.uint8
    assert S.shape == (1000, 12) and Z.shape == (1000, 12) and int(Z.max()) <= 15 and int(q.max()) <= 15
    assert float(S.float().min()) > 0
    assert case.algorithmic_bytes == 2 * 5 * 768 + 1000 * 384 + 3 * 1000 * 12 + 4 * 5 * 1000
