"""CPU tests of the 2:4 structured-sparse GEMM oracle: its pins, its argument checks,
planted mistakes, and the seeded inputs."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest
import torch

import sp_pins
from oracle import oracle
from oracle.oracle import Oracle
import tlg_workloads as W

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "tlg_oracle.c")


@pytest.fixture(scope="module")
def O():
    return oracle.default()


@pytest.mark.parametrize("pin", sp_pins.ALL_SP_PINS, ids=lambda f: f.__name__)
def test_sp_pin(O, pin):
    pin(O)


def test_sp_rejects_bad_arguments(O):
    z8 = np.zeros(64, np.uint8)
    a16 = np.zeros(64, np.uint16)
    with pytest.raises(ValueError):
        O.spgemm(1, 1, 12, a16, a16, z8)                    # K not a multiple of 8
    with pytest.raises(ValueError):
        O.spgemm(1, 1, 16, a16, a16, z8, dtype="f32")
    with pytest.raises(ValueError):
        O.spgemm_points(1, 1, 16, a16, a16, z8, [1], [0])


SP_MUTANTS = {
    "metadata_nibbles_swapped": ("const int sh = 4 * (int)(q % 2);", "const int sh = 4 * (int)(1 - q % 2);"),
    "position_fields_swapped": ("const int p0 = (int)((byte >> sh) & 3u), p1 = (int)((byte >> (sh + 2)) & 3u);",
                                "const int p1 = (int)((byte >> sh) & 3u), p0 = (int)((byte >> (sh + 2)) & 3u);"),
    "second_value_dropped": ("w[4 * q + p1] += dec(dt, Wv[n * (K / 2) + 2 * q + 1]);", "(void)p1;"),
    "groups_of_eight": ("const uint32_t byte = Wm[n * (K / 8) + q / 2];", "const uint32_t byte = Wm[n * (K / 8) + q / 4];"),
}


@pytest.mark.parametrize("name", sorted(SP_MUTANTS))
def test_sp_pins_catch_planted_mistake(tmp_path, name):
    src = open(ORACLE_SRC).read()
    old, new = SP_MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"mut_{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"libmut_{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", str(path),
                    "-o", str(so), "-lm", "-lpthread"], check=True)
    mut = Oracle(str(so))
    caught = False
    for pin in sp_pins.ALL_SP_PINS:
        try:
            pin(mut)
        except AssertionError:
            caught = True
            break
    assert caught, f"no pin caught the planted mistake {name}"


def test_sp_inputs_are_seeded_and_well_formed():
    case = W.SP_CONFIGS["sp2"]
    a, b = W.make_sp_inputs(case), W.make_sp_inputs(case)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    A, Wv, Wm, dense = a
    assert A.shape == (1000, 768) and Wv.shape == (1500, 384) and Wm.shape == (1500, 96)
    assert ((dense != 0).reshape(1500, 192, 4).sum(axis=2) <= 2).all()
    assert case.flops == 1000 * 1500 * 768
