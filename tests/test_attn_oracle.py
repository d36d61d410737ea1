"""CPU tests of the attention-forward oracle: its pins, its argument checks, planted
mistakes, and the seeded attention inputs."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest
import torch

import attn_pins
from oracle import oracle
from oracle.oracle import Oracle
import tlg_workloads as W

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "tlg_oracle.c")


@pytest.fixture(scope="module")
def O():
    return oracle.default()


@pytest.mark.parametrize("pin", attn_pins.ALL_ATTN_PINS, ids=lambda f: f.__name__)
def test_attn_pin(O, pin):
    pin(O)


def test_attn_rejects_bad_arguments(O):
    z = np.zeros(64, np.uint16)
    with pytest.raises(ValueError):
        O.attn(1, 4, 1, 0, z, z, z)                        # dim 0
    with pytest.raises(ValueError):
        O.attn(1, 4, 1, 16, z, z, z, dtype="f32")          # operands are 16-bit
    with pytest.raises(ValueError):
        O.attn(1, 4, 1, 16, z, z, z, scale=float("inf"))
    with pytest.raises(ValueError):
        O.attn(1, 4, 1, 16, z, z, z, rows=(2, 5))          # rows past seq
    with pytest.raises(ValueError):
        O.attn_points(1, 4, 1, 16, z, z, z, [0], [4], [0])
    assert O.attn(0, 4, 1, 16, z, z, z).shape == (0, 4, 1, 16)


ATTN_MUTANTS = {
    "causal_excludes_diagonal": ("const int64_t nkeys = j->causal ? i + 1 : S;",
                                 "const int64_t nkeys = j->causal ? i : S;"),
    "scale_dropped": ("s[t] = j->scale * dot;", "s[t] = dot;"),
    "keys_read_as_bhsd": ("const uint16_t *k = j->K + ((b * S + t) * H + h) * D;",
                          "const uint16_t *k = j->K + ((b * H + h) * S + t) * D;"),
    "value_of_the_query_row": ("const uint16_t *v = j->V + ((b * S + t) * H + h) * D;",
                               "const uint16_t *v = j->V + ((b * S + i) * H + h) * D;"),
    "normaliser_counts_keys": ("denom += w;", "denom += 1.0;"),
    "max_from_first_key_only": ("if (s[t] > mx) mx = s[t];", "if (t == 0) mx = s[t];"),
}


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_attn_pins_catch_planted_mistake(tmp_path, name):
    src = open(ORACLE_SRC).read()
    old, new = ATTN_MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"mut_{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"libmut_{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", str(path),
                    "-o", str(so), "-lm", "-lpthread"], check=True)
    mut = Oracle(str(so))
    caught = False
    for pin in attn_pins.ALL_ATTN_PINS:
        try:
            pin(mut)
        except AssertionError:
            caught = True
            break
    assert caught, f"no pin caught the planted mistake {name}"


def test_attn_inputs_are_seeded_and_well_formed():
    case = W.ATTN_CONFIGS["fa1"]
    a, b = W.make_attn_inputs(case), W.make_attn_inputs(case)
    for x, y in zip(a, b):
        assert torch.equal(x, y) and x.shape == (1, 1024, 8, 64) and x.dtype == torch.float16
    assert not torch.equal(a[0], a[1])
    k = W.make_attn_inputs(case.with_(dist="uniform_keys", S=16))[1]
    assert float(k.abs().max()) == 0.0
    assert case.flops == 4 * 64 * (1024 * 1025 // 2) * 8
    assert W.ATTN_CONFIGS["fa2"].flops == 4 * 128 * 777 * 777 * 6
    pb, pi, ph = W.sample_attn_rows(W.ATTN_CONFIGS["fa3"], 64)
    assert pb.max() < 4 and pi.max() < 4096 and ph.max() < 32 and len(pb) == 64


def test_attn_oracle_fa1_sampled_rows_match_torch(O):
    """The page's instance (causal, 1x1024x8x64): oracle rows against torch's float64 attention."""
    case = W.ATTN_CONFIGS["fa1"]
    q, k, v = W.make_attn_inputs(case)
    pb, pi, ph = W.sample_attn_rows(case, 32)
    got = O.attn_points(case.B, case.S, case.H, case.D, W.bits16(q), W.bits16(k), W.bits16(v), pb, pi, ph,
                        causal=case.causal)
    ref = attn_pins._sdpa(q, k, v, case.causal, case.softmax_scale)
    assert np.allclose(got, ref[pb, pi, ph], rtol=1e-12, atol=1e-13)
