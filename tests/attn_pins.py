"""Pins of the attention-forward oracle: checks against things other than the oracle
itself (torch's float64 scaled_dot_product_attention, closed forms of the softmax
for flat and one-hot scores, and invariances of the definition).  Each pin raises
AssertionError."""
from __future__ import annotations

import numpy as np
import torch

TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)


def _rand(shape, dt, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(TDT[dt])


def _sdpa(q, k, v, causal, scale):
    """torch's own attention on the decoded values, in float64, [B, S, H, D] in and out."""
    f = lambda t: t.double().permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(f(q), f(k), f(v), is_causal=bool(causal), scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def pin_attn_matches_torch_sdpa(O):
    """Random operands, causal and not, default and explicit scale, fp16 and bf16."""
    for it, (B, S, H, D, dt, causal, scale) in enumerate([(2, 37, 3, 16, "f16", 1, None), (1, 29, 2, 64, "f16", 0, 0.3),
                                                          (2, 19, 1, 8, "bf16", 1, 1.7), (1, 70, 2, 32, "bf16", 0, None)]):
        q, k, v = (_rand((B, S, H, D), dt, 100 * it + s) for s in range(3))
        sc = 1.0 / np.sqrt(D) if scale is None else scale
        got = O.attn(B, S, H, D, _bits(q), _bits(k), _bits(v), dtype=dt, causal=causal, scale=scale)
        ref = _sdpa(q, k, v, causal, sc)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), (it, float(np.abs(got - ref).max()))


def pin_attn_flat_scores_give_prefix_mean(O):
    """K = 0: every allowed key scores 0, so each output is the plain mean of the allowed V rows."""
    B, S, H, D = 2, 23, 3, 8
    q, v = _rand((B, S, H, D), "f16", 7), _rand((B, S, H, D), "f16", 8)
    k = torch.zeros((B, S, H, D), dtype=torch.float16)
    vv = v.double().numpy()
    for causal in (1, 0):
        got = O.attn(B, S, H, D, _bits(q), _bits(k), _bits(v), causal=causal)
        if causal:
            want = np.cumsum(vv, axis=1) / np.arange(1, S + 1).reshape(1, S, 1, 1)
        else:
            want = np.broadcast_to(vv.mean(axis=1, keepdims=True), vv.shape)
        assert np.allclose(got, want, rtol=1e-13, atol=1e-14), causal


def pin_attn_one_hot_closed_form(O):
    """Q_i = a e_i, K_j = e_j, scale 1: the score matrix is a times the identity, so
    o_i = (e^a v_i + sum of the other allowed v_j) / (e^a + number of other allowed keys)."""
    S = D = 8
    a = 3.0
    q = torch.zeros((1, S, 1, D)); k = torch.zeros((1, S, 1, D))
    for i in range(S):
        q[0, i, 0, i] = a
        k[0, i, 0, i] = 1.0
    q, k = q.half(), k.half()
    v = _rand((1, S, 1, D), "f16", 9)
    vv = v.double().numpy()[0, :, 0, :]
    ea = np.exp(a)
    for causal in (1, 0):
        got = O.attn(1, S, 1, D, _bits(q), _bits(k), _bits(v), causal=causal, scale=1.0)[0, :, 0, :]
        for i in range(S):
            others = [j for j in (range(i) if causal else range(S)) if j != i]
            want = (ea * vv[i] + vv[others].sum(axis=0)) / (ea + len(others))
            assert np.allclose(got[i], want, rtol=1e-13, atol=1e-15), (causal, i)


def pin_attn_large_scores_stay_finite(O):
    """Scores of 800 (exp overflows double without the row maximum): the one-hot rows of the
    previous pin, now with a = 800, give o_i = v_i to double precision."""
    S = D = 8
    q = torch.zeros((1, S, 1, D)); k = torch.zeros((1, S, 1, D))
    for i in range(S):
        q[0, i, 0, i] = 800.0
        k[0, i, 0, i] = 1.0
    q, k = q.half(), k.half()
    v = _rand((1, S, 1, D), "f16", 10)
    for causal in (1, 0):
        got = O.attn(1, S, 1, D, _bits(q), _bits(k), _bits(v), causal=causal, scale=1.0)
        assert np.isfinite(got).all(), causal
        assert np.allclose(got, v.double().numpy(), rtol=1e-15, atol=0.0), causal


def pin_attn_causal_first_row_is_v0(O):
    """Under the causal rule the first query sees only the first key: o_0 = v_0 exactly."""
    B, S, H, D = 3, 17, 2, 16
    q, k, v = (_rand((B, S, H, D), "bf16", 20 + s) for s in range(3))
    got = O.attn(B, S, H, D, _bits(q), _bits(k), _bits(v), dtype="bf16", causal=1)
    assert np.array_equal(got[:, 0], v.double().numpy()[:, 0])


def pin_attn_key_shift_invariance(O):
    """Adding one vector u to every key adds scale*q_i.u to every score of row i, which the
    softmax ignores.  Small integers keep K and K + u exact in fp16."""
    B, S, H, D = 1, 31, 2, 16
    g = torch.Generator().manual_seed(30)
    q = torch.randint(-3, 4, (B, S, H, D), generator=g).half()
    k = torch.randint(-3, 4, (B, S, H, D), generator=g).half()
    u = torch.randint(-3, 4, (1, 1, H, D), generator=g).half()
    v = _rand((B, S, H, D), "f16", 31)
    for causal in (1, 0):
        a = O.attn(B, S, H, D, _bits(q), _bits(k), _bits(v), causal=causal, scale=0.2)
        b = O.attn(B, S, H, D, _bits(q), _bits(k + u), _bits(v), causal=causal, scale=0.2)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-13), causal


def pin_attn_noncausal_key_permutation(O):
    """Without the causal rule the keys form a set: permuting K and V rows together changes nothing."""
    B, S, H, D = 2, 41, 2, 32
    q, k, v = (_rand((B, S, H, D), "f16", 40 + s) for s in range(3))
    perm = torch.randperm(S, generator=torch.Generator().manual_seed(41))
    a = O.attn(B, S, H, D, _bits(q), _bits(k), _bits(v), causal=0)
    b = O.attn(B, S, H, D, _bits(q), _bits(k[:, perm]), _bits(v[:, perm]), causal=0)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def pin_attn_heads_and_batches_independent(O):
    """Changing the keys of one (batch, head) changes that head's output only."""
    B, S, H, D = 2, 13, 3, 8
    q, k, v = (_rand((B, S, H, D), "f16", 50 + s) for s in range(3))
    k2 = k.clone()
    k2[1, :, 2] = _rand((S, D), "f16", 53)
    a = O.attn(B, S, H, D, _bits(q), _bits(k), _bits(v), causal=0)
    b = O.attn(B, S, H, D, _bits(q), _bits(k2), _bits(v), causal=0)
    same = np.ones((B, H), dtype=bool); same[1, 2] = False
    for bb in range(B):
        for h in range(H):
            assert np.array_equal(a[bb, :, h], b[bb, :, h]) == bool(same[bb, h]), (bb, h)


def pin_attn_points_and_rows(O):
    B, S, H, D = 2, 33, 3, 16
    q, k, v = (_rand((B, S, H, D), "f16", 60 + s) for s in range(3))
    full = O.attn(B, S, H, D, _bits(q), _bits(k), _bits(v), causal=1)
    pb = np.array([0, 1, 1, 0]); pi = np.array([0, 32, 5, 17]); ph = np.array([2, 0, 1, 1])
    pts = O.attn_points(B, S, H, D, _bits(q), _bits(k), _bits(v), pb, pi, ph, causal=1)
    assert np.array_equal(full[pb, pi, ph], pts)
    part = O.attn(B, S, H, D, _bits(q), _bits(k), _bits(v), causal=1, rows=(10, 20), nthreads=3)
    assert np.array_equal(part, full[:, 10:20])


ALL_ATTN_PINS = [pin_attn_matches_torch_sdpa, pin_attn_flat_scores_give_prefix_mean, pin_attn_one_hot_closed_form,
                 pin_attn_large_scores_stay_finite, pin_attn_causal_first_row_is_v0, pin_attn_key_shift_invariance, pin_attn_noncausal_key_permutation,
                 pin_attn_heads_and_batches_independent, pin_attn_points_and_rows]
