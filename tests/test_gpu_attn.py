"""GPU parity of the attention forward (tlg_attn_fwd) against the CPU attention oracle on
the same seeded fp16/bf16 bits.  Tolerance per element (derived in the oracle):
|gpu - o| <= 2u (|o| + max|V|) + 1e-5, u = 2^-11 (fp16) or 2^-8 (bf16).  At full size,
flat scores and integer scores (exact power-of-two probabilities) with integer values
are checked at every output against exact values, within (u + 2^-20) |o|."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import tlg_workloads as W
from oracle import oracle as O
from parity import log, out_values

pytestmark = pytest.mark.gpu


def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _run(case: W.AttnCase, q, k, v, guard: int = 0):
    """Run through the binding; with guard > 0 (elements), O sits inside a larger buffer whose
    guard bands must come back untouched."""
    import tiled_dense_gemm_02_amd as tlg
    dev = _device()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    n = q.numel()
    if guard:
        buf = torch.empty(guard + n + guard, dtype=q.dtype, device=dev)
        buf.view(torch.int16).fill_(0x5A5A)
        O_ = buf[guard:guard + n].view(q.shape)
    else:
        buf, O_ = None, torch.empty_like(qd)
    tlg.attention(qd, kd, vd, O_, causal=bool(case.causal), scale=case.scale)
    torch.cuda.synchronize()
    if guard:
        g = buf.view(torch.int16)
        assert bool((g[:guard] == 0x5A5A).all()) and bool((g[guard + n:] == 0x5A5A).all()), "guard band written"
    return O_


def _check(case: W.AttnCase, gpu: np.ndarray, o: np.ndarray, vmax: float):
    tol = O.attn_tolerance(o, vmax, case.dtype)
    err = np.abs(gpu - o)
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{case.name}: {int(bad.sum())} of {bad.size} outside tolerance; first {idx.tolist()} "
                             f"gpu={gpu[bad][:5]} oracle={o[bad][:5]}")
    return float(err.max()) if err.size else 0.0


def _full(case: W.AttnCase, guard: int = 0):
    log(f"[case] {case.name} B={case.B} S={case.S} H={case.H} D={case.D} causal={case.causal} {case.dtype}")
    q, k, v = W.make_attn_inputs(case)
    out = _run(case, q, k, v, guard)
    o = O.attn(case.B, case.S, case.H, case.D, W.bits16(q), W.bits16(k), W.bits16(v), dtype=case.dtype,
               causal=case.causal, scale=case.softmax_scale)
    err = _check(case, out_values(out), o, float(v.float().abs().max()))
    log(f"    max|err| = {err:.3e}")


def test_fa1_page_instance_full():
    _full(W.ATTN_CONFIGS["fa1"])


def test_fa2_ragged_noncausal_full():
    _full(W.ATTN_CONFIGS["fa2"], guard=4096)


@pytest.mark.parametrize("name", ["fa3", "fa4"])
def test_full_size_sampled(name):
    case = W.ATTN_CONFIGS[name]
    log(f"[case] {name} sampled")
    q, k, v = W.make_attn_inputs(case)
    out = out_values(_run(case, q, k, v))
    pb, pi, ph = W.sample_attn_rows(case, 384)
    o = O.attn_points(case.B, case.S, case.H, case.D, W.bits16(q), W.bits16(k), W.bits16(v), pb, pi, ph,
                      dtype=case.dtype, causal=case.causal, scale=case.softmax_scale)
    err = _check(case, out[pb, pi, ph], o, float(v.float().abs().max()))
    assert np.isfinite(out).all()
    log(f"    max|err| = {err:.3e}")


def _check_prefix_mean(case: W.AttnCase):
    """Every output of a flat-score case against the exact mean of V's integers.

    With K = 0 every score is exactly zero, so every allowed key gets probability
    2^0 = 1 in the operand type; the row sum is the exact key count and the weighted
    sum of integers in [-4, 4] is exact in fp32.  O is then the exact mean o rounded
    twice in fp32 (the reciprocal of the count, the product) and once to the operand
    type: |gpu - o| <= (u + 2^-20) |o| with u = 2^-11 (fp16) or 2^-8 (bf16), where
    |o| >= 1/S whenever o != 0 keeps o in the normal range.  A key block dropped,
    repeated or taken from the wrong rows moves some output of the last rows by at
    least 1/S, far outside this bound."""
    log(f"[case] {case.name} B={case.B} S={case.S} H={case.H} D={case.D} causal={case.causal} {case.dtype} "
        f"flat scores, integer values, every output")
    q, k, v = W.make_attn_inputs(case)
    out = _run(case, q, k, v)
    vi = v.float().numpy().astype(np.int64)
    del q, k, v
    u = 2.0 ** -11 if case.dtype == "f16" else 2.0 ** -8
    count = np.arange(1, case.S + 1, dtype=np.float64)[:, None, None]
    worst = 0.0
    for b in range(case.B):
        if case.causal:
            o = np.cumsum(vi[b], axis=0) / count
        else:
            o = np.broadcast_to(vi[b].sum(axis=0) / case.S, vi[b].shape)
        got = out_values(out[b])
        err = np.abs(got - o)
        bad = ~(err <= (u + 2.0 ** -20) * np.abs(o))
        if bad.any():
            idx = np.argwhere(bad)[:5]
            raise AssertionError(f"{case.name} batch {b}: {int(bad.sum())} of {bad.size} outputs off the exact "
                                 f"mean; first (i, h, d) {idx.tolist()} gpu={got[bad][:5]} exact={o[bad][:5]}")
        nz = o != 0
        if nz.any():
            worst = max(worst, float((err[nz] / np.abs(o[nz])).max()))
    log(f"    max relative error {worst:.3e} (bound {u + 2.0 ** -20:.3e})")


@pytest.mark.parametrize("name", ["fa3", "fa4"])
def test_full_size_flat_scores_every_output(name):
    """The two large causal workloads at full size, every output checked: the causal
    mask and every key block of every (batch, head) enter each row exactly once."""
    _check_prefix_mean(W.ATTN_CONFIGS[name].with_(name=f"{name}-flat-int", dist="flat_int_values", seed=1450))


@pytest.mark.parametrize("shape", [(2, 4000, 8, 128, 0), (1, 4000, 4, 64, 1)], ids=lambda s: "x".join(map(str, s)))
def test_ragged_flat_scores_every_output_bf16(shape):
    """A partial last key block (4000 = 62.5 blocks of 64), with and without the mask."""
    B, S, H, D, causal = shape
    _check_prefix_mean(W.AttnCase(f"flat-int-{B}x{S}x{H}x{D}-c{causal}", B, S, H, D, causal=causal, dtype="bf16",
                                  dist="flat_int_values", seed=1460 + causal))


def _dyadic_expected(case: W.AttnCase, q, k, v, b: int) -> np.ndarray:
    """Softmax-weighted means of the dyadic-score recipe for batch b, [S, H, D], exactly:
    query i's weights are 2^(k[j,0] + q[i,1] k[j,1]) (the row maximum is 0 at key 0), so
    with two query classes the weighted sums over the allowed keys are prefix sums of
    dyadic numbers, exact in float64, and one division gives each output."""
    kb = k[b].float().numpy().astype(np.float64)
    vb = v[b].float().numpy().astype(np.float64)
    cls = q[b, :, :, 1].float().numpy()
    out = np.empty(vb.shape)
    for c in (0.0, 1.0):
        w = np.exp2(kb[:, :, 0] + c * kb[:, :, 1])
        if case.causal:
            o = np.cumsum(w[:, :, None] * vb, axis=0) / np.cumsum(w, axis=0)[:, :, None]
        else:
            o = np.broadcast_to((w[:, :, None] * vb).sum(axis=0) / w.sum(axis=0)[:, None], vb.shape)
        sel = cls == c
        out[sel] = o[sel]
    return out


def _check_dyadic(case: W.AttnCase):
    """Every output of a dyadic-score case against its exact value.

    With the scale ln 2 the kernel's folded factor scale*log2(e) is exactly 1, every
    score is an integer in [-6, 0] and every row's first key block holds its maximum 0,
    so each probability is an exact power of two in [2^-6, 1] in the operand type and
    the row sums and P V sums (multiples of 2^-6 below 2^14) are exact in fp32.  The
    result differs from the exact value only by the two fp32 roundings of the division
    and the rounding to the operand type: |gpu - o| <= (u + 2^-20) |o|, plus half the
    fp16 subnormal spacing (2^-25) since |o| can be as small as 2^-6 / S.  The expected
    values are pinned to the oracle on sampled rows."""
    log(f"[case] {case.name} B={case.B} S={case.S} H={case.H} D={case.D} causal={case.causal} {case.dtype} "
        f"dyadic scores, every output")
    q, k, v = W.make_attn_inputs(case)
    out = _run(case, q, k, v)
    pb, pi, ph = W.sample_attn_rows(case, 64)
    o_pts = O.attn_points(case.B, case.S, case.H, case.D, W.bits16(q), W.bits16(k), W.bits16(v), pb, pi, ph,
                          dtype=case.dtype, causal=case.causal, scale=case.softmax_scale)
    u = 2.0 ** -11 if case.dtype == "f16" else 2.0 ** -8
    floor = 2.0 ** -25 if case.dtype == "f16" else 0.0
    worst = 0.0
    for b in range(case.B):
        o = _dyadic_expected(case, q, k, v, b)
        sel = pb == b
        if sel.any():
            ref = o[pi[sel], ph[sel]]
            assert np.allclose(ref, o_pts[sel], rtol=1e-12, atol=1e-15), "closed form disagrees with the oracle"
        got = out_values(out[b])
        err = np.abs(got - o)
        bad = ~(err <= (u + 2.0 ** -20) * np.abs(o) + floor)
        if bad.any():
            idx = np.argwhere(bad)[:5]
            raise AssertionError(f"{case.name} batch {b}: {int(bad.sum())} of {bad.size} outputs off the exact "
                                 f"value; first (i, h, d) {idx.tolist()} gpu={got[bad][:5]} exact={o[bad][:5]}")
        nz = np.abs(o) > 2.0 ** -14
        if nz.any():
            worst = max(worst, float((err[nz] / np.abs(o[nz])).max()))
    log(f"    max relative error (|o| > 2^-14) {worst:.3e} (bound {u + 2.0 ** -20:.3e})")


@pytest.mark.parametrize("name", ["fa3", "fa4"])
def test_full_size_dyadic_scores_every_output(name):
    """The two large causal workloads at full size through the exponentials, row sums and
    P V products with query-dependent scores, every output checked."""
    _check_dyadic(W.ATTN_CONFIGS[name].with_(name=f"{name}-dyadic", dist="dyadic_scores", scale=math.log(2.0),
                                             seed=1470))


@pytest.mark.parametrize("shape", [(2, 4000, 8, 128, 0), (1, 4000, 4, 64, 1)], ids=lambda s: "x".join(map(str, s)))
def test_ragged_dyadic_scores_every_output_bf16(shape):
    B, S, H, D, causal = shape
    _check_dyadic(W.AttnCase(f"dyadic-{B}x{S}x{H}x{D}-c{causal}", B, S, H, D, causal=causal, dtype="bf16",
                             dist="dyadic_scores", scale=math.log(2.0), seed=1480 + causal))


SWEEP = [(1, 1, 1, 64, 1), (1, 2, 3, 128, 0), (2, 63, 2, 64, 1), (1, 64, 2, 128, 1), (1, 65, 1, 64, 0),
         (2, 127, 1, 128, 1), (1, 128, 2, 64, 1), (1, 129, 2, 128, 0), (3, 200, 2, 64, 1), (1, 300, 3, 128, 1),
         (1, 257, 1, 64, 0), (1, 513, 1, 128, 1)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", SWEEP, ids=lambda s: "x".join(map(str, s)))
def test_shape_sweep(shape, dtype):
    B, S, H, D, causal = shape
    seed = 1300 + B * 7 + S * 3 + H + D + causal
    _full(W.AttnCase(f"sweep-{B}x{S}x{H}x{D}-c{causal}-{dtype}", B, S, H, D, causal=causal, dtype=dtype, seed=seed),
          guard=2048)


def test_explicit_scale_and_flat_keys():
    """K = 0 gives the prefix mean of V (causal) whatever the scale; a large explicit
    scale on random keys makes the softmax nearly one-hot."""
    _full(W.AttnCase("flat-keys", 2, 333, 2, 64, causal=1, dist="uniform_keys", scale=5.0, seed=1401))
    _full(W.AttnCase("sharp", 1, 300, 2, 128, causal=0, scale=1.0, seed=1402))
    _full(W.AttnCase("sharp-bf16", 1, 300, 2, 64, causal=1, scale=0.9, dtype="bf16", seed=1403))


@pytest.mark.parametrize("dist", ["ramp_up", "ramp_down"])
def test_score_ramps(dist):
    """Scores rising along the keys by ~0.2 (log2 units) per position: a row's reference
    maximum then moves only every few dozen keys, and unnormalised probabilities up to
    2^8 are rounded to the operand type in between.  Falling scores: it never moves
    after the first key, and most probabilities are tiny."""
    _full(W.AttnCase(f"{dist}-f16", 2, 777, 2, 64, causal=1, dist=dist, seed=1420))
    _full(W.AttnCase(f"{dist}-bf16-d128", 1, 520, 2, 128, causal=0, dist=dist, dtype="bf16", seed=1421))


@pytest.mark.parametrize("scale", [-0.3, -2.0, 0.0])
def test_negative_and_zero_scale(scale):
    """A negative scale turns the row maximum of the scaled scores into the scale times the
    row minimum of the raw scores; a zero scale gives every allowed key the same weight."""
    _full(W.AttnCase(f"scale{scale}", 1, 333, 2, 128, causal=1, scale=scale, seed=1410))
    _full(W.AttnCase(f"scale{scale}-d64-full", 2, 200, 1, 64, causal=0, scale=scale, dtype="bf16", seed=1411))


def test_deterministic():
    case = W.ATTN_CONFIGS["fa1"].with_(name="attn-determinism", B=2, S=640)
    q, k, v = W.make_attn_inputs(case)
    a = _run(case, q, k, v)
    b = _run(case, q, k, v)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("shape", [(1, 200, 2, 64, 1, "f16"), (2, 777, 3, 128, 0, "f16"), (1, 1024, 4, 128, 1, "bf16"),
                                   (3, 129, 5, 64, 0, "bf16"), (1, 4096, 2, 64, 1, "f16")])
def test_query_blocks_of_64_and_128_bit_identical(shape):
    """Workgroups of 64 or 128 queries form every query's sums in the same order (the same
    key blocks, MFMA steps and reference-maximum moves): their outputs must be equal bit for
    bit, and the automatic choice must be one of them."""
    import tiled_dense_gemm_02_amd as tlg
    B, S, H, D, causal, dtype = shape
    case = W.AttnCase(f"qblock-{B}x{S}x{H}x{D}-c{causal}-{dtype}", B, S, H, D, causal=causal, dtype=dtype, seed=1430)
    log(f"[case] {case.name}")
    dev = _device()
    q, k, v = (t.to(dev) for t in W.make_attn_inputs(case))
    outs = {}
    for bq in (64, 128, 0):
        outs[bq] = tlg.attention(q, k, v, causal=bool(causal), block_q=bq)
    torch.cuda.synchronize()
    assert torch.equal(outs[64].view(torch.int16), outs[128].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[64].view(torch.int16))
    o = O.attn(B, S, H, D, W.bits16(q.cpu()), W.bits16(k.cpu()), W.bits16(v.cpu()), dtype=dtype, causal=causal)
    gpu = O.decode(W.bits16(outs[0].cpu()), dtype).reshape(o.shape)
    _check(case, gpu, o, float(v.float().abs().max()))


def test_error_paths_enqueue_nothing():
    import tiled_dense_gemm_02_amd as tlg
    dev = _device()
    x = torch.zeros((1, 64, 2, 64), dtype=torch.float16, device=dev)
    o = torch.full_like(x, 3.0)
    p, po = x.data_ptr(), o.data_ptr()
    assert tlg.attention_ptrs(p + 8, p, p, po, 1, 32, 2, 64, torch.float16, 1, 0.125) == -4     # misaligned
    assert tlg.attention_ptrs(p, p, p, p, 1, 64, 2, 64, torch.float16, 1, 0.125) == -1          # O overlaps Q
    assert tlg.attention_ptrs(p, p, p, po, 1, 64, 2, 96, torch.float16, 1, 0.125) == -2         # dim 96
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())
