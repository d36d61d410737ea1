"""Seeded synthetic inputs for the tiled GEMM C = act(A·B).

This module only draws random operands and describes the workload shapes.  It
holds none of the GEMM arithmetic: both the HIP path (through the Python
binding) and the CPU oracle consume the bits it produces, and neither imports
the other.

Recipe (the pages fix no seed or generator; this is the reading used here):
  * CPU ``torch.Generator().manual_seed(seed)``, drawing A first, then B, then
    (when needed) the prior contents of C, each as float32;
  * ``uniform``: ``2 * torch.rand(shape) - 1`` (values in [-1, 1));
    ``normal``: ``torch.randn(shape) / sqrt(K)``;
    ``smallint``: integers drawn uniformly from [lo, hi];
  * then a round-to-nearest-even cast to float16 / bfloat16 on the CPU.  The
    rounded bits are the inputs of both sides.
  * Operands are drawn directly in their stored shape: A is M×K (K×M when
    transpose_A), B is K×N (N×K when transpose_B).  The entries are i.i.d., so
    the distribution does not depend on the storage order.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


@dataclass(frozen=True)
class GemmCase:
    name: str
    M: int
    N: int
    K: int
    ab: str = "f16"          # operand dtype: "f16" | "bf16"
    c: str = "f16"           # output dtype: "f16" | "bf16" | "f32"
    transpose_A: int = 0
    transpose_B: int = 0
    relu: int = 0
    clear_accum: int = 1
    dist: str = "uniform"    # "uniform" | "normal" | "smallint"
    seed: int = 0
    lo: int = -4             # smallint range
    hi: int = 4
    note: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def a_shape(self):
        return (self.K, self.M) if self.transpose_A else (self.M, self.K)

    @property
    def b_shape(self):
        return (self.N, self.K) if self.transpose_B else (self.K, self.N)

    def elem_bytes(self, which: str) -> int:
        d = self.c if which == "c" else self.ab
        return 4 if d == "f32" else 2

    @property
    def algorithmic_bytes(self) -> int:
        """One read of A and B and one write of C (plus a read of C when accumulating)."""
        sa = self.elem_bytes("a")
        sc = self.elem_bytes("c")
        c_reads = 0 if self.clear_accum else sc * self.M * self.N
        return sa * self.M * self.K + sa * self.K * self.N + sc * self.M * self.N + c_reads

    def with_(self, **kw) -> "GemmCase":
        return replace(self, **kw)


# The five workloads of the method (the fifth is a pair).  Seeds are 1000 + index.
CONFIGS = {
    "c1": GemmCase("c1", 256, 256, 256, relu=1, dist="uniform", seed=1001,
                   note="C=ReLU(A·B) 256^3 fp16, uniform [-1,1]"),
    "c2": GemmCase("c2", 1024, 1024, 1024, relu=0, dist="uniform", seed=1002,
                   note="C=A·B 1024^3 fp16, uniform [-1,1] (quickstart tile example)"),
    "c3": GemmCase("c3", 4096, 4096, 4096, relu=1, dist="normal", seed=1003,
                   note="C=ReLU(A·B) 4096^3 fp16, normal(0,1)/sqrt(K)"),
    "c4": GemmCase("c4", 1000, 1500, 777, ab="bf16", c="f32", transpose_B=1,
                   dist="uniform", seed=1004,
                   note="ragged 1000x1500x777 bf16, B stored NxK, fp32 out"),
    "c5a": GemmCase("c5a", 8192, 8192, 8192, dist="normal", seed=1005,
                    note="8192^3 fp16, normal(0,1)/sqrt(K)"),
    "c5b": GemmCase("c5b", 16, 16384, 8192, transpose_B=1, dist="uniform", seed=1006,
                    note="skinny 16x16384x8192 fp16, B stored NxK (HBM-bound)"),
}


def _draw(shape, case: GemmCase, g: torch.Generator) -> torch.Tensor:
    if case.dist == "uniform":
        x = torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    elif case.dist == "normal":
        x = torch.randn(shape, generator=g, dtype=torch.float32) / math.sqrt(max(case.K, 1))
    elif case.dist == "smallint":
        x = torch.randint(case.lo, case.hi + 1, shape, generator=g, dtype=torch.int64).to(torch.float32)
    else:
        raise ValueError(f"unknown distribution {case.dist!r}")
    return x


def make_inputs(case: GemmCase, with_c: bool | None = None):
    """Return CPU tensors (A, B, C_in) in stored shapes; C_in is None when clear_accum."""
    g = torch.Generator().manual_seed(case.seed)
    dt = DTYPES[case.ab]
    A = _draw(case.a_shape, case, g).to(dt).contiguous()
    B = _draw(case.b_shape, case, g).to(dt).contiguous()
    need_c = (not case.clear_accum) if with_c is None else with_c
    C = _draw((case.M, case.N), case, g).to(DTYPES[case.c]).contiguous() if need_c else None
    return A, B, C


def bits16(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a CPU fp16/bf16 tensor as a flat uint16 array (no copy of values' meaning)."""
    assert t.dtype in (torch.float16, torch.bfloat16)
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)


def raw_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of an fp16/bf16/fp32 CPU tensor (uint16 or uint32 flat array)."""
    if t.dtype == torch.float32:
        return t.contiguous().view(torch.int32).numpy().view(np.uint32).reshape(-1)
    return bits16(t)


def sample_points(M: int, N: int, count: int, seed: int = 7):
    """Output coordinates for sampled checks: the four corners, the last row/column, plus random points."""
    rng = np.random.default_rng(seed)
    ms = [0, 0, M - 1, M - 1]
    ns = [0, N - 1, 0, N - 1]
    extra = max(count - 4, 0)
    ms += list(rng.integers(0, M, extra))
    ns += list(rng.integers(0, N, extra))
    return np.asarray(ms, dtype=np.int64), np.asarray(ns, dtype=np.int64)


# ---------------------------------------------------------------------------
# Block-scaled ("MX") operands: FP8 elements (E4M3 or E5M2) in which every 32
# consecutive elements along K share one E8M0 power-of-two scale.  Both A and B
# are stored K-contiguous (A [M, K], B [N, K]); the scales are [M, K/32] and
# [N, K/32] bytes.
#
# Recipe (the pages give the format, not a generator; this is the reading used):
#   * the same seeded CPU generator, drawing A's values, then B's, then the
#     prior C when needed, as float32 ("normal": A ~ N(0,1)/sqrt(K), B ~ N(0,1),
#     so C is O(1); "uniform": U[-1, 1) for both);
#   * per block of 32 values, the shared exponent X = floor(log2(max |v|)) minus
#     the element format's largest exponent (8 for E4M3, 15 for E5M2), the usual
#     way of converting to a block-scaled format; the scale byte is X + 127;
#   * elements v / 2^X, clamped to the format's largest finite value, cast to
#     FP8 with torch's round-to-nearest-even conversion;
#   * "smallint": elements are integers drawn from [lo, hi] (exact in both FP8
#     formats) and scale bytes are drawn from [125, 129], so every product is an
#     exact multiple of 2^-4 and the fp32 sums are exact.
# ---------------------------------------------------------------------------
FP8_DTYPES = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FP8_EMAX = {"e4m3": 8, "e5m2": 15, "e2m1": 2}
FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0, "e2m1": 6.0}
# MXFP4: E2M1 elements (the magnitudes of codes 0..7), two per byte, element 2i in
# the low nibble of byte i.  torch has no conversion to this format, so values are
# rounded to the nearest magnitude here, ties to the even code (RNE).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_codes(x: torch.Tensor) -> np.ndarray:
    """Round-to-nearest-even E2M1 codes of finite values with |x| <= 6."""
    v = np.asarray(x, dtype=np.float64)
    a = np.abs(v)
    d = np.abs(a[..., None] - E2M1_MAGNITUDES)                 # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    tie_ok = d == best
    # among equally near magnitudes take the even code (codes 0..7 in magnitude order)
    even = tie_ok & ((np.arange(8) % 2) == 0)
    code = np.where(even.any(axis=-1), even.argmax(axis=-1), tie_ok.argmax(axis=-1)).astype(np.uint8)
    return code | (np.signbit(v) & (code > 0)).astype(np.uint8) << 3


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """[rows, K] codes 0..15 -> [rows, K/2] bytes (element 2i in the low nibble of byte i)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


@dataclass(frozen=True)
class MxCase:
    name: str
    M: int
    N: int
    K: int
    fmt: str = "e4m3"        # element format of A and B: "e4m3", "e5m2" or "e2m1" (MXFP4, packed)
    c: str = "f16"
    relu: int = 0
    clear_accum: int = 1
    dist: str = "normal"     # "normal" | "uniform" | "smallint"
    seed: int = 0
    lo: int = -4
    hi: int = 4
    note: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """One read of A, B and their scales, one write of C (plus a read when accumulating)."""
        sc = 4 if self.c == "f32" else 2
        c_reads = 0 if self.clear_accum else sc * self.M * self.N
        elem = self.K // 2 if self.fmt == "e2m1" else self.K
        return (self.M + self.N) * elem + (self.M + self.N) * (self.K // 32) + sc * self.M * self.N + c_reads

    def with_(self, **kw) -> "MxCase":
        return replace(self, **kw)


MX_CONFIGS = {
    "mx1": MxCase("mx1", 256, 256, 256, relu=1, seed=1101,
                  note="C=ReLU(A·B) 256^3 MXFP8 (E4M3, E8M0 scales per 32 of K), fp16 out"),
    "mx2": MxCase("mx2", 1000, 1500, 768, fmt="e5m2", c="f32", dist="uniform", seed=1102,
                  note="ragged 1000x1500x768 MXFP8 (E5M2), fp32 out"),
    "mx3": MxCase("mx3", 8192, 8192, 8192, seed=1103,
                  note="8192^3 MXFP8 (E4M3, E8M0 scales per 32 of K), fp16 out"),
    "mx4": MxCase("mx4", 256, 256, 256, fmt="e2m1", relu=1, seed=1104,
                  note="C=ReLU(A·B) 256^3 MXFP4 (E2M1, E8M0 scales per 32 of K), fp16 out"),
    "mx5": MxCase("mx5", 1000, 1500, 768, fmt="e2m1", c="f32", dist="uniform", seed=1105,
                  note="ragged 1000x1500x768 MXFP4 (E2M1), fp32 out"),
    "mx6": MxCase("mx6", 8192, 8192, 8192, fmt="e2m1", seed=1106,
                  note="8192^3 MXFP4 (E2M1, E8M0 scales per 32 of K), fp16 out"),
}


def _mx_quantize(v: torch.Tensor, fmt: str, g: torch.Generator, case: MxCase):
    rows, K = v.shape
    if case.dist == "smallint":
        elems = torch.randint(case.lo, case.hi + 1, (rows, K), generator=g).to(torch.float32)
        scales = torch.randint(125, 130, (rows, K // 32), generator=g).to(torch.uint8)
    else:
        blocks = v.reshape(rows, K // 32, 32)
        amax = blocks.abs().amax(dim=2).clamp_min(2.0 ** -100)
        X = torch.floor(torch.log2(amax)) - FP8_EMAX[fmt]
        X = X.clamp(-127, 127)
        scales = (X + 127).to(torch.uint8)
        elems = (blocks / torch.exp2(X).unsqueeze(2)).clamp(-FP8_MAX[fmt], FP8_MAX[fmt]).reshape(rows, K)
    if fmt == "e2m1":
        q = torch.from_numpy(pack_e2m1(e2m1_codes(elems.numpy()))).contiguous()
    else:
        q = elems.to(FP8_DTYPES[fmt]).view(torch.uint8).contiguous()
    return q, scales.contiguous()


def make_mx_inputs(case: MxCase, with_c: bool | None = None):
    """CPU uint8 tensors (A [M,K], SA [M,K/32], B [N,K], SB [N,K/32]; A [M,K/2] and
    B [N,K/2] packed for E2M1) and the prior C (or None when clear_accum)."""
    if case.K % 32:
        raise ValueError("block-scaled operands need K % 32 == 0")
    g = torch.Generator().manual_seed(case.seed)
    if case.dist == "uniform":
        va = torch.rand((case.M, case.K), generator=g) * 2.0 - 1.0
        vb = torch.rand((case.N, case.K), generator=g) * 2.0 - 1.0
    elif case.dist in ("normal", "smallint"):
        va = torch.randn((case.M, case.K), generator=g) / math.sqrt(max(case.K, 1))
        vb = torch.randn((case.N, case.K), generator=g)
    else:
        raise ValueError(f"unknown distribution {case.dist!r}")
    A, SA = _mx_quantize(va, case.fmt, g, case)
    B, SB = _mx_quantize(vb, case.fmt, g, case)
    need_c = (not case.clear_accum) if with_c is None else with_c
    C = None
    if need_c:
        C = (torch.rand((case.M, case.N), generator=g) * 2.0 - 1.0).to(DTYPES[case.c]).contiguous()
    return A, SA, B, SB, C


# ---------------------------------------------------------------------------
# Attention forward (the FlashAttention tile program of the handbook page,
# section "FlashAttention: online softmax as tile code"): Q, K, V and O are
# [batch, seq, heads, dim] tensors of fp16 (or bf16), as on that page.
#
# Recipe (the page gives shapes, not values; this is the reading used):
#   * the same seeded CPU generator, drawing Q, then K, then V as float32;
#   * "normal": i.i.d. N(0, 1) entries, so with the page's scale 1/sqrt(dim)
#     the scores are O(1) and the softmax is neither flat nor one-hot;
#   * "uniform_keys": K all zeros (every allowed key gets the same weight, so
#     the output is the mean of the allowed V rows), Q and V N(0, 1);
#   * then a round-to-nearest-even cast to the operand dtype on the CPU; the
#     rounded bits are the inputs of both sides.
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class AttnCase:
    name: str
    B: int
    S: int
    H: int
    D: int
    causal: int = 1
    dtype: str = "f16"
    dist: str = "normal"     # "normal" | "uniform_keys" | "flat_int_values" | "dyadic_scores" | "ramp_up" | "ramp_down"
    scale: float | None = None   # None: 1/sqrt(D), the page's choice
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.D) if self.scale is None else float(self.scale)

    @property
    def shape(self):
        return (self.B, self.S, self.H, self.D)

    @property
    def flops(self) -> int:
        """Two products of 2*D flops per allowed (query, key) pair."""
        pairs = self.S * (self.S + 1) // 2 if self.causal else self.S * self.S
        return 4 * self.D * pairs * self.B * self.H

    @property
    def algorithmic_bytes(self) -> int:
        """One read of Q, K and V and one write of O."""
        return 4 * self.B * self.S * self.H * self.D * 2

    def with_(self, **kw) -> "AttnCase":
        return replace(self, **kw)


ATTN_CONFIGS = {
    "fa1": AttnCase("fa1", 1, 1024, 8, 64, causal=1, seed=1201,
                    note="causal attention, batch 1, seq 1024, 8 heads, dim 64 (the page's instance), fp16"),
    "fa2": AttnCase("fa2", 2, 777, 3, 128, causal=0, seed=1202,
                    note="non-causal attention, ragged seq 777, dim 128, fp16"),
    "fa3": AttnCase("fa3", 4, 4096, 32, 128, causal=1, seed=1203,
                    note="causal attention, batch 4, seq 4096, 32 heads, dim 128, fp16"),
    "fa4": AttnCase("fa4", 4, 4096, 32, 64, causal=1, seed=1204,
                    note="causal attention, batch 4, seq 4096, 32 heads, dim 64, fp16"),
}


def make_attn_inputs(case: AttnCase):
    """CPU tensors Q, K, V of shape [B, S, H, D] in the case's dtype."""
    g = torch.Generator().manual_seed(case.seed)
    q = torch.randn(case.shape, generator=g)
    k = torch.randn(case.shape, generator=g)
    v = torch.randn(case.shape, generator=g)
    if case.dist == "uniform_keys":
        k = torch.zeros(case.shape)
    elif case.dist == "flat_int_values":
        # Every score is zero and V holds small integers: each allowed key gets
        # probability 1 exactly, so O is the exact mean of V's integers over the
        # allowed keys, rounded once to the operand type.
        k = torch.zeros(case.shape)
        v = torch.randint(-4, 5, case.shape, generator=g).to(torch.float32)
    elif case.dist == "dyadic_scores":
        # Integer scores in [-6, 0] with every row's maximum 0 at key 0: query i's
        # score for key j is k[j,0] + q[i,1] k[j,1] with q[i,0] = 1, q[i,1] in {0, 1},
        # k[j,0] in [-4, 0], k[j,1] in [-2, 0] and key 0 all zero (the other
        # coordinates of Q are arbitrary, those of K zero).  With the scale ln 2 the
        # probabilities are exact powers of two in [2^-6, 1]; V holds integers in
        # [-4, 4], so every sum over keys is exact in fp32.
        q = torch.randint(-3, 4, case.shape, generator=g).to(torch.float32)
        q[..., 0] = 1.0
        q[..., 1] = torch.randint(0, 2, case.shape[:3], generator=g).to(torch.float32)
        k = torch.zeros(case.shape)
        k[..., 0] = torch.randint(-4, 1, case.shape[:3], generator=g).to(torch.float32)
        k[..., 1] = torch.randint(-2, 1, case.shape[:3], generator=g).to(torch.float32)
        k[:, 0] = 0.0
        v = torch.randint(-4, 5, case.shape, generator=g).to(torch.float32)
    elif case.dist in ("ramp_up", "ramp_down"):
        # Scores that rise (fall) by about 0.2 in log2 units per key position: every
        # query is close to the first axis and key j's first coordinate is j steps.
        sign = 1.0 if case.dist == "ramp_up" else -1.0
        step = sign * 0.2 / (math.log2(math.e) * case.softmax_scale)
        q = 0.1 * q
        q[..., 0] = 1.0
        k = 0.1 * k
        k[..., 0] = step * torch.arange(case.S, dtype=torch.float32).view(1, case.S, 1)
    elif case.dist != "normal":
        raise ValueError(f"unknown distribution {case.dist!r}")
    dt = DTYPES[case.dtype]
    return q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous()


def sample_attn_rows(case: AttnCase, count: int, seed: int = 11):
    """Output rows (b, i, h) for sampled checks: the first and last query of the first and
    last (batch, head), plus random rows."""
    rng = np.random.default_rng(seed)
    pb = [0, 0, case.B - 1, case.B - 1]
    pi = [0, case.S - 1, 0, case.S - 1]
    ph = [0, 0, case.H - 1, case.H - 1]
    extra = max(count - 4, 0)
    pb += list(rng.integers(0, case.B, extra))
    pi += list(rng.integers(0, case.S, extra))
    ph += list(rng.integers(0, case.H, extra))
    return tuple(np.asarray(x, dtype=np.int64) for x in (pb, pi, ph))


# ---------------------------------------------------------------------------
# Dequant GEMM with 4-bit weights (the pages' "dequant GEMM": packed weights,
# scale / zero point, convert, multiply): C = act(A W^T) with A [M, K] in the
# operand dtype and W given as 4-bit codes [N, K/2] bytes, scales [N, K/G] in
# the operand dtype and zero points [N, K/G] uint8.  pack_w4 below is the one
# writer of the packed layout (8 codes of k = 8w..8w+7 per little-endian 32-bit
# word, even k in the low half-word at nibbles 0..3, odd k in the high
# half-word at nibbles 4..7).
#
# Recipe (the pages give no quantizer; this is the usual asymmetric one):
#   * the same seeded CPU generator draws A (uniform in [-1, 1)) and then the
#     float weights (N(0, 1));
#   * per row and group of G weights: s = (max - min) / 15 rounded to the
#     operand dtype (1 when the group is constant), z = round(-min / s) clamped
#     to 0..15, q = round(w / s) + z clamped to 0..15;
#   * "smallint": A holds integers in [lo, hi], codes are uniform in 0..15,
#     every scale is 1 and every zero point 8, so the weights are the integers
#     q - 8 and the fp32 sums are exact.
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class W4Case:
    name: str
    M: int
    N: int
    K: int
    G: int = 128
    ab: str = "f16"
    c: str = "f16"
    relu: int = 0
    dist: str = "normal"     # "normal" | "smallint" | "smallint_groups"
    seed: int = 0
    lo: int = -4
    hi: int = 4
    note: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """One read of A, the packed weights, scales and zero points; one write of C."""
        sc = 4 if self.c == "f32" else 2
        kg = self.K // self.G
        return 2 * self.M * self.K + self.N * self.K // 2 + 3 * self.N * kg + sc * self.M * self.N

    def with_(self, **kw) -> "W4Case":
        return replace(self, **kw)


W4_CONFIGS = {
    "w4a": W4Case("w4a", 16, 16384, 8192, seed=1501,
                  note="decode-shaped C = A W^T, 16 x 16384 x 8192, 4-bit weights in groups of 128, fp16"),
    "w4b": W4Case("w4b", 5, 1000, 768, G=64, ab="bf16", c="f32", relu=1, seed=1502,
                  note="ragged 5 x 1000 x 768, groups of 64, bf16 activations, fp32 out, ReLU"),
    "w4c": W4Case("w4c", 40, 4096, 4096, G=32, c="bf16", seed=1503,
                  note="40 x 4096 x 4096 (three 16-row tiles), groups of 32, fp16 in, bf16 out"),
}


def pack_w4(q: np.ndarray) -> np.ndarray:
    """[N, K] codes in 0..15 -> [N, K/2] bytes in the packed layout described above."""
    q = np.asarray(q, dtype=np.uint32)
    N, K = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    g = q.reshape(N, K // 8, 8)
    word = np.zeros((N, K // 8), dtype=np.uint32)
    for j in range(8):
        shift = 4 * (j // 2) + (16 if j % 2 else 0)
        word |= (g[:, :, j] & 15) << shift
    return word.astype("<u4").view(np.uint8).reshape(N, K // 2)


def make_w4_inputs(case: W4Case):
    """CPU tensors: A [M, K] (operand dtype), Wq [N, K/2] uint8, S [N, K/G] (operand dtype),
    Z [N, K/G] uint8; plus the codes [N, K] (uint8) for tests of the format."""
    if case.K % case.G or case.K % 8:
        raise ValueError("K must be a multiple of the group size and of 8")
    g = torch.Generator().manual_seed(case.seed)
    dt = DTYPES[case.ab]
    N, K, G = case.N, case.K, case.G
    if case.dist == "smallint":
        A = torch.randint(case.lo, case.hi + 1, (case.M, K), generator=g).to(dt)
        q = torch.randint(0, 16, (N, K), generator=g).to(torch.uint8)
        S = torch.ones((N, K // G), dtype=dt)
        Z = torch.full((N, K // G), 8, dtype=torch.uint8)
    elif case.dist == "smallint_groups":
        # Integers, with a power-of-two scale in {1/2, 1, 2, 4} and a zero point in
        # 0..15 drawn per row and group: every weight (q - z) s is a multiple of 1/2
        # of magnitude at most 60, exact in fp16 and bf16, so sums stay exact while
        # every group's own scale and zero point matter.
        A = torch.randint(case.lo, case.hi + 1, (case.M, K), generator=g).to(dt)
        q = torch.randint(0, 16, (N, K), generator=g).to(torch.uint8)
        S = torch.pow(2.0, torch.randint(-1, 3, (N, K // G), generator=g).to(torch.float32)).to(dt)
        Z = torch.randint(0, 16, (N, K // G), generator=g).to(torch.uint8)
    elif case.dist == "normal":
        A = (torch.rand((case.M, K), generator=g) * 2.0 - 1.0).to(dt)
        w = torch.randn((N, K), generator=g).reshape(N, K // G, G)
        mn, mx = w.amin(dim=2), w.amax(dim=2)
        s = ((mx - mn) / 15.0).to(dt)
        s = torch.where(s.float() > 0, s, torch.ones_like(s))
        sf = s.float()
        z = torch.clamp(torch.round(-mn / sf), 0, 15)
        q = torch.clamp(torch.round(w / sf.unsqueeze(2)) + z.unsqueeze(2), 0, 15).to(torch.uint8).reshape(N, K)
        S, Z = s.contiguous(), z.to(torch.uint8).contiguous()
    else:
        raise ValueError(f"unknown distribution {case.dist!r}")
    Wq = torch.from_numpy(pack_w4(q.numpy()))
    return A.contiguous(), Wq.contiguous(), S.contiguous(), Z.contiguous(), q


# ---------------------------------------------------------------------------
# 2:4 structured-sparse GEMM: C = act(A W^T) with W [N, K] holding at most two
# values in every group of four consecutive k, given compressed (compress_24
# below is the one writer of the metadata): Wv [N, K/2] values in the operand
# dtype, two per group in order; Wm [N, K/8] bytes, group q's two positions at
# bits 4*(q%2) and 4*(q%2) + 2 of byte q/2 of the row.
#
# Recipe: the seeded generator draws A (uniform in [-1, 1), or N(0,1)/sqrt(K/2)
# for "normal"), then per group two distinct positions (uniform, ascending) and
# their values (uniform in [-1, 1), or N(0, 1)); "smallint": integer A and values.
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class SpCase:
    name: str
    M: int
    N: int
    K: int
    ab: str = "f16"
    c: str = "f16"
    relu: int = 0
    dist: str = "uniform"    # "uniform" | "normal" | "smallint"
    seed: int = 0
    lo: int = -4
    hi: int = 4
    note: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        """Multiply-adds with the stored (nonzero) weights only: 2 * M * N * K/2."""
        return self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        sc = 4 if self.c == "f32" else 2
        return 2 * self.M * self.K + self.N * self.K + self.N * self.K // 8 + sc * self.M * self.N

    def with_(self, **kw) -> "SpCase":
        return replace(self, **kw)


SP_CONFIGS = {
    "sp1": SpCase("sp1", 256, 256, 256, relu=1, seed=1601,
                  note="C=ReLU(A W^T) 256^3 with 2:4 sparse W, fp16"),
    "sp2": SpCase("sp2", 1000, 1500, 768, ab="bf16", c="f32", seed=1602,
                  note="ragged 1000x1500x768, 2:4 sparse W, bf16 in, fp32 out"),
    "sp3": SpCase("sp3", 8192, 8192, 8192, dist="normal", seed=1603,
                  note="8192^3 with 2:4 sparse W (4096 stored values per row), fp16"),
}


def compress_24(positions: np.ndarray) -> np.ndarray:
    """Positions [N, K/2] (0..3; two per group of four k, in the order of the stored
    values) -> Wm [N, K/8] uint8."""
    pos = np.asarray(positions, dtype=np.uint8) & 3
    N, H = pos.shape
    if H % 4:
        raise ValueError("K must be a multiple of 8")
    p = pos.reshape(N, H // 4, 4)            # two groups (four positions) per byte
    return (p[:, :, 0] | (p[:, :, 1] << 2) | (p[:, :, 2] << 4) | (p[:, :, 3] << 6)).astype(np.uint8)


def make_sp_inputs(case: SpCase):
    """CPU tensors A [M, K], Wv [N, K/2] (operand dtype), Wm [N, K/8] uint8, plus the dense
    weights [N, K] as float64 (for tests of the format)."""
    if case.K % 8:
        raise ValueError("K must be a multiple of 8")
    g = torch.Generator().manual_seed(case.seed)
    dt = DTYPES[case.ab]
    M, N, K = case.M, case.N, case.K
    if case.dist == "smallint":
        A = torch.randint(case.lo, case.hi + 1, (M, K), generator=g).to(dt)
    elif case.dist == "normal":
        A = (torch.randn((M, K), generator=g) / math.sqrt(max(K // 2, 1))).to(dt)
    else:
        A = (torch.rand((M, K), generator=g) * 2.0 - 1.0).to(dt)
    # two distinct ascending positions per group: one of the six pairs
    pairs = torch.tensor([[0, 1], [0, 2], [0, 3], [1, 2], [1, 3], [2, 3]], dtype=torch.int64)
    choice = torch.randint(0, 6, (N, K // 4), generator=g)
    pos = pairs[choice].reshape(N, K // 2)
    if case.dist == "smallint":
        vals = torch.randint(case.lo, case.hi + 1, (N, K // 2), generator=g).to(dt)
    elif case.dist == "normal":
        vals = torch.randn((N, K // 2), generator=g).to(dt)
    else:
        vals = (torch.rand((N, K // 2), generator=g) * 2.0 - 1.0).to(dt)
    Wm = compress_24(pos.numpy())
    dense = np.zeros((N, K), dtype=np.float64)
    q = np.arange(K // 2) // 2
    rows = np.arange(N)[:, None]
    np.add.at(dense, (rows, 4 * q[None, :] + pos.numpy()), vals.double().numpy())
    return A.contiguous(), vals.contiguous(), torch.from_numpy(Wm).contiguous(), dense
