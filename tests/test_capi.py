"""CPU tests of the C-ABI library: it loads, exports every declared symbol, and its host
logic (validation, variant choice, plan geometry) behaves as documented.  No kernel is
launched: every run() call here fails validation before reaching the device."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

import tiled_dense_gemm_02_amd as tlg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tlg.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

OK, INVALID, UNSUPPORTED, NULL, MISALIGNED = 0, -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tlg_\w+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = tlg.load_library()
    names = declared_functions()
    assert "tlg_gemm_create" in names and "tlg_gemm_run" in names and "tlg_gemm_destroy" in names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in tlg.h but not exported"
    assert b"gfx950" in lib.tlg_version()


def _create(M, N, K, ab=1, c=1, tA=0, tB=0, clear=1, epi=0, variant=None):
    lib = tlg.load_library()
    h = ctypes.c_void_p()
    if variant is None:
        st = lib.tlg_gemm_create(ctypes.byref(h), M, N, K, ab, c, tA, tB, clear, epi)
    else:
        st = lib.tlg_gemm_create_variant(ctypes.byref(h), M, N, K, ab, c, tA, tB, clear, epi, variant)
    return st, h


def test_create_rejects_bad_arguments():
    lib = tlg.load_library()
    assert lib.tlg_gemm_create(None, 1, 1, 1, 1, 1, 0, 0, 1, 0) == NULL
    for args, want in [((-1, 4, 4), INVALID), ((4, -1, 4), INVALID), ((4, 4, -1), INVALID),
                       ((1 << 25, 4, 4), INVALID), ((4, 4, 1 << 23), INVALID)]:
        st, h = _create(*args)
        assert st == want and not h.value
    assert _create(4, 4, 4, ab=3)[0] == UNSUPPORTED          # fp32 operands
    assert _create(4, 4, 4, ab=7)[0] == INVALID
    assert _create(4, 4, 4, c=0)[0] == INVALID
    assert _create(4, 4, 4, tA=2)[0] == INVALID
    assert _create(4, 4, 4, clear=3)[0] == INVALID
    assert _create(4, 4, 4, epi=2)[0] == INVALID
    assert _create(4, 4, 4, variant=14)[0] == INVALID
    assert _create(4, 4, 4, variant=9)[0] == UNSUPPORTED                # the block-scaled kernel needs FP8
    assert _create(100, 100, 777, tA=1, tB=1, variant=8)[0] == UNSUPPORTED
    # forced variants that cannot run the request
    assert _create(16, 64, 777, tB=1, variant=3)[0] == UNSUPPORTED      # skinny needs K % 8 == 0
    assert _create(16, 64, 64, tB=0, variant=3)[0] == UNSUPPORTED       # skinny needs B stored [N,K]
    assert _create(100, 100, 777, variant=1)[0] == UNSUPPORTED          # 256 tile needs 128-bit loads
    # direct loads: B stored [K, N] needs N % 8 == 0; K-contiguous operands take any K
    assert _create(100, 100, 777, variant=6)[0] == UNSUPPORTED
    assert _create(100, 100, 777, tA=1, tB=1, variant=7)[0] == UNSUPPORTED
    assert _create(100, 104, 777, variant=6)[0] == OK
    assert _create(100, 100, 777, tB=1, variant=7)[0] == OK
    assert _create(100, 100, 96, variant=4)[0] == INVALID               # EMPTY is chosen, never forced
    assert lib.tlg_gemm_destroy(None) == OK


def _info(**kw):
    g = tlg.Gemm(**kw)
    return g, g.info


def test_variant_choice_and_geometry_for_the_workloads():
    import tlg_workloads as W
    C = W.CONFIGS

    def info(case, variant="auto"):
        return tlg.select(case.M, case.N, case.K, case.ab, case.c, transpose_A=case.transpose_A,
                          transpose_B=case.transpose_B, epilogue="relu" if case.relu else "none",
                          variant=variant)

    # at most 128 tiles of 128x128 with A stored [M,K]: 32x128 tiles while they fit one wave of 256
    # workgroups, else 64x128 tiles
    i = info(C["c1"])
    assert (i.variant, i.block_m, i.block_n, i.grid, i.k_tiles, i.splits) == (13, 32, 128, 16, 2, 1)
    # 1024^3: 64 tiles of 128x128 (too short a K to split) -> 256 tiles of 32x128, 8 K tiles of 128 each
    i = info(C["c2"])
    assert (i.variant, i.block_m, i.block_n, i.block_k, i.grid, i.k_tiles) == (13, 32, 128, 128, 256, 8)
    assert (i.stages, i.threads, i.lds_bytes, i.splits, i.workspace_bytes) == (4, 512, 4 * (32 + 128) * 128 * 2, 1, 0)
    i = info(C["c2"], "tile64dma")
    assert (i.variant, i.block_m, i.block_n, i.block_k, i.grid, i.k_tiles) == (10, 64, 128, 128, 128, 8)
    assert (i.stages, i.threads, i.lds_bytes, i.splits, i.workspace_bytes) == (3, 512, 3 * (64 + 128) * 128 * 2, 1, 0)
    # the boundary: 256 tiles of 32x128 take them, 257 (or 384) fall back to 64x128
    assert tlg.select(1024, 1024, 512).variant == 13
    assert tlg.select(1056, 1024, 512).variant == 10
    assert tlg.select(1024, 1536, 1024, transpose_B=True).variant == 10
    i = info(C["c2"], "tile128dma")
    assert (i.variant, i.block_m, i.grid, i.lds_bytes) == (7, 128, 64, 4 * 2 * 128 * 64 * 2)
    # A stored [K,M]: 64-row tiles of an M-contiguous operand do not exist
    assert tlg.select(1024, 1024, 1024, transpose_A=True).variant == 7
    for v in ("tile64dma", "tile32dma"):
        with pytest.raises(tlg.TlgError, match="UNSUPPORTED"):
            tlg.select(1024, 1024, 1024, transpose_A=True, variant=v)
    # B stored [K, N]: 127 rows of k apart must stay inside a 31-bit lane offset
    assert tlg.select(64, 8454656, 128, variant="tile64dma").variant == 10
    with pytest.raises(tlg.TlgError, match="UNSUPPORTED"):
        tlg.select(64, 8454664, 128, variant="tile64dma")
    assert tlg.select(64, 8454664, 128, transpose_B=True, variant="tile64dma").variant == 10
    assert tlg.select(32, 8454656, 128, variant="tile32dma").variant == 13
    with pytest.raises(tlg.TlgError, match="UNSUPPORTED"):
        tlg.select(32, 8454664, 128, variant="tile32dma")
    # B stored [N, K] is fine: 1000x1500x777 forced
    assert tlg.select(1000, 1500, 777, "bf16", "f32", transpose_B=True, variant="tile64dma").grid == 16 * 12
    # forced split: 4 ranges of 4 K tiles (256 workgroups)
    i = info(C["c2"], "tile128dma_sk")
    assert (i.variant, i.block_m, i.block_n, i.block_k, i.grid, i.k_tiles, i.splits) == (8, 128, 128, 64, 256, 4, 4)
    assert i.workspace_bytes == 64 * 4 * 128 * 128 * 4 + 256
    i = info(C["c3"])
    assert (i.variant, i.block_m, i.grid, i.k_tiles, i.lds_bytes, i.threads) == (6, 256, 256, 64, 131072, 512)
    i = info(C["c4"])
    assert (i.variant, i.vec_a, i.vec_b, i.grid, i.k_tiles, i.splits) == (10, 8, 8, 16 * 12, 7, 1)
    # forced split of 1000x1500x777: 8 x 12 = 96 tiles, 13 K tiles -> 2 ranges (7 + 6 K tiles)
    i = info(C["c4"], "tile128dma_sk")
    assert (i.variant, i.vec_a, i.vec_b, i.grid, i.k_tiles, i.splits) == (8, 8, 8, 8 * 12 * 2, 7, 2)
    i = info(C["c5a"])
    assert (i.variant, i.grid, i.k_tiles) == (6, 1024, 128)
    i = info(C["c5b"])
    assert (i.variant, i.grid, i.vec_a, i.vec_b) == (3, 256, 8, 8)
    # a plan without a workspace needs no device, and describes itself
    c5b = C["c5b"]
    assert "skinny" in tlg.Gemm(c5b.M, c5b.N, c5b.K, transpose_B=True).describe()


def test_split_k_choice():
    """Ranges of whole K tiles: ~256 workgroups, at most 8 ranges, >= 2 K tiles per range,
    no empty range; only for fewer than 128 tiles of 128x128 and at least 48 K tiles."""
    for M, N, K in [(128, 128, 64 * 64), (256, 384, 8192), (1024, 1024, 1024), (512, 512, 600),
                    (1000, 1500, 777), (128, 256, 513), (2048, 1024, 4096), (1536, 1280, 2048),
                    (1024, 1024, 3072), (1000, 1500, 3000), (640, 640, 5000), (100, 3000, 20000)]:
        i = tlg.select(M, N, K, transpose_B=True)
        tiles, kt = -(-M // 128) * -(-N // 128), -(-K // 64)
        if tiles >= 128 or kt < 48:
            assert i.splits == 1 and i.variant != 8
            continue
        s = i.splits
        per = -(-kt // s)
        assert i.variant == (8 if s > 1 else 10)
        assert 1 <= s <= 8 and per >= 2 and (s - 1) * per < kt
        assert i.k_tiles == per and i.grid == tiles * s
        assert s == 8 or tiles * s <= 256 or s == 1
        if s > 1:
            assert i.workspace_bytes == tiles * s * 128 * 128 * 4 + -(-tiles * 4 // 256) * 256
    assert tlg.select(128, 128, 4096).splits == 8
    assert tlg.select(1024, 1024, 1024, variant="tile128dma_sk").splits == 4
    lib = tlg.load_library()
    assert lib.tlg_gemm_select(None, 1, 1, 1, 1, 1, 0, 0, 1, 0, 0) == NULL
    assert lib.tlg_gemm_select(ctypes.byref(tlg.PlanInfo()), -1, 1, 1, 1, 1, 0, 0, 1, 0, 0) == INVALID


def test_wave_count_rule_between_tile_sizes():
    """From 128 tiles of 256x256 up, the wave count picks the tile size: 0.37 x (waves of
    128x128 tiles) against 0.97 x (waves of 256x256 tiles)."""
    want = {(8192, 1536, 8192): 6,     # 192 tiles of 256^2 (one partial wave) vs 3 waves of 128^2
            (3000, 3000, 3000): 6,     # 144 vs 576 (3 waves)
            (8192, 1024, 8192): 7,     # 128 tiles of 256^2 vs 512 of 128^2 (2 waves)
            (2816, 2816, 1024): 7,     # 121 tiles of 256^2: below half the chip
            (4600, 4350, 4100): 7,     # 306 (2 waves, the second nearly empty) vs 1224 (5 waves)
            (4096, 4096, 4096): 6, (8192, 8192, 8192): 6}
    for (M, N, K), v in want.items():
        assert tlg.select(M, N, K, transpose_B=(M, N, K) == (4600, 4350, 4100)).variant == v, (M, N, K)


def test_skinny_rule_for_up_to_64_rows():
    """A stored [M,K], B stored [N,K]: the skinny kernel for M <= 16 always; for 16 < M <= 32
    (32 x 64 blocks) from K = 1024 on; for 32 < M <= 64 (64 x 32 blocks) while its blocks
    fit about 1.5 rounds of the CUs, or two with K >= 4096."""
    want = {(16, 16384, 256): (3, 16), (24, 16384, 8192): (3, 32), (32, 16384, 1024): (3, 32),
            (24, 4096, 512): (13, 32), (64, 8192, 2048): (3, 64), (64, 16384, 8192): (3, 64),
            (64, 16384, 2048): (13, 32), (48, 28672, 8192): (7, 128)}
    for (M, N, K), (v, bm) in want.items():
        i = tlg.select(M, N, K, transpose_B=True)
        assert (i.variant, i.block_m) == (v, bm), (M, N, K, i.variant, i.block_m)
    # B stored [K,N]: no skinny kernel
    assert tlg.select(32, 16384, 8192).variant != 3


def test_plan_geometry_matches_the_pages_worked_figures():
    """LDS bytes and K trips of the 128x128x64 fp16 tile against the handbook's exercise answers."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "page_geometry.txt")) if l.strip() and l[0] != "#"]
    # the unsplit 128x128 direct-load ring has 4 slots, the register-staged 128x128
    # variant keeps two stages
    for variant, stages_wanted in (("tile128dma", 4), ("tile128", 2)):
        row = [r for r in rows if int(r[3]) == stages_wanted][0]
        bm, bn, bk, stages, eb, K, per_op, per_stage, total, b_off, trips = map(int, row)
        i = tlg.select(1024, 1024, K, variant=variant)
        assert (i.block_m, i.block_n, i.block_k, i.stages) == (bm, bn, bk, stages)
        assert i.lds_bytes == total and i.k_tiles == trips
        assert bm * bk * eb == per_op and per_stage == 2 * per_op
    # the three-stage figures follow from the same per-stage size
    for r in rows:
        st, tot, boff = int(r[3]), int(r[8]), int(r[9])
        assert st * per_stage == tot and st * per_op == boff


def test_run_validation_happens_before_any_launch():
    lib = tlg.load_library()
    g = tlg.Gemm(64, 64, 64)
    assert lib.tlg_gemm_run(None, 16, 16, 16, None) == NULL
    assert g.run_ptrs(0, 4096, 8192) == NULL
    assert g.run_ptrs(4096, 0, 8192) == NULL
    assert g.run_ptrs(4096, 8192, 0) == NULL
    # (every pointer set below fails validation: nothing is ever launched on them)
    # direct loads: K-contiguous A at element alignment, B stored [K, N] at 16 bytes
    assert g.info.variant == 13
    assert g.run_ptrs(4096 + 1, 1 << 20, 1 << 21) == MISALIGNED     # A not element-aligned
    assert g.run_ptrs(4096, (1 << 20) + 2, 1 << 21) == MISALIGNED   # B not 16-byte aligned
    assert g.run_ptrs(4096, (1 << 20) + 8, 1 << 21) == MISALIGNED
    assert g.run_ptrs(4096, 1 << 20, (1 << 21) + 1) == MISALIGNED   # C not element-aligned
    staged = tlg.Gemm(64, 64, 64, variant="tile128")                 # register-staged 128-bit loads
    assert staged.run_ptrs(4096 + 8, 1 << 20, 1 << 21) == MISALIGNED
    # C overlapping A or B
    assert g.run_ptrs(1 << 20, 1 << 24, (1 << 20) + 4096) == INVALID
    assert g.run_ptrs(1 << 24, 1 << 20, (1 << 20) - 64) == INVALID
    narrow = tlg.Gemm(64, 64, 63, variant="tile128")  # K % 8 != 0: 16-bit loads, 2-byte alignment
    assert narrow.info.vec_a == 1
    assert narrow.run_ptrs(4096 + 1, 1 << 20, 1 << 21) == MISALIGNED
    f32 = tlg.Gemm(64, 64, 64, out_dtype="f32")
    assert f32.run_ptrs(4096, 1 << 20, (1 << 21) + 2) == MISALIGNED
    # an empty output is a no-op plan that never touches its pointers
    assert tlg.Gemm(0, 64, 64).run_ptrs(0, 0, 0) == OK


def test_python_binding_checks_shapes_and_devices():
    import torch
    g = tlg.Gemm(8, 8, 8)
    with pytest.raises(ValueError):
        g.run(torch.zeros(8, 8, dtype=torch.float16), torch.zeros(8, 8, dtype=torch.float16),
              torch.zeros(8, 8, dtype=torch.float16))       # host tensors are refused
    with pytest.raises(tlg.TlgError):
        tlg.Gemm(-1, 8, 8)


def test_tune_validates_before_touching_a_device():
    lib = tlg.load_library()
    h = ctypes.c_void_p()
    res = (tlg.TuneResult * 4)()
    n = ctypes.c_int32(-1)
    args = (64, 64, 64, 1, 1, 0, 0, 1, 0)
    assert lib.tlg_gemm_tune(None, *args, 4096, 8192, 16384, None, 5, res, 4, ctypes.byref(n)) == NULL
    assert lib.tlg_gemm_tune(ctypes.byref(h), *args, 4096, 8192, 16384, None, 0, res, 4, ctypes.byref(n)) == INVALID
    assert lib.tlg_gemm_tune(ctypes.byref(h), *args, 4096, 8192, 16384, None, 1001, res, 4, None) == INVALID
    assert lib.tlg_gemm_tune(ctypes.byref(h), *args, 4096, 8192, 16384, None, 5, None, 4, None) == NULL
    assert lib.tlg_gemm_tune(ctypes.byref(h), -1, 64, 64, 1, 1, 0, 0, 1, 0, 4096, 8192, 16384, None, 5, res, 4,
                             ctypes.byref(n)) == INVALID
    assert lib.tlg_gemm_tune(ctypes.byref(h), 64, 64, 64, 3, 1, 0, 0, 1, 0, 4096, 8192, 16384, None, 5, res, 4,
                             None) == UNSUPPORTED
    assert lib.tlg_gemm_tune(ctypes.byref(h), *args, None, 8192, 16384, None, 5, res, 4, ctypes.byref(n)) == NULL
    assert lib.tlg_gemm_tune(ctypes.byref(h), *args, 4096, 8192, None, None, 5, res, 4, ctypes.byref(n)) == NULL
    assert not h.value and n.value == 0
    # an empty output needs no timing (and no device)
    assert lib.tlg_gemm_tune(ctypes.byref(h), 0, 64, 64, 1, 1, 0, 0, 1, 0, None, None, None, None, 5, res, 4,
                             ctypes.byref(n)) == OK
    assert h.value and n.value == 0
    info = tlg.PlanInfo()
    assert lib.tlg_gemm_query(h, ctypes.byref(info)) == OK and info.variant == 4
    assert lib.tlg_gemm_destroy(h) == OK


def test_block_scaled_plans():
    """FP8 block-scaled requests: only A [M,K], B [N,K] with whole 128-wide K tiles; the
    plan runs through tlg_gemm_run_mx only, and run-time checks precede any launch."""
    lib = tlg.load_library()
    E4M3, E5M2 = 4, 5
    i = tlg.select(8192, 8192, 8192, "e4m3", "f16", transpose_B=True)
    assert (i.variant, i.block_m, i.block_n, i.block_k, i.grid, i.k_tiles, i.threads) == (9, 256, 256, 128, 1024, 64, 512)
    assert i.lds_bytes == 2 * (2 * 256 * 128 + 2 * 256 * 4)
    i = tlg.select(1000, 1500, 768, "e5m2", "f32", transpose_B=True)
    assert (i.variant, i.grid, i.k_tiles) == (9, 4 * 6, 6)
    assert tlg.select(0, 16, 128, "e4m3", transpose_B=True).variant == 4
    for kw, want in ((dict(transpose_B=False), UNSUPPORTED), (dict(transpose_A=True, transpose_B=True), UNSUPPORTED)):
        with pytest.raises(tlg.TlgError) as e:
            tlg.select(256, 256, 256, "e4m3", **kw)
        assert e.value.status == want
    assert _create(256, 256, 96, ab=E4M3, tB=1)[0] == UNSUPPORTED            # K % 128 != 0
    assert _create(256, 256, 256, ab=E5M2, tB=1, variant=6)[0] == UNSUPPORTED  # 16-bit kernel, FP8 data
    st, h = _create(256, 256, 256, ab=E4M3, tB=1)
    assert st == OK
    try:
        # the plain run refuses a block-scaled plan; the scaled run checks its pointers
        assert lib.tlg_gemm_run(h, 4096, 8192, 1 << 20, None) == INVALID
        run = lib.tlg_gemm_run_mx
        assert run(h, 4096, 8192, 12288, 16384, None, None) == NULL
        assert run(h, 4096, None, 12288, 16384, 1 << 20, None) == NULL
        assert run(h, 4096 + 8, 8192, 12288, 16384, 1 << 20, None) == MISALIGNED   # A 16-byte aligned
        assert run(h, 4096, 8192 + 2, 12288, 16384, 1 << 20, None) == MISALIGNED   # SA 4-byte aligned
        assert run(h, 4096, 8192, 12288, 16384, (1 << 20) + 1, None) == MISALIGNED  # C element-aligned
        assert run(h, 1 << 20, 8192, 12288, 16384, (1 << 20) + 4096, None) == INVALID  # C overlaps A
        assert run(None, 1, 1, 1, 1, 1, None) == NULL
    finally:
        lib.tlg_gemm_destroy(h)
    st, h16 = _create(64, 64, 64)
    assert lib.tlg_gemm_run_mx(h16, 4096, 8192, 12288, 16384, 1 << 20, None) == INVALID
    lib.tlg_gemm_destroy(h16)
    # no tuning for the block-scaled GEMM (one kernel serves it)
    hh = ctypes.c_void_p()
    assert lib.tlg_gemm_tune(ctypes.byref(hh), 256, 256, 256, E4M3, 1, 0, 1, 1, 0, 4096, 8192, 16384, None, 3,
                             None, 0, None) == UNSUPPORTED


def test_attention_validation_happens_before_any_launch():
    """tlg_attn_fwd rejects bad requests with distinct statuses before touching a device
    (these pointers are never dereferenced)."""
    lib = tlg.load_library()
    f = lib.tlg_attn_fwd
    p = 1 << 20                                         # 16-byte aligned fake address
    ok = (p, p + (1 << 24), p + (2 << 24), p + (3 << 24))
    assert f(*ok, -1, 64, 2, 64, 1, 1, 0.125, None) == -1        # negative batch
    assert f(*ok, 1, 64, 2, 0, 1, 1, 0.125, None) == -1          # dim 0
    assert f(*ok, 1, 64, 2, 64, 1, 2, 0.125, None) == -1         # causal flag
    assert f(*ok, 1, 64, 2, 64, 1, 1, float("nan"), None) == -1  # scale
    assert f(*ok, 1, 64, 2, 64, 9, 1, 0.125, None) == -1         # unknown dtype
    assert f(*ok, 1, 64, 2, 64, 3, 1, 0.125, None) == -2         # fp32 operands
    assert f(*ok, 1, 64, 2, 64, 4, 1, 0.125, None) == -2         # FP8 operands
    assert f(*ok, 1, 64, 2, 96, 1, 1, 0.125, None) == -2         # dim 96
    assert f(*ok, 1, 1 << 22, 64, 128, 1, 1, 0.125, None) == -2  # 2^31 bytes per batch
    assert f(None, None, None, None, 0, 64, 2, 64, 1, 1, 0.125, None) == 0   # empty: nothing to do
    assert f(None, p, p, p, 1, 64, 2, 64, 1, 1, 0.125, None) == -3
    assert f(p + 8, ok[1], ok[2], ok[3], 1, 64, 2, 64, 1, 1, 0.125, None) == -4
    assert f(p, ok[1], ok[2], p + 4096, 1, 64, 2, 64, 1, 1, 0.125, None) == -1   # O overlaps Q
    fb = lib.tlg_attn_fwd_block                          # the same checks, and the block size
    assert fb(*ok, 1, 64, 2, 64, 1, 1, 0.125, 96, None) == -1
    assert fb(*ok, 1, 64, 2, 64, 1, 1, 0.125, -64, None) == -1
    assert fb(*ok, 1, 64, 2, 96, 1, 1, 0.125, 64, None) == -2
    assert fb(None, None, None, None, 0, 64, 2, 64, 1, 1, 0.125, 128, None) == 0
    assert fb(p + 8, ok[1], ok[2], ok[3], 1, 64, 2, 64, 1, 1, 0.125, 64, None) == -4
    with pytest.raises(ValueError):
        tlg.attention(torch.zeros(1, 4, 1, 64), torch.zeros(1, 4, 1, 64), torch.zeros(1, 4, 1, 64))


def test_attention_query_block_rule():
    """64 queries per workgroup while blocks of 128 would number at most 256 over all
    (batch, head) pairs, or at most 1024 for causal attention with dim 64, else 128 (host
    only)."""
    qb = tlg.attention_query_block
    assert qb(1, 1024, 8, 64, True) == 64           # the page's instance: 8 x 8 = 64 blocks of 128
    assert qb(2, 777, 3, 128, False) == 64          # 7 x 3 x 2 = 42
    assert qb(1, 2048, 16, 128, True) == 64         # 16 x 16 = 256
    assert qb(1, 2049, 16, 128, True) == 128        # 17 x 16 = 272
    assert qb(1, 2049, 16, 64, False) == 128
    assert qb(1, 2049, 16, 64, True) == 64          # causal dim 64: up to 1024 blocks
    assert qb(2, 4096, 16, 64, True) == 64          # 1024
    assert qb(2, 4097, 16, 64, True) == 128         # 1056
    assert qb(4, 4096, 32, 64, True) == 128 and qb(4, 4096, 32, 128, True) == 128
    assert qb(1, 1, 1, 64, False) == 64
    assert qb(0, 64, 2, 64, True) == 0 and qb(1, 0, 2, 64, True) == 0 and qb(1, 64, -1, 64, True) == 0
    big = (1 << 62) - 1                  # products of the factors would overflow 64 bits
    assert qb(big, big, big, 64, True) == 128 and qb(1, 128, big, 64, True) == 128


def test_dequant_and_sparse_validation_happens_before_any_launch():
    """tlg_gemm_w4 and tlg_gemm_sp reject bad requests with distinct statuses before
    touching a device (these pointers are never dereferenced)."""
    lib = tlg.load_library()
    p = 1 << 20
    a, w, s, z, c = p, p + (1 << 24), p + (2 << 24), p + (3 << 24), p + (4 << 24)
    w4 = lib.tlg_gemm_w4
    assert w4(a, w, s, z, c, -1, 64, 256, 128, 1, 1, 0, None) == -1          # negative M
    assert w4(a, w, s, z, c, 16, 64, 256, 96, 1, 1, 0, None) == -1           # group not a multiple of 32
    assert w4(a, w, s, z, c, 16, 64, 200, 32, 1, 1, 0, None) == -1          # K % G
    assert w4(a, w, s, z, c, 16, 64, 256, 128, 3, 1, 0, None) == -1         # fp32 operands
    assert w4(a, w, s, z, c, 16, 64, 256, 128, 1, 1, 2, None) == -1         # epilogue
    assert w4(a, w, s, z, c, 16, 64, 32 * 256, 32, 1, 1, 0, None) == -2     # K / G = 256 > 255
    assert w4(None, None, None, None, None, 0, 64, 256, 128, 1, 1, 0, None) == 0
    assert w4(None, w, s, z, c, 16, 64, 256, 128, 1, 1, 0, None) == -3
    assert w4(a + 8, w, s, z, c, 16, 64, 256, 128, 1, 1, 0, None) == -4
    assert w4(a, w, s + 1, z, c, 16, 64, 256, 128, 1, 1, 0, None) == -4
    assert w4(a, w, s, z, a + 64, 16, 64, 256, 128, 1, 1, 0, None) == -1    # C overlaps A
    sp = lib.tlg_gemm_sp
    assert sp(a, w, z, c, 64, 64, -64, 1, 1, 0, None) == -1
    assert sp(a, w, z, c, 64, 64, 96, 1, 1, 0, None) == -2                 # K % 64
    assert sp(a, w, z, c, 64, 64, 128, 4, 1, 0, None) == -1                # FP8 operands
    assert sp(None, None, None, None, 0, 64, 128, 1, 1, 0, None) == 0
    assert sp(a, None, z, c, 64, 64, 128, 1, 1, 0, None) == -3
    assert sp(a, w, z + 2, c, 64, 64, 128, 1, 1, 0, None) == -4           # metadata 4-byte aligned
    assert sp(a, w, z, w + 16, 64, 64, 128, 1, 1, 0, None) == -1          # C overlaps Wv


def test_noalloc_entry_point_host_checks():
    """tlg_gemm_run_noalloc refuses bad requests before touching a device: the plan
    checks of create, the pointer checks of run, block-scaled dtypes; M or N == 0 is a
    no-op that needs no pointers."""
    lib = tlg.load_library()
    f = lib.tlg_gemm_run_noalloc
    a = ctypes.c_void_p(0x10000)
    assert f(-1, 4, 4, 1, 1, 0, 0, 1, 0, a, a, a, None) == INVALID
    assert f(4, 4, 1 << 23, 1, 1, 0, 0, 1, 0, a, a, a, None) == INVALID
    assert f(4, 4, 4, 3, 1, 0, 0, 1, 0, a, a, a, None) == UNSUPPORTED       # fp32 operands
    assert f(4, 4, 128, 4, 1, 0, 1, 1, 0, a, a, a, None) == UNSUPPORTED     # E4M3: tlg_gemm_run_mx
    assert f(4, 4, 4, 1, 1, 2, 0, 1, 0, a, a, a, None) == INVALID           # flag not 0/1
    assert f(4, 4, 4, 1, 1, 0, 0, 1, 0, None, a, a, None) == NULL
    assert f(4, 4, 4, 1, 1, 0, 0, 1, 0, a, a, None, None) == NULL
    assert f(0, 4, 4, 1, 1, 0, 0, 1, 0, None, None, None, None) == OK        # empty output: nothing to do
    # C overlapping A
    assert f(64, 64, 64, 1, 1, 0, 0, 1, 0, a, ctypes.c_void_p(0x900000), a, None) == INVALID
    assert lib.tlg_status_string(-7) == b"TLG_ERR_TOO_LARGE"
