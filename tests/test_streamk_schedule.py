"""CPU check of the persistent stream-K schedule (the work decomposition of the
stream-K variants): for many grids and K-tile counts, the segments that the
workgroups walk cover every (tile, K tile) exactly once, every partial segment has
its own workspace slot below 2G, the slots the electing workgroup sums are exactly
the contributors' own slots in K order, and every loop ends.  The arithmetic is the
kernel's (gemm_lds.hpp, kModeStreamK) and the plan's split into whole and shared
tiles (tlg_api.cpp, streamk_split), restated here; the plan facts themselves are
checked against tlg_gemm_select."""
from __future__ import annotations

import itertools

import pytest

import tiled_dense_gemm_02_amd as tlg

G = 256


def split(tiles, TP):
    """(whole tiles, shared tiles, persistent grid)."""
    if TP == 0:
        return tiles, 0, min(G, tiles)
    waves = tiles // G
    dp = (waves - 1) * G if waves >= 2 else 0
    sk = tiles - dp
    return dp, sk, G if dp else min(G, sk * TP)


def walk(tiles, TP):
    """Segments per workgroup: (tile, k0, tp, base, ns, self, first)."""
    dp, sk, Gp = split(tiles, TP)
    W = sk * TP
    out = {}
    G = Gp
    for g in range(G):
        ndp = (dp - g + G - 1) // G if g < dp else 0
        beg, end = g * W // G, (g + 1) * W // G
        it, j, segs = beg, 0, []
        while True:
            assert j < tiles + sk + 2, "loop must end"
            if j < ndp:
                segs.append((g + j * G, 0, TP, 0, 1, 0, 0))
            else:
                if it >= end:
                    break
                r = it // TP
                k0 = it - r * TP
                k1 = min(TP, k0 + (end - it))
                tb = r * TP
                gf, gl = ((tb + 1) * G - 1) // W, ((tb + TP) * G - 1) // W
                first = 0 if tb == gf * W // G else 1
                self = 2 * (g - gf) + (0 if it == beg else 1)
                segs.append((dp + r, k0, k1 - k0, 2 * gf, gl - gf + 1, self, first))
                it += k1 - k0
            j += 1
        out[g] = segs
    return out, dp, sk


CASES = [(t, tp) for t in (1, 5, 64, 96, 127, 200, 255, 256, 257, 306, 400, 511, 512, 513, 576, 1024, 1100)
         for tp in (0, 1, 2, 3, 13, 16, 64, 128)]


@pytest.mark.parametrize("tiles,TP", CASES)
def test_schedule_covers_every_k_tile_once(tiles, TP):
    out, dp, sk = walk(tiles, TP)
    cover = {}
    slots = {}
    finished = {}
    for g, segs in out.items():
        for (tile, k0, tp, base, ns, self, first) in segs:
            assert 0 <= tile < tiles and (tp >= 1 or TP == 0) and 0 <= k0 and k0 + tp <= TP
            if ns == 1:
                finished[tile] = finished.get(tile, 0) + 1
            for k in range(k0, k0 + tp):
                assert (tile, k) not in cover, f"tile {tile} K tile {k} twice"
                cover[(tile, k)] = g
            if ns > 1:
                slot = base + self
                assert 0 <= slot < 2 * len(out)
                assert slot not in slots, f"slot {slot} used twice"
                slots[slot] = (tile, k0)
            else:
                assert k0 == 0 and tp == TP, "a lone segment covers its whole tile"
    assert len(cover) == tiles * TP
    # the finisher of each shared tile sums exactly its contributors' slots, in K order
    by_tile = {}
    for g, segs in out.items():
        for (tile, k0, tp, base, ns, self, first) in segs:
            if ns > 1:
                by_tile.setdefault(tile, []).append((k0, base + self, base, ns, first))
    for tile, parts in by_tile.items():
        parts.sort()
        base, ns, first = parts[0][2], parts[0][3], parts[0][4]
        assert all(p[2] == base and p[3] == ns and p[4] == first for p in parts), "contributors disagree"
        assert len(parts) == ns
        want = [base + (first if s == 0 else 2 * s) for s in range(ns)]
        assert [p[1] for p in parts] == want
        finished[tile] = finished.get(tile, 0) + 1          # the one elected segment
        assert ns <= 3 or tiles < G, "at most three partial segments per tile once every workgroup has a tile"
        assert ns <= len(out)
    assert finished == {t: 1 for t in range(tiles)}, "every tile's epilogue runs exactly once"


@pytest.mark.parametrize("M,N,K,variant", [(4600, 4350, 4100, "tile256dma_streamk"),
                                           (8192, 4608, 1024, "tile256dma_streamk"),
                                           (1024, 1024, 1024, "tile128dma_streamk"),
                                           (1000, 1500, 777, "tile128dma_streamk"),
                                           (8192, 8192, 512, "tile256dma_streamk"),
                                           (300, 200, 0, "tile128dma_streamk"),
                                           (128, 128, 128, "tile128dma_streamk")])
def test_plan_facts_match_the_schedule(M, N, K, variant):
    b = 256 if variant.startswith("tile256") else 128
    tiles = -(-M // b) * -(-N // b)
    dp, sk, Gp = split(tiles, -(-K // 64))
    info = tlg.select(M, N, K, transpose_B=True, variant=variant)
    assert (info.dp_tiles, info.sk_tiles, info.grid) == (dp, sk, Gp)
    assert info.block_m == b and info.block_n == b
    ws = 2 * Gp * b * b * 4 + (-(-sk * 4 // 256)) * 256 if sk else 0
    assert info.workspace_bytes == ws


def test_streamk_refuses_what_the_direct_loads_cannot_serve():
    with pytest.raises(tlg.TlgError):
        tlg.select(1000, 1001, 64, variant="tile256dma_streamk")   # B stored [K, N] with N % 8 != 0
