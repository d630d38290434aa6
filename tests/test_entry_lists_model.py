"""Host model of the entry-list build in attend.hip (count, scans, fill).

The chunk pass reads, for every chunk, the (query, slot) entries that chose it,
in query order.  The library builds these lists per counting tile of queries:
per-chunk counts from 64-query bitmaps, a column scan over tiles, a scan over
chunks, then a fill.  The fill either scatters each entry to its final place or
stages the tile's entries in LDS in chunk order and writes each chunk's run
contiguously.  This model replays both fills' index arithmetic on small random
selections and checks that every LDS stage slot and every destination is in
bounds and that the two fills place every entry identically.  It also checks the
tile-size and LDS-fit rules at the benchmark shapes.
"""
import numpy as np
import pytest

SUB = 64                  # queries per ranking sub-tile
MAX_LDS = 160 * 1024      # LDS per workgroup


def idx_tile(B, Hkv, T):
    tile = 1024
    while tile > 256 and B * Hkv * ((T + tile - 1) // tile) < 1024:
        tile //= 2
    return tile


def staged_fits(NCs, tile, topk):
    return NCs * 12 + tile * topk * 4 + 256 <= MAX_LDS


def _popc(x):
    return bin(int(x)).count("1")


def _bitmap(idx, i0, NCs):
    T = idx.shape[0]
    bm = [0] * NCs
    for ql in range(SUB):
        if i0 + ql >= T:
            break
        for c in idx[i0 + ql]:
            if 0 <= c < NCs:
                bm[c] |= 1 << ql
    return bm


def build_both(idx, NCs, tile):
    """Entry arrays from the direct fill and from the staged fill, and each
    chunk's list base and length."""
    T, topk = idx.shape
    ntiles = (T + tile - 1) // tile
    cnt = np.zeros((ntiles, NCs), dtype=np.int64)
    for t in range(ntiles):
        for i0 in range(t * tile, min((t + 1) * tile, T), SUB):
            cnt[t] += [_popc(w) for w in _bitmap(idx, i0, NCs)]
    toff = np.cumsum(cnt, 0) - cnt            # column scan: each tile's offset in a chunk's list
    bcount = cnt.sum(0)
    bbase = np.cumsum(bcount) - bcount        # scan over chunks: each list's base
    total = int(bcount.sum())
    direct = np.full(total, -1, dtype=np.int64)
    staged = np.full(total, -1, dtype=np.int64)
    for t in range(ntiles):
        nxt = toff[t + 1] if t + 1 < ntiles else bcount
        counts = nxt - toff[t]
        run = np.cumsum(counts) - counts      # each chunk's start in the stage
        pos = bbase + toff[t]                 # each chunk's next place in HBM
        stage = np.full(tile * topk, -1, dtype=np.int64)
        for i0 in range(t * tile, min((t + 1) * tile, T), SUB):
            bm = _bitmap(idx, i0, NCs)
            for e in range(SUB * topk):
                ql, sl = divmod(e, topk)
                i = i0 + ql
                if i >= T:
                    break
                c = idx[i, sl]
                if c < 0 or c >= NCs:
                    continue
                rank = _popc(bm[c] & ((1 << ql) - 1))
                assert 0 <= pos[c] + rank < total
                direct[pos[c] + rank] = i * 64 + sl
                j = run[c] + rank
                assert 0 <= j < tile * topk
                stage[j] = i * 64 + sl
            p = np.array([_popc(w) for w in bm])
            run = run + p
            pos = pos + p
        for c in range(NCs):                  # chunk c's run: stage[run[c-1], run[c])
            e0 = run[c - 1] if c > 0 else 0
            for j in range(run[c] - e0):
                d = bbase[c] + toff[t][c] + j
                assert 0 <= d < total
                staged[d] = stage[e0 + j]
    return direct, staged, bbase, bcount


@pytest.mark.parametrize("T,NCs,topk,tile,seed", [
    (300, 5, 3, 256, 0),      # ragged last tile
    (1000, 13, 8, 256, 1),
    (777, 40, 16, 512, 2),
    (2100, 7, 4, 1024, 3),    # more entries per chunk than a sub-tile holds
    (129, 3, 2, 256, 4),      # one tile, a ragged sub-tile
])
def test_staged_fill_places_entries_as_direct_fill(T, NCs, topk, tile, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(-1, NCs, size=(T, topk))   # -1: padding slots
    dup = rng.random(T) < 0.1
    idx[dup, 1] = idx[dup, 0]                     # a chunk listed twice in a row counts once
    direct, staged, bbase, bcount = build_both(idx, NCs, tile)
    assert (direct >= 0).all()                    # every place is written
    assert (direct == staged).all()
    for c in range(NCs):                          # each list in query order
        q = direct[bbase[c]:bbase[c] + bcount[c]] // 64
        assert (np.diff(q) > 0).all()


def test_tile_and_fill_choice_at_benchmark_shapes():
    # 8K prefill (8 KV heads): short tiles so the grid has enough workgroups
    assert idx_tile(1, 8, 8192) == 256
    assert staged_fits(8192 // 64, 256, 16)
    # 128K prefill: 1024-query tiles, 2048 chunks, k = 32: staged fill (152 KB)
    assert idx_tile(1, 8, 131072) == 1024
    assert staged_fits(2048, 1024, 32)
    # 512K prefill: 8192 chunks leave no room for a 1024-query stage: direct fill
    assert idx_tile(1, 8, 524288) == 1024
    assert not staged_fits(8192, 1024, 32)
