"""Host grouping of sequences by shared leading blocks (pkv_prefix_tiles).

The rule, written out here in plain Python and compared with the library on
random forked tables: sequences with at least one whole block before their
last position are grouped by their first block id (groups in ascending id,
members in ascending index); a group of at least max(2, min_sharers)
members has the prefix = the longest run of leading ids every member shares
with the first one, capped for each member at (L - 1) // block_size; groups
with a prefix of at least one block are cut into tiles of 16; no prefix is
longer than 1024 blocks.
"""

import ctypes

import numpy as np
import pytest

import paged_attention_amd as pkv


def reference(tables, lens, bs, min_sharers):
    batch, maxb = tables.shape
    full = [min((int(L) - 1) // bs, maxb, 1024) if L >= 2 else 0 for L in lens]
    groups = {}
    for b in range(batch):
        if full[b] >= 1:
            groups.setdefault(int(tables[b, 0]), []).append(b)
    prefix = [0] * batch
    tiles = []
    for key in sorted(groups):
        members = groups[key]
        if len(members) < max(2, min_sharers):
            continue
        p = full[members[0]]
        for m in members[1:]:
            lim = min(p, full[m])
            lcp = 0
            while lcp < lim and tables[m, lcp] == tables[members[0], lcp]:
                lcp += 1
            p = lcp
        if p < 1:
            continue
        for k in range(0, len(members), 16):
            chunk = members[k:k + 16]
            tiles.append([p, len(chunk)] + chunk + [-1] * (16 - len(chunk)))
            for m in chunk:
                prefix[m] = p
    return np.array(prefix, dtype=np.int32), np.array(tiles, dtype=np.int32).reshape(-1, 18)


def forked_tables(rng, batch, maxb, bs, roots):
    """Rows forked from a few roots: each shares a random leading run of its root's ids."""
    next_id = [0]

    def fresh(n):
        ids = np.arange(next_id[0], next_id[0] + n, dtype=np.int32)
        next_id[0] += n
        return ids

    root_rows = [fresh(maxb) for _ in range(roots)]
    tables = np.zeros((batch, maxb), dtype=np.int32)
    lens = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        root = root_rows[rng.integers(roots)]
        keep = int(rng.integers(0, maxb + 1))
        tables[b, :keep] = root[:keep]
        tables[b, keep:] = fresh(maxb - keep)
        lens[b] = int(rng.integers(0, maxb * bs + 1))
    return tables, lens


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("bs", [8, 16, 32])
def test_matches_the_rule(seed, bs):
    rng = np.random.default_rng(seed * 31 + bs)
    batch = int(rng.integers(1, 120))
    maxb = int(rng.integers(1, 12))
    tables, lens = forked_tables(rng, batch, maxb, bs, roots=int(rng.integers(1, 5)))
    for min_sharers in (0, 2, 3, 17):
        spb, tiles = pkv.prefix_tiles(tables, lens, bs, min_sharers)
        want_spb, want_tiles = reference(tables, lens, bs, min_sharers)
        assert np.array_equal(spb, want_spb)
        assert np.array_equal(tiles, want_tiles)
        # invariants the grouped kernels rely on
        seen = set()
        for t in tiles:
            p, n, members = int(t[0]), int(t[1]), [int(x) for x in t[2:2 + t[1]]]
            assert 1 <= n <= 16 and all(x == -1 for x in t[2 + n:])
            for m in members:
                assert m not in seen
                seen.add(m)
                assert spb[m] == p and p * bs < lens[m]
                assert np.array_equal(tables[m, :p], tables[members[0], :p])
        assert seen == {b for b in range(batch) if spb[b] > 0}


def test_big_group_splits_into_tiles_and_refuses_small_output():
    bs, maxb, batch = 16, 4, 40
    tables = np.tile(np.arange(maxb, dtype=np.int32), (batch, 1))
    tables[:, 3] = 100 + np.arange(batch)          # a private last block each
    lens = np.full(batch, 3 * bs + 5, dtype=np.int32)
    spb, tiles = pkv.prefix_tiles(tables, lens, bs)
    assert np.all(spb == 3)
    assert tiles[:, 1].tolist() == [16, 16, 8]
    assert tiles[:, 2:].max() == batch - 1
    # too little room for the tiles: refused, outputs untouched
    t = np.ascontiguousarray(tables)
    ln = np.ascontiguousarray(lens)
    out_spb = np.full(batch, 7, dtype=np.int32)
    out_tiles = np.full((2, 18), 7, dtype=np.int32)
    n = ctypes.c_int32(-5)
    st = pkv._lib.pkv_prefix_tiles(t.ctypes.data, maxb, ln.ctypes.data, batch, bs, 2, out_spb.ctypes.data,
                                   out_tiles.ctypes.data, 2, ctypes.byref(n))
    assert st == pkv.PKV_ERR_INVALID and n.value == -5
    assert np.all(out_spb == 7) and np.all(out_tiles == 7)


def test_no_group_when_nothing_is_shared_or_too_short():
    bs = 16
    tables = np.arange(12, dtype=np.int32).reshape(4, 3)
    lens = np.array([40, 40, 40, 40], dtype=np.int32)
    spb, tiles = pkv.prefix_tiles(tables, lens, bs)
    assert not spb.any() and tiles.shape == (0, 18)
    tables[:] = tables[0]                            # all share every block ...
    lens[:] = bs                                     # ... but none has a whole block before its last position
    spb, tiles = pkv.prefix_tiles(tables, lens, bs)
    assert not spb.any() and tiles.shape == (0, 18)
    lens[:] = bs + 1
    spb, tiles = pkv.prefix_tiles(tables, lens, bs)
    assert spb.tolist() == [1, 1, 1, 1] and tiles.shape == (1, 18)
