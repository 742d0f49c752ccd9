"""Pins of the oracle allocator: hand-derived traces, closed forms, invariants."""

import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import allocator as oa

ERR = {"REFCOUNT": oa.ERR_REFCOUNT, "BAD_BLOCK": oa.ERR_BAD_BLOCK, "NO_BLOCKS": oa.ERR_NO_BLOCKS,
       "INVALID": oa.ERR_INVALID}


@pytest.fixture(scope="module")
def traces(golden_dir):
    with open(os.path.join(golden_dir, "allocator_trace.json")) as f:
        return json.load(f)


def test_block_trace(traces):
    t = traces["blocks"]
    a = oa.OracleAllocator(t["num_blocks"], t["block_size"], t["free_order"])
    for op in t["ops"]:
        kind = op["op"]
        if "error" in op:
            with pytest.raises(oa.AllocatorError) as ei:
                if kind == "alloc":
                    a.alloc()
                else:
                    getattr(a, kind)(op["block"])
            assert ei.value.code == ERR[op["error"]]
            continue
        if kind == "alloc":
            assert a.alloc() == op["expect"]
        elif kind in ("incref", "decref"):
            getattr(a, kind)(op["block"])
        elif kind == "refcount":
            assert a.refcount(op["block"]) == op["expect"]
        elif kind == "free_list":
            assert a.free_list() == op["expect"]
        elif kind == "num_free":
            assert a.num_free() == op["expect"]


def test_sequence_trace(traces):
    t = traces["sequences"]
    a = oa.OracleAllocator(t["num_blocks"], t["block_size"], t["free_order"])
    rows, lens = {}, {}
    for op in t["ops"]:
        kind = op["op"]
        if kind == "reserve":
            row = rows.setdefault(op["seq"], [])
            before = (list(row), a.free_list(), list(a.ref))
            if "error" in op:
                with pytest.raises(oa.AllocatorError) as ei:
                    a.reserve(row, op["cur_len"], op["n_new"])
                assert ei.value.code == ERR[op["error"]]
                assert (row, a.free_list(), a.ref) == before
                continue
            slots, pairs = a.reserve(row, op["cur_len"], op["n_new"])
            assert slots == op["expect_slots"]
            assert [list(p) for p in pairs] == op["expect_pairs"]
            assert row == op["expect_row"]
            lens[op["seq"]] = op["cur_len"] + op["n_new"]
        elif kind == "fork":
            rows[op["dst"]] = a.fork(rows[op["src"]], len(rows[op["src"]]))
            assert rows[op["dst"]] == op["expect_row"]
        elif kind == "release":
            a.release(rows[op["seq"]], len(rows[op["seq"]]))
            del rows[op["seq"]]
        elif kind == "refcount":
            assert a.refcount(op["block"]) == op["expect"]
        elif kind == "free_list":
            assert a.free_list() == op["expect"]
        elif kind == "num_free":
            assert a.num_free() == op["expect"]


def test_decode_growth_one_token_at_a_time():
    # Appending one token per step takes a fresh block exactly every bs tokens
    # and fills each block's slots in order.
    bs = 8
    a = oa.OracleAllocator(16, bs, list(range(16))[::-1])
    row = []
    for p in range(50):
        slots, pairs = a.reserve(row, p, 1)
        assert pairs == []
        assert len(row) == p // bs + 1
        assert slots == [row[p // bs] * bs + p % bs]
    assert row == [15, 14, 13, 12, 11, 10, 9]
    assert a.num_free() == 16 - 7


def test_prefix_cow_closed_form():
    # One prefix of 520 tokens (33 blocks of 16, the last holding 8 tokens)
    # shared by 64 sequences, then private suffixes.  Blocks 0..31 stay
    # shared; block 32 is copied for 63 sequences and kept by the last one;
    # physical blocks = 32 + sum_i (ceil(L_i / 16) - 32).
    bs, nseq, prefix = 16, 64, 520
    rng = np.random.default_rng(123)
    suffix = rng.geometric(1 / 300, size=nseq)
    lens = prefix + suffix
    pool = 32 + int(sum(math.ceil(x / bs) - 32 for x in lens))
    a = oa.OracleAllocator(pool + 3, bs, rng.permutation(pool + 3))
    row0 = []
    slots, pairs = a.reserve(row0, 0, prefix)
    assert len(row0) == 33 and pairs == []
    rows = [row0] + [a.fork(row0, 33) for _ in range(nseq - 1)]
    assert all(a.refcount(b) == nseq for b in row0)
    shared = list(row0)
    all_pairs = []
    for i in range(nseq):
        _, pairs = a.reserve(rows[i], prefix, int(suffix[i]))
        all_pairs += pairs
    assert len(all_pairs) == nseq - 1
    assert all(src == shared[32] for src, _ in all_pairs)
    used = pool + 3 - a.num_free()
    assert used == pool
    assert a.refcount(shared[32]) == 1 and rows[-1][32] == shared[32]
    assert all(a.refcount(b) == nseq for b in shared[:32])
    assert all(r[:32] == shared[:32] for r in rows)
    # The storage claim O(N x L) -> O(L + N x dL): far fewer blocks than unshared.
    unshared = sum(math.ceil(x / bs) for x in lens)
    assert used < 0.5 * unshared


def test_all_or_nothing_reserve():
    a = oa.OracleAllocator(4, 4)
    row = []
    before = (a.free_list(), list(a.ref))
    with pytest.raises(oa.AllocatorError) as ei:
        a.reserve(row, 0, 17)  # needs 5 blocks
    assert ei.value.code == oa.ERR_NO_BLOCKS
    assert (a.free_list(), a.ref, row) == (before[0], before[1], [])
    # A shared partial block needs one copy on top of the new blocks.
    r0 = []
    a.reserve(r0, 0, 2)
    r1 = a.fork(r0, 1)
    a.alloc(), a.alloc()          # leave exactly one free block
    assert a.num_free() == 1
    with pytest.raises(oa.AllocatorError):
        a.reserve(r1, 2, 3)       # copy (1) + one new block (1) > 1 free
    assert r1 == r0 and a.refcount(r0[0]) == 2


def test_reserve_validation():
    a = oa.OracleAllocator(8, 4)
    with pytest.raises(oa.AllocatorError) as ei:
        a.reserve([], 5, 1)       # row does not cover cur_len
    assert ei.value.code == oa.ERR_INVALID
    with pytest.raises(oa.AllocatorError) as ei:
        a.release([3], 1)         # block 3 is free
    assert ei.value.code == oa.ERR_REFCOUNT
    with pytest.raises(oa.AllocatorError) as ei:
        oa.OracleAllocator(4, 4, [0, 1, 1, 2])
    assert ei.value.code == oa.ERR_INVALID


def test_batch_reserve_rolls_back():
    a = oa.OracleAllocator(3, 4)
    rows = [[], [], []]
    a.reserve(rows[0], 0, 4)
    a.reserve(rows[1], 0, 4)
    snapshot = (a.free_list(), list(a.ref), [list(r) for r in rows])
    with pytest.raises(oa.AllocatorError):
        a.reserve_batch(rows, [4, 4, 0], [1, 1, 1])   # needs 3 blocks, 1 free
    assert (a.free_list(), a.ref, rows) == snapshot


def _check_invariants(a, live_rows):
    refs = np.array(a.ref)
    in_rows = {}
    for row in live_rows.values():
        for b in row:
            in_rows[b] = in_rows.get(b, 0) + 1
    # Every reference is a table entry and vice versa.
    for b in range(a.num_blocks):
        assert refs[b] == in_rows.get(b, 0)
    free = a.free_list()
    assert len(set(free)) == len(free)
    assert not (set(free) & set(in_rows))
    assert len(free) + len(in_rows) == a.num_blocks


@settings(max_examples=150, deadline=None)
@given(st.data())
def test_random_traces_keep_invariants(data):
    nb = data.draw(st.integers(1, 24))
    bs = data.draw(st.sampled_from([1, 2, 4, 8]))
    order = data.draw(st.permutations(list(range(nb))))
    a = oa.OracleAllocator(nb, bs, order)
    rows = {}
    next_id = 0
    for _ in range(data.draw(st.integers(1, 40))):
        kind = data.draw(st.sampled_from(["new", "grow", "fork", "release"]))
        if kind == "new":
            row = []
            try:
                a.reserve(row, 0, data.draw(st.integers(0, 3 * bs)))
            except oa.AllocatorError as e:
                assert e.code == oa.ERR_NO_BLOCKS
                continue
            rows[next_id] = row
            next_id += 1
        elif rows:
            sid = data.draw(st.sampled_from(sorted(rows)))
            if kind == "grow":
                cur = data.draw(st.integers((len(rows[sid]) - 1) * bs + 1 if rows[sid] else 0, len(rows[sid]) * bs))
                try:
                    a.reserve(rows[sid], cur, data.draw(st.integers(0, 2 * bs)))
                except oa.AllocatorError as e:
                    assert e.code == oa.ERR_NO_BLOCKS
            elif kind == "fork":
                rows[next_id] = a.fork(rows[sid], len(rows[sid]))
                next_id += 1
            else:
                a.release(rows[sid], len(rows[sid]))
                del rows[sid]
        _check_invariants(a, rows)
    for sid in list(rows):
        a.release(rows[sid], len(rows[sid]))
        del rows[sid]
    # Releasing everything returns the whole pool: no leaks.
    assert a.num_free() == nb and sorted(a.free_list()) == list(range(nb))
