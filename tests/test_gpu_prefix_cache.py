"""Prefix-cache hits feeding decode attention on the GPU.

Block tables are built by the library's prefix cache (``pkv_prefix_match``,
``pkv_prefix_register``) and reservations, the K/V of the blocks that missed
are written by ``pkv_append``, and decode attention runs over those tables.
A hit maps a request's table entries onto blocks another request wrote, with
no copy (icman.com.cn/news/78786 §3.2–§3.4); the oracle side replays the same
operations on ``OracleCachingAllocator`` and ``oracle.pool`` and computes
attention by its definition.  Also checked: the tables bit-exact, the whole
pools bit-exact (untouched slots keep their NaN poison, so a hit block is
never written again), a hit on a cached block that had been released (revived
from the LRU list), and a request after its blocks were evicted.

K/V rows stand in for a model's: the row at position p of a request is a
seeded function of the request's tokens 0..p, so a block whose key (the whole
prefix) matches holds exactly the rows the new request would have computed,
and each output is also checked against contiguous attention over rows
computed from scratch.
"""

import hashlib

import numpy as np
import pytest
import torch

import paged_attention_amd as pkv
from oracle import attention as oatt
from oracle import pool as opool
from oracle import prefix_cache as opc
from tests import paged_case as pc

pytestmark = pytest.mark.gpu

DEV = "cuda"
BS, H, D, NB = 16, 8, 128, 64
SCALE = 1.0 / np.sqrt(D)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _rows(tokens, p0, p1):
    """K and V rows (fp16) of positions p0..p1-1: each a seeded function of the tokens up to it."""
    ks, vs = [], []
    toks = np.asarray(tokens, dtype="<i4")
    for p in range(p0, p1):
        seed = int.from_bytes(hashlib.blake2b(toks[: p + 1].tobytes(), digest_size=8).digest(), "little")
        g = np.random.default_rng(seed)
        ks.append(g.standard_normal((H, D), dtype=np.float32).astype(np.float16))
        vs.append(g.standard_normal((H, D), dtype=np.float32).astype(np.float16))
    if not ks:
        return np.zeros((0, H, D), np.float16), np.zeros((0, H, D), np.float16)
    return np.stack(ks), np.stack(vs)


class Side:
    """Both allocators, both pools, and the per-request tables and tokens."""

    def __init__(self):
        order = np.random.default_rng(17).permutation(NB).astype(np.int32)
        self.lib = pkv.BlockAllocator(NB, BS, order)
        self.lib.enable_prefix_cache()
        self.orc = opc.OracleCachingAllocator(NB, BS, order.tolist())
        self.kc = torch.full((NB, BS, H, D), float("nan"), dtype=torch.float16, device=DEV)
        self.vc = torch.full_like(self.kc, float("nan"))
        self.okp = np.full((NB, BS, H, D), np.nan, dtype=np.float16)
        self.ovp = self.okp.copy()
        self.rows, self.orows, self.toks, self.lens = {}, {}, {}, {}

    def admit(self, name, tokens):
        """Match the cached prefix, reserve and write the rest, register the full blocks."""
        hits = self.lib.prefix_match(tokens, 1 << 20)
        ohits = self.orc.match(tokens, 1 << 20)
        assert hits == ohits, (name, hits, ohits)
        row, orow = list(hits), list(ohits)
        cur = len(hits) * BS
        slots, pairs = self.lib.reserve(row, cur, len(tokens) - cur)
        oslots, opairs = self.orc.reserve(orow, cur, len(tokens) - cur)
        assert list(slots) == list(oslots) and row == orow and not pairs and not opairs
        self._write(oslots, *_rows(tokens, cur, len(tokens)))
        nfull = len(tokens) // BS
        new = self.lib.prefix_register(tokens, row, nfull, len(hits))
        onew = self.orc.register(tokens, orow, nfull, len(hits))
        assert new == onew
        self.rows[name], self.orows[name], self.toks[name], self.lens[name] = row, orow, list(tokens), len(tokens)
        return len(hits)

    def step(self, name, token):
        """One decode step: reserve the next position and write its rows."""
        toks = self.toks[name] + [token]
        row, orow, cur = self.rows[name], self.orows[name], self.lens[name]
        slots, pairs = self.lib.reserve(row, cur, 1)
        oslots, opairs = self.orc.reserve(orow, cur, 1)
        assert list(slots) == list(oslots) and row == orow and list(map(tuple, pairs)) == list(map(tuple, opairs))
        if opairs:   # a shared partly filled block: copy before the write
            pt = torch.tensor(np.asarray(opairs, dtype=np.int32).reshape(-1, 2), device=DEV)
            pkv.pkv_copy_blocks([self.kc], [self.vc], pt)
            opool.copy_blocks([self.okp], [self.ovp], opairs)
        self._write(oslots, *_rows(toks, cur, cur + 1))
        self.toks[name], self.lens[name] = toks, cur + 1

    def release(self, name):
        self.lib.release(self.rows.pop(name))
        orow = self.orows.pop(name)
        self.orc.release(orow, len(orow))
        del self.toks[name], self.lens[name]

    def _write(self, slots, k, v):
        if len(slots):
            st = torch.tensor(np.asarray(slots, dtype=np.int64), device=DEV)
            pkv.pkv_append(torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), st, self.kc, self.vc)
            opool.append(self.okp, self.ovp, k, v, list(slots))

    def check(self, names, label):
        """Pools and allocator state against the oracle, then decode of ``names`` against both references."""
        assert self.lib.free_list() == self.orc.free_list()
        assert self.lib.prefix_lru() == self.orc.lru_order()
        assert self.lib.prefix_cached() == self.orc.cached()
        for b in range(NB):
            assert self.lib.refcount(b) == self.orc.refcount(b)
        torch.cuda.synchronize()
        assert np.array_equal(pc.to_bits(self.kc), pc.storage_bits(self.okp))
        assert np.array_equal(pc.to_bits(self.vc), pc.storage_bits(self.ovp))
        B = len(names)
        maxb = max(len(self.rows[n]) for n in names)
        tables = np.zeros((B, maxb), dtype=np.int32)
        for i, n in enumerate(names):
            tables[i, : len(self.rows[n])] = self.rows[n]
        lens = np.array([self.lens[n] for n in names], dtype=np.int32)
        q = np.random.default_rng(len(label)).standard_normal((B, H, D), dtype=np.float32).astype(np.float16)
        out = torch.empty((B, H, D), dtype=torch.float16, device=DEV)
        pkv.pkv_attention_decode(out, torch.from_numpy(q).to(DEV), self.kc, self.vc, torch.from_numpy(tables).to(DEV),
                                 torch.from_numpy(lens).to(DEV), int(lens.max()), scale=SCALE, work_groups=24)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        ref = oatt.decode_attention(q, self.okp, self.ovp, tables, lens, "f16", SCALE)
        err = float(np.max(np.abs(got - ref)))
        assert err <= 2e-3, (label, err)
        scratch = [_rows(self.toks[n], 0, self.lens[n]) for n in names]
        ref2 = oatt.contiguous_attention(q, [s[0] for s in scratch], [s[1] for s in scratch], "f16", SCALE)
        assert float(np.max(np.abs(got - ref2))) <= 2e-3, label
        pc.record_error("prefix cache hits feeding decode (f16)", err, "f16")


def test_prefix_cache_tables_feed_decode():
    rng = np.random.default_rng(5)
    system = rng.integers(0, 32000, 64).tolist()          # a 4-block system prompt
    s = Side()
    assert s.admit("A", system + rng.integers(0, 32000, 20).tolist()) == 0   # empty cache: nothing hits
    assert s.admit("B", system + rng.integers(0, 32000, 30).tolist()) == 4   # the prompt's 4 blocks hit
    assert s.rows["B"][:4] == s.rows["A"][:4]               # the same physical blocks, no copy
    s.step("A", 7)
    s.step("B", 9)
    s.check(["A", "B"], "shared system prompt")

    # A leaves: its own full block (keyed) joins the LRU list, its partly
    # filled block returns to the free queue.  A new request with A's tokens
    # revives the cached block from the LRU list.
    a_tokens, a4 = s.toks["A"], s.rows["A"][4]
    s.release("A")
    assert s.lib.prefix_lru() == [a4]
    assert s.admit("C", a_tokens) == 5
    assert s.rows["C"][4] == a4 and s.lib.prefix_lru() == []
    s.step("C", 11)
    s.check(["B", "C"], "revived LRU block")

    # B leaves; a request of one block more than the free queue holds takes
    # the whole queue and evicts B's cached block.
    b_tokens, b4 = s.toks["B"], s.rows["B"][4]
    s.release("B")
    assert s.lib.prefix_lru() == [b4]
    n_free = len(s.lib.free_list())
    assert s.admit("D", rng.integers(0, 32000, (n_free + 1) * BS - 3).tolist()) == 0
    assert b4 in s.rows["D"] and s.lib.free_list() == [] and s.lib.prefix_lru() == []
    s.step("D", 3)
    s.check(["C", "D"], "eviction of a cached block")

    # C leaves: the prompt's blocks and A's block become evictable.  B's
    # tokens again: the prompt hits (revived), B's own block was evicted and
    # is recomputed into the free queue's block and the oldest cached block.
    c5 = s.rows["C"][5]
    s.release("C")
    assert s.lib.free_list() == [c5] and s.lib.prefix_lru() == s.orc.lru_order()
    assert s.admit("E", b_tokens) == 4
    assert s.rows["E"][4:] == [c5, a4]
    s.check(["D", "E"], "request after eviction")

    # D leaves; F forks E while E's last block is partly filled: F's first
    # write copies that block (copy-on-write), E then writes in place, and
    # the cached blocks they share stay untouched.
    s.release("D")
    s.rows["F"] = s.lib.fork(s.rows["E"])
    s.orows["F"] = s.orc.fork(s.orows["E"], len(s.orows["E"]))
    assert s.rows["F"] == s.orows["F"]
    s.toks["F"], s.lens["F"] = list(s.toks["E"]), s.lens["E"]
    s.step("F", 8)
    assert s.rows["F"][5] != s.rows["E"][5] and s.rows["F"][:5] == s.rows["E"][:5]
    s.step("E", 6)
    s.check(["E", "F"], "fork and copy-on-write over cached blocks")
