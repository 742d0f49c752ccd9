"""Pins of the prefix-cache oracle (oracle.prefix_cache).

Checked against: a trace derived by hand from the pages' rules
(tests/golden/prefix_cache_trace.json); properties the chained keys must have
(a key names its whole prefix: equal blocks behind different prefixes differ,
a shared prefix gives shared keys, partial blocks have none); and a
brute-force model that matches whole token prefixes as tuples, with no hashing
at all, over random request traces.  Planted mistakes must fail a pin.
"""

import random
from collections import OrderedDict

import numpy as np
import pytest

from oracle import prefix_cache as opc
from oracle.allocator import AllocatorError
from tests import prefix_trace


def test_golden_trace():
    assert prefix_trace.run(lambda n, bs, order: opc.OracleCachingAllocator(n, bs, order)) == []


def test_chained_keys_name_the_whole_prefix():
    bs = 4
    a = list(range(12))
    b = [99] * 4 + list(range(4, 12))       # differs only in the first block
    ka, kb = opc.block_keys(a, bs), opc.block_keys(b, bs)
    assert len(ka) == 3 and len(set(ka)) == 3
    assert ka[0] != kb[0] and ka[1] != kb[1] and ka[2] != kb[2]   # same later blocks, different prefix
    assert opc.block_keys(a + [1, 2, 3], bs) == ka                 # a partial block has no key
    assert opc.block_keys(a[:8] + [5, 5, 5, 5], bs)[:2] == ka[:2]  # shared prefix, shared keys
    assert opc.block_keys([], bs) == [] and opc.block_keys([1, 2, 3], bs) == []
    assert all(len(k) == 32 for k in ka)


class PrefixModel:
    """Brute-force reference: the cache maps the full token prefix (a tuple)
    ending at each registered block to that block; no hashing."""

    def __init__(self, n, bs, order):
        self.bs = bs
        self.free = list(order)
        self.ref = [0] * n
        self.by_prefix = {}
        self.prefix_of = {}
        self.lru = OrderedDict()

    def available(self):
        return len(self.free) + len(self.lru)

    def alloc(self):
        if self.free:
            b = self.free.pop(0)
        else:
            b, _ = self.lru.popitem(last=False)
            del self.by_prefix[self.prefix_of.pop(b)]
        self.ref[b] = 1
        return b

    def drop(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.prefix_of:
                self.lru[b] = None
            else:
                self.free.append(b)

    def match(self, tokens, cap):
        hits = []
        for i in range(min(len(tokens) // self.bs, cap)):
            b = self.by_prefix.get(tuple(tokens[:(i + 1) * self.bs]))
            if b is None:
                break
            hits.append(b)
        for b in hits:
            if self.ref[b] == 0:
                del self.lru[b]
            self.ref[b] += 1
        return hits

    def register(self, tokens, row, n):
        new = 0
        for i in range(min(n, len(tokens) // self.bs)):
            p = tuple(tokens[:(i + 1) * self.bs])
            b = row[i]
            if p in self.by_prefix or b in self.prefix_of:
                continue
            self.by_prefix[p] = b
            self.prefix_of[b] = p
            new += 1
        return new


def _random_trace(seed, impl_factory):
    """Drive the oracle and the model with the same random requests; return (oracle, model) event logs."""
    rng = random.Random(seed)
    n, bs = rng.randint(4, 24), rng.choice([1, 2, 4])
    order = list(range(n))
    rng.shuffle(order)
    o = impl_factory(n, bs, order)
    m = PrefixModel(n, bs, order)
    vocab = [1, 2, 3]                         # tiny vocabulary: prefixes collide often
    stems = [[rng.choice(vocab) for _ in range(rng.randint(0, 12))] for _ in range(4)]
    live = []                                  # (tokens, row)
    log_o, log_m = [], []
    for _ in range(60):
        if live and rng.random() < 0.35:
            toks, row = live.pop(rng.randrange(len(live)))
            o.release(row, len(row))
            for b in row:
                m.drop(b)
            continue
        toks = list(rng.choice(stems)) + [rng.choice(vocab) for _ in range(rng.randint(0, 6))]
        cap = rng.randint(0, 8)
        ho = o.match(toks, cap)
        hm = m.match(toks, cap)
        log_o.append(("match", list(ho)))
        log_m.append(("match", list(hm)))
        row = list(ho)
        cur = len(row) * bs
        need = -(-len(toks) // bs) - len(row)
        try:
            o.reserve(row, cur, len(toks) - cur)
            ok = True
        except AllocatorError:
            ok = False
        mrow = list(hm)
        if need <= m.available():
            for _ in range(need):
                mrow.append(m.alloc())
            okm = True
        else:
            okm = False
        log_o.append(("reserve", ok, list(row)))
        log_m.append(("reserve", okm, list(mrow)))
        if not ok:
            o.release(row, len(row))
            for b in hm:
                m.drop(b)
            continue
        log_o.append(("register", o.register(toks, row, len(row), len(ho) if rng.random() < 0.5 else 0)))
        log_m.append(("register", m.register(toks, mrow, len(mrow))))
        live.append((toks, row))
        log_o.append(("state", o.free_list(), o.lru_order(), list(o.ref)))
        log_m.append(("state", list(m.free), list(m.lru), list(m.ref)))
    return log_o, log_m


@pytest.mark.parametrize("seed", range(40))
def test_matches_brute_force_prefix_model(seed):
    lo, lm = _random_trace(seed, lambda n, bs, order: opc.OracleCachingAllocator(n, bs, order))
    assert lo == lm


# Plausible mistakes, planted in copies of the oracle (never in the product).
class _Unchained(opc.OracleCachingAllocator):
    def match(self, tokens, capacity):
        return self._with_keys(super().match, tokens, capacity)

    def register(self, tokens, row, n):
        return self._with_keys(super().register, tokens, row, n)

    def _with_keys(self, fn, *args):
        saved = opc.block_keys
        opc.block_keys = lambda toks, bs: [
            __import__("hashlib").sha256(np.asarray(toks[i * bs:(i + 1) * bs], "<i4").tobytes()).digest()
            for i in range(len(toks) // bs)]
        try:
            return fn(*args)
        finally:
            opc.block_keys = saved


class _MostRecentFirst(opc.OracleCachingAllocator):
    def alloc(self):
        if not self.free and self.lru:
            b, _ = self.lru.popitem(last=True)
            del self.index[self.key_of.pop(b)]
            self.ref[b] = 1
            return b
        return super().alloc()


class _EvictFirst(opc.OracleCachingAllocator):
    def alloc(self):
        if self.lru:
            b, _ = self.lru.popitem(last=False)
            del self.index[self.key_of.pop(b)]
            self.ref[b] = 1
            return b
        return super().alloc()


class _Overwrite(opc.OracleCachingAllocator):
    def register(self, tokens, row, n):
        keys = opc.block_keys(tokens, self.block_size)[:n]
        for i, key in enumerate(keys):
            b = int(row[i])
            old = self.index.get(key)
            if old is not None and old != b:
                del self.key_of[old]
            self.index[key] = b
            self.key_of[b] = key
        return len(keys)


class _NoRevive(opc.OracleCachingAllocator):
    def match(self, tokens, capacity):
        hits = []
        for key in opc.block_keys(tokens, self.block_size)[:max(capacity, 0)]:
            b = self.index.get(key)
            if b is None:
                break
            hits.append(b)
        for b in hits:
            self.ref[b] += 1              # forgets to take the block off the LRU list
        return hits


@pytest.mark.parametrize("cls", [_Unchained, _MostRecentFirst, _EvictFirst, _Overwrite, _NoRevive])
def test_pins_catch_planted_mistakes(cls):
    make = lambda n, bs, order: cls(n, bs, order)  # noqa: E731
    caught = bool(prefix_trace.run(make))
    if not caught:
        for seed in range(40):
            try:
                lo, lm = _random_trace(seed, make)
            except Exception:
                caught = True
                break
            if lo != lm:
                caught = True
                break
    assert caught, f"{cls.__name__} passed every pin"
