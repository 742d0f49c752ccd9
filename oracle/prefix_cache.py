"""Block-level prefix cache over the block allocator (oracle; test infrastructure only).

What the pages specify:

* Cached KV is organised per block, one key per block computed from the
  token sequence itself (not a request id), with a collision-resistant hash
  such as SHA-256 (icman.com.cn/news/78786 §3.2); the block size is the
  paging block size (same section).
* Matching walks the new request's blocks from the first one and stops at
  the first miss; the hit blocks are the reusable prefix (same section;
  the lookup happens for each logical block before allocation,
  hnwysp.cn/news/103996 §4.2, §4.3; m.lqnn.cn/news/240480 §3.2 step 1).
* A hit attaches the cached block to the request's table and increments its
  count; nothing is copied (icman.com.cn/news/78786 §3.4).
* Only blocks whose count is zero may be evicted, least recently used first
  (icman.com.cn/news/78786 §3.3); zero-count blocks are the first thing the
  pool reclaims when it runs out (hnwysp.cn/news/103996 §3.5).
* Keys are extended block by block rather than recomputed from the start
  (icman.com.cn/news/78786 §4.4 second detail).

Readings where the pages leave the detail open (listed in the design notes):

* Key chaining: ``key_i = SHA-256(key_{i-1} || tokens of block i)``, tokens
  as little-endian int32, ``key_{-1}`` = 32 zero bytes.  A key therefore
  names the whole prefix up to and including its block, so equal blocks
  behind different prefixes never match.  Only full blocks get keys.
* Cached blocks whose count falls to zero stay cached and join an LRU list
  ordered by that moment; the free queue is used first, and only when it is
  empty is the least recently released cached block evicted (its key
  dropped) and handed out as a fresh block.
* ``register`` keeps the first block recorded for a key; a later block with
  the same content stays an ordinary block.  A block already holding a
  different key cannot be registered again.
"""

from __future__ import annotations

import hashlib
from collections import OrderedDict

import numpy as np

from .allocator import ERR_INVALID, ERR_NO_BLOCKS, ERR_REFCOUNT, AllocatorError, OracleAllocator

ZERO_KEY = bytes(32)


def block_keys(tokens, block_size: int) -> list:
    """Chained SHA-256 keys of the full blocks of ``tokens``."""
    toks = np.asarray(tokens, dtype="<i4")
    keys, prev = [], ZERO_KEY
    for i in range(len(toks) // block_size):
        prev = hashlib.sha256(prev + toks[i * block_size:(i + 1) * block_size].tobytes()).digest()
        keys.append(prev)
    return keys


class OracleCachingAllocator(OracleAllocator):
    """OracleAllocator plus the prefix cache: key index, per-block key, LRU of zero-count cached blocks."""

    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None):
        super().__init__(num_blocks, block_size, initial_free_order)
        self.index = {}               # key -> block
        self.key_of = {}              # block -> key
        self.lru = OrderedDict()      # zero-count cached blocks, least recently released first

    def available(self) -> int:
        return len(self.free) + len(self.lru)

    def _snapshot(self):
        return super()._snapshot(), dict(self.index), dict(self.key_of), OrderedDict(self.lru)

    def _restore(self, snap) -> None:
        base, self.index, self.key_of, self.lru = snap
        super()._restore(base)

    def alloc(self) -> int:
        if self.free:
            b = self.free.popleft()
        elif self.lru:
            b, _ = self.lru.popitem(last=False)          # evict the least recently released
            del self.index[self.key_of.pop(b)]
        else:
            raise AllocatorError(ERR_NO_BLOCKS, "out of blocks")
        self.ref[b] = 1
        return b

    def decref(self, b: int) -> None:
        self._check(b)
        if self.ref[b] < 1:
            raise AllocatorError(ERR_REFCOUNT, f"decref of free block {b}")
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                self.lru[b] = None
            else:
                self.free.append(b)

    def match(self, tokens, capacity: int) -> list:
        """Blocks of the longest cached prefix of ``tokens`` (at most ``capacity``), each incremented."""
        hits = []
        for key in block_keys(tokens, self.block_size)[:max(capacity, 0)]:
            b = self.index.get(key)
            if b is None:
                break
            hits.append(b)
        for b in hits:
            if self.ref[b] == 0:
                del self.lru[b]
            self.ref[b] += 1
        return hits

    def register(self, tokens, row, n_blocks: int, first_block: int = 0) -> int:
        """Record the full blocks ``row[first_block:]`` of a sequence under their keys; returns how many were new.

        Blocks before ``first_block`` are the ones ``match`` returned for
        these tokens; the key chain resumes from the key of the last of them.
        """
        if n_blocks > len(row):
            raise AllocatorError(ERR_INVALID, "row holds fewer blocks than n_blocks")
        n = min(n_blocks, len(tokens) // self.block_size)
        if first_block < 0 or first_block > n:
            raise AllocatorError(ERR_INVALID, "first_block out of range")
        prev = ZERO_KEY
        if first_block > 0:
            b = int(row[first_block - 1])
            if b not in self.key_of:
                raise AllocatorError(ERR_INVALID, f"block {b} before first_block is not cached")
            prev = self.key_of[b]
        toks = np.asarray(tokens, dtype="<i4")
        bs = self.block_size
        keys = []
        for i in range(first_block, n):
            prev = hashlib.sha256(prev + toks[i * bs:(i + 1) * bs].tobytes()).digest()
            keys.append(prev)
        for i, key in zip(range(first_block, n), keys):
            b = int(row[i])
            self._check(b)
            if self.ref[b] < 1:
                raise AllocatorError(ERR_REFCOUNT, f"register of free block {b}")
            if b in self.key_of and self.key_of[b] != key:
                raise AllocatorError(ERR_INVALID, f"block {b} already holds another key")
        new = 0
        for i, key in zip(range(first_block, n), keys):
            b = int(row[i])
            if key in self.index or b in self.key_of:
                continue
            self.index[key] = b
            self.key_of[b] = key
            new += 1
        return new

    def cached(self) -> int:
        return len(self.key_of)

    def lru_order(self) -> list:
        return list(self.lru)
