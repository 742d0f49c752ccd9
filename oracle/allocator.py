"""Host block allocator (oracle; test infrastructure only).

Semantics, as the pages state them:

* The pool is carved once into fixed-size blocks, every block threaded onto a
  free list (hnwysp.cn/news/103996 §3.2, §4.1; icman.com.cn/news/78786 §2.3).
* The free list is a queue: allocation takes the head, release returns the
  block to the tail (hnwysp.cn/news/103996 §3.4); ``PagePool.allocate_pages``
  likewise hands out the front of its list (m.lqnn.cn/news/240480 §4.2).
* Each block carries a reference count: +1 when another sequence shares it,
  -1 on release, and only a count that reaches zero returns the block
  (hnwysp.cn/news/103996 §3.3, §4.2, §4.4 ``free_block``;
  icman.com.cn/news/78786 §3.3).
* A request that cannot get every block it needs takes none and reports the
  pool as exhausted (``allocate_pages`` checks the free count first and raises,
  m.lqnn.cn/news/240480 §4.2; ``alloc_block`` returns nothing when the pool is
  full, hnwysp.cn/news/103996 §4.4).
* Decode grows a sequence one slot at a time: a free slot in the last block is
  used, otherwise a new block is appended to the table
  (hnwysp.cn/news/103996 §4.2; m.lqnn.cn/news/240480 §3.2 step 3).
* Writing into a block other sequences still reference first copies the whole
  block into a fresh one (copy-on-write, hnwysp.cn/news/103996 §3.3;
  icman.com.cn/news/78786 §3.4).

Readings where the pages are silent (listed again in the design notes):

* ``free_block``'s condition has lost its comparison operator in the text;
  it is read as "return early while the decremented count is still positive".
* A copy happens only when the count is above one at the first write into
  the block within a reservation; the last remaining holder writes in place.
* The whole reservation is all-or-nothing: the number of fresh blocks plus
  the possible copy is checked against the free count before anything moves.
"""

from __future__ import annotations

from collections import deque

# Status codes shared in meaning (not in code) with the C interface.
OK = 0
ERR_INVALID = -1
ERR_NO_BLOCKS = -2
ERR_BAD_BLOCK = -3
ERR_REFCOUNT = -4


class AllocatorError(Exception):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


class OracleAllocator:
    """FIFO free queue of block ids with per-block reference counts."""

    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocatorError(ERR_INVALID, "num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if initial_free_order is None else [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocatorError(ERR_INVALID, "initial free order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks

    # -- single blocks -------------------------------------------------
    def _check(self, b: int) -> None:
        if not (0 <= b < self.num_blocks):
            raise AllocatorError(ERR_BAD_BLOCK, f"block {b} out of range")

    def alloc(self) -> int:
        if not self.free:
            raise AllocatorError(ERR_NO_BLOCKS, "out of blocks")
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def incref(self, b: int) -> None:
        self._check(b)
        if self.ref[b] < 1:
            raise AllocatorError(ERR_REFCOUNT, f"incref of free block {b}")
        self.ref[b] += 1

    def decref(self, b: int) -> None:
        self._check(b)
        if self.ref[b] < 1:
            raise AllocatorError(ERR_REFCOUNT, f"decref of free block {b}")
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    def refcount(self, b: int) -> int:
        self._check(b)
        return self.ref[b]

    def num_free(self) -> int:
        return len(self.free)

    def available(self) -> int:
        """Blocks a reservation may take (the free queue; a prefix cache adds its evictable blocks)."""
        return len(self.free)

    def _snapshot(self):
        return deque(self.free), list(self.ref)

    def _restore(self, snap) -> None:
        self.free, self.ref = snap

    def free_list(self) -> list:
        return list(self.free)

    # -- sequences over block-table rows --------------------------------
    def _check_row(self, row, n_blocks: int) -> None:
        counts = {}
        for j in range(n_blocks):
            b = int(row[j])
            self._check(b)
            counts[b] = counts.get(b, 0) + 1
        for b, c in counts.items():
            if self.ref[b] < c:
                raise AllocatorError(ERR_REFCOUNT, f"block {b} referenced {c}x but refcount {self.ref[b]}")

    def fork(self, row, n_blocks: int) -> list:
        """Share every block of ``row`` with a new sequence (prefix hit)."""
        self._check_row(row, n_blocks)
        for j in range(n_blocks):
            self.incref(int(row[j]))
        return [int(row[j]) for j in range(n_blocks)]

    def release(self, row, n_blocks: int) -> None:
        """Drop a sequence: decrement its blocks in logical order."""
        self._check_row(row, n_blocks)
        for j in range(n_blocks):
            self.decref(int(row[j]))

    def reserve(self, row: list, cur_len: int, n_new: int):
        """Make room for positions cur_len .. cur_len+n_new-1 of one sequence.

        ``row`` is the sequence's block-table row (a Python list, grown and
        patched in place).  Returns ``(slots, cow_pairs)``: the flat slot
        ``block * block_size + position % block_size`` of every new position,
        and the (source, destination) block pairs that must be copied before
        the new rows are written.
        """
        bs = self.block_size
        if cur_len < 0 or n_new < 0:
            raise AllocatorError(ERR_INVALID, "negative length")
        if len(row) != -(-cur_len // bs):
            raise AllocatorError(ERR_INVALID, "row length does not match cur_len")
        self._check_row(row, len(row))
        end = cur_len + n_new
        fresh = -(-end // bs) - len(row)
        # A partially filled block that is shared must be copied before the write.
        cow = 0
        if n_new > 0 and cur_len % bs != 0 and self.ref[row[cur_len // bs]] > 1:
            cow = 1
        if fresh + cow > self.available():
            raise AllocatorError(ERR_NO_BLOCKS, "out of blocks")
        slots, pairs = [], []
        written = set()
        for p in range(cur_len, end):
            j = p // bs
            if j == len(row):
                row.append(self.alloc())
                written.add(j)
            elif j not in written:
                written.add(j)
                src = row[j]
                if self.ref[src] > 1:
                    dst = self.alloc()
                    pairs.append((src, dst))
                    self.decref(src)
                    row[j] = dst
            slots.append(row[j] * bs + p % bs)
        return slots, pairs

    def reserve_batch(self, rows: list, cur_lens, n_new):
        """Reserve for several sequences in ascending index order, all or nothing."""
        snap = self._snapshot()
        saved_rows = [list(r) for r in rows]
        slots, pairs = [], []
        try:
            for i, row in enumerate(rows):
                s, p = self.reserve(row, int(cur_lens[i]), int(n_new[i]))
                slots.extend(s)
                pairs.extend(p)
        except AllocatorError:
            self._restore(snap)
            for r, old in zip(rows, saved_rows):
                r[:] = old
            raise
        return slots, pairs
