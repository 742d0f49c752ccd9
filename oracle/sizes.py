"""Closed-form sizes of a paged KV cache (oracle; test infrastructure only).

Every function here is a formula the pages state in words:

* bytes per token = 2 (K and V) x layers x heads x head_dim x dtype bytes
  (icman.com.cn/news/78786 §1.1; hnwysp.cn/news/103996 §1.2 writes the same
  with hidden size = heads x head_dim; m.lqnn.cn/news/240480 §3.1 gives the
  per-layer figure).
* blocks needed by a sequence = ceil(length / block_size), and the unused
  tail of the last block is the internal fragmentation
  (icman.com.cn/news/78786 §2.1-§2.2; hnwysp.cn/news/103996 §3.1).
* pool blocks = usable bytes / (block_size x bytes per token), and the token
  capacity is blocks x block_size (icman.com.cn/news/78786 §4.1).
"""

from __future__ import annotations

import math

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "int8": 1, "fp8": 1}


def kv_bytes_per_token(num_layers: int, num_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """K plus V bytes one token occupies across all layers (icman.com.cn/news/78786 §1.1)."""
    return 2 * num_layers * num_heads * head_dim * dtype_bytes


def kv_bytes_per_token_hidden(num_layers: int, hidden: int, dtype_bytes: int) -> int:
    """Same count written with the hidden size (hnwysp.cn/news/103996 §1.2)."""
    return 2 * num_layers * hidden * dtype_bytes


def blocks_for_length(length: int, block_size: int) -> int:
    """Number of fixed-size blocks a sequence of ``length`` tokens occupies."""
    if length < 0 or block_size <= 0:
        raise ValueError("length must be >= 0 and block_size > 0")
    return -(-length // block_size)


def fragmentation_tokens(lengths, block_size: int) -> int:
    """Unused token slots in the last block of every sequence, summed.

    Internal fragmentation is the only waste of paging (icman.com.cn/news/78786
    §2.1: at most the unfilled slots of a sequence's last block).
    """
    total = 0
    for length in lengths:
        total += blocks_for_length(int(length), block_size) * block_size - int(length)
    return total


def block_bytes(block_size: int, bytes_per_token: int) -> int:
    """Bytes one physical block holds (hnwysp.cn/news/103996 §3.1: 16 x 512 KB = 8 MB)."""
    return block_size * bytes_per_token


def pool_blocks(usable_bytes: int, block_size: int, bytes_per_token: int) -> int:
    """Whole blocks that fit in ``usable_bytes`` (icman.com.cn/news/78786 §4.1)."""
    return usable_bytes // block_bytes(block_size, bytes_per_token)


def pool_token_capacity(num_blocks: int, block_size: int) -> int:
    """Tokens a pool of ``num_blocks`` blocks can hold (icman.com.cn/news/78786 §4.1)."""
    return num_blocks * block_size


def max_requests(num_blocks: int, block_size: int, tokens_per_request: int) -> int:
    """Requests of a given length that fit, ignoring per-request tail waste.

    The page divides the pooled token capacity by the average request length
    (icman.com.cn/news/78786 §4.1).
    """
    return pool_token_capacity(num_blocks, block_size) // tokens_per_request


def table_bytes(num_entries: int, entry_bytes: int) -> int:
    """Size of a block table (hnwysp.cn/news/103996 §3.1: 1M entries x 8 B)."""
    return num_entries * entry_bytes


def expected_tail_waste_fraction(block_size: int, mean_length: float) -> float:
    """Half a block per sequence over the mean length (hnwysp.cn/news/103996 §3.1).

    The page states the average tail waste is about half a block; the
    fraction of a sequence's slots wasted is then (block_size / 2) / mean.
    """
    return (block_size / 2.0) / mean_length


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def logical_kv_bytes(lengths, num_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """K+V bytes one decode call reads for one layer: sum of lengths x 2 x H x D x s."""
    return int(sum(int(x) for x in lengths)) * 2 * num_heads * head_dim * dtype_bytes


def unique_kv_bytes(block_tables, lengths, block_size: int, num_heads: int, head_dim: int,
                    dtype_bytes: int) -> int:
    """K+V bytes of the distinct token slots a decode call reads (shared blocks once)."""
    seen = set()
    for row, length in zip(block_tables, lengths):
        for t in range(int(length)):
            seen.add((int(row[t // block_size]), t % block_size))
    return len(seen) * 2 * num_heads * head_dim * dtype_bytes


def gib(x: float) -> int:
    return int(x * (1 << 30))


def mib(x: float) -> int:
    return int(x * (1 << 20))


__all__ = [name for name in dir() if not name.startswith("_") and name not in {"annotations", "math"}]
