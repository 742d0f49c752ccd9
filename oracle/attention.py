"""Decode attention over a paged KV cache, by its plain definition (oracle).

Test infrastructure only.  Paged attention must produce exactly what ordinary
attention over the logically contiguous cache produces: the block table only
relocates rows (hnwysp.cn/news/103996 §2.2 "logically contiguous, physically
scattered"; icman.com.cn/news/78786 §2.1, §2.4; m.lqnn.cn/news/240480 §3.3
maps logical position ``pos`` to ``(table[pos // page], pos % page)``).

For one decode query per sequence ``b`` and head ``h`` over the ``L_b``
cached tokens (the token appended this step included — the new K/V are
joined to the history before attention, hnwysp.cn/news/103996 §1.1):

    idx_t = table_b[t // bs] * bs + t % bs            t = 0 .. L_b - 1
    s_t   = scale * <q_{b,h}, K[idx_t, h]>
    w_t   = exp(s_t - max_t s_t)
    out   = sum_t w_t V[idx_t, h] / sum_t w_t

Readings (the pages never write the softmax out): base-e softmax with
``scale = 1/sqrt(head_dim)`` unless given, the usual scaled dot-product form;
``L_b = 0`` yields a zero row.  Everything is computed in float64 from inputs
upcast from their stored dtype.
"""

from __future__ import annotations

import numpy as np


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Upcast stored values to float64; bf16 arrives as its uint16 bit patterns."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype in ("f16", "f32"):
        return np.asarray(x).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype}")


def gather_indices(row, length: int, block_size: int) -> np.ndarray:
    """Flat pool slots of logical positions 0..length-1 of one sequence."""
    t = np.arange(length, dtype=np.int64)
    blocks = np.asarray(row, dtype=np.int64)[t // block_size]
    return blocks * block_size + t % block_size


def attend_one(q_vec: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """Softmax(scale * keys @ q) @ values for one query, in float64."""
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    s = scale * (keys @ q_vec)
    w = np.exp(s - s.max())
    return (w @ values) / w.sum()


def decode_attention(q, k_pool, v_pool, block_tables, seq_lens, dtype: str, scale: float | None = None,
                     heads=None) -> np.ndarray:
    """Decode attention for every sequence and head; returns float64 ``[B][H][D]``.

    ``q``: ``[B][H][D]``; pools: ``[num_blocks][block_size][H][D]``; tables:
    ``[B][max_blocks]`` int; lengths: ``[B]``.  ``heads`` restricts the heads
    computed (others stay zero) for sampled checks of large cases.
    """
    nb, bs, nh, d = k_pool.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qf = to_f64(q, dtype)
    kflat = k_pool.reshape(nb * bs, nh, d)
    vflat = v_pool.reshape(nb * bs, nh, d)
    nbatch = qf.shape[0]
    out = np.zeros((nbatch, nh, d), dtype=np.float64)
    head_list = range(nh) if heads is None else heads
    for b in range(nbatch):
        length = int(seq_lens[b])
        if length == 0:
            continue
        idx = gather_indices(block_tables[b], length, bs)
        keys = to_f64(kflat[idx], dtype)
        vals = to_f64(vflat[idx], dtype)
        for h in head_list:
            out[b, h] = attend_one(qf[b, h], keys[:, h, :], vals[:, h, :], scale)
    return out


def decode_attention_pairs(q, k_pool, v_pool, block_tables, seq_lens, dtype: str, pairs,
                           scale: float | None = None) -> dict:
    """Oracle outputs for selected ``(b, h)`` pairs only (large-case sampling)."""
    nb, bs, nh, d = k_pool.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    kflat = k_pool.reshape(nb * bs, nh, d)
    vflat = v_pool.reshape(nb * bs, nh, d)
    res = {}
    for b, h in pairs:
        length = int(seq_lens[b])
        idx = gather_indices(block_tables[b], length, bs)
        keys = to_f64(kflat[idx, h, :], dtype)
        vals = to_f64(vflat[idx, h, :], dtype)
        res[(b, h)] = attend_one(to_f64(q[b, h], dtype), keys, vals, scale)
    return res


def contiguous_attention(q, keys, values, dtype: str, scale: float | None = None) -> np.ndarray:
    """Attention over an unpaged per-sequence cache ``keys[b]: [L_b][H][D]``.

    The replaced baseline keeps each request's K/V contiguous
    (m.lqnn.cn/news/240480 §2.1); paging must reproduce it exactly.
    """
    nh, d = q.shape[1], q.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qf = to_f64(q, dtype)
    out = np.zeros(qf.shape, dtype=np.float64)
    for b in range(qf.shape[0]):
        kb = to_f64(keys[b], dtype)
        vb = to_f64(values[b], dtype)
        for h in range(nh):
            out[b, h] = attend_one(qf[b, h], kb[:, h, :], vb[:, h, :], scale)
    return out
