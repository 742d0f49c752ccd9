"""K/V block pool updates (oracle; test infrastructure only).

Layout: one pool for K and one for V per layer, each ``[num_blocks][block_size]
[num_heads][head_dim]``.  This is the ``[page, slot, head, dim]`` order of the
index redirection in m.lqnn.cn/news/240480 §3.3 (the page's pseudo-code
strides disagree with its own stated order; the stated order is taken).

Both operations are pure byte moves, so the oracle works on the raw storage
arrays (float32, float16, or the uint16 bit patterns of bfloat16) and the
GPU result must match bit for bit.
"""

from __future__ import annotations

import numpy as np


def append(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, slots) -> None:
    """Write token t's K/V rows to flat slot ``slots[t]``; a negative slot is skipped.

    The new token's K and V are stored at its (block, offset) position before
    attention reads them (hnwysp.cn/news/103996 §1.1, §4.2;
    m.lqnn.cn/news/240480 §3.2 step 3).
    """
    nb, bs, h, d = k_pool.shape
    kf = k_pool.reshape(nb * bs, h, d)
    vf = v_pool.reshape(nb * bs, h, d)
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        if s >= nb * bs:
            raise IndexError(f"slot {s} outside a pool of {nb * bs} slots")
        kf[s] = k_new[t]
        vf[s] = v_new[t]


def copy_blocks(k_pools, v_pools, pairs) -> None:
    """Copy whole blocks ``src -> dst`` in every given layer, K and V alike.

    Copy-on-write duplicates the entire shared block before the branching
    sequence writes into it (hnwysp.cn/news/103996 §3.3).  The pairs act as one
    simultaneous copy, so destinations must be distinct and never a source.
    """
    srcs = [int(s) for s, _ in pairs]
    dsts = [int(d) for _, d in pairs]
    if len(set(dsts)) != len(dsts) or set(dsts) & set(srcs):
        raise ValueError("copy pairs overlap")
    for kp, vp in zip(k_pools, v_pools):
        for s, d in zip(srcs, dsts):
            kp[d] = kp[s]
            vp[d] = vp[s]


def swap_blocks(dst_pools, src_pools, pairs) -> None:
    """Copy block ``s`` of every source pool to block ``d`` of the matching destination pool.

    Preemption moves a request's blocks to host memory and back instead of
    recomputing them (icman.com.cn/news/78786 §4.2): a whole-block bit copy
    between two pools, like copy-on-write but across pools.  Destinations
    must be distinct.
    """
    dsts = [int(d) for _, d in pairs]
    if len(set(dsts)) != len(dsts):
        raise ValueError("swap destinations repeat")
    for dp, sp in zip(dst_pools, src_pools):
        for s, d in pairs:
            dp[int(d)] = sp[int(s)]
