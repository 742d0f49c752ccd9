"""Cumulative attention score per cached token (oracle; test infrastructure only).

A token's importance can be measured by how much attention the queries of
past steps paid to it: after each attention computation, every key position
adds the attention weight it received (zskr.cn/news/1363082.html §3.1,
"cumulative attention score"), and the running total decays exponentially
once per step so that recent attention counts more (same page, §4.1: decay
factor such as 0.995).  This is the input of windowed eviction; the eviction
and recomputation around it need a model and are not part of this path.

Readings where the page leaves the detail open (listed in the design notes):

* Per sequence and logical position t < L_b, one float:
  ``S[b][t] <- decay * S[b][t] + (1/H) * sum_h p_{b,h}(t)``, where
  ``p_{b,h}`` is this decode step's softmax distribution of head h over the
  L_b cached positions.  Heads are averaged (each distribution sums to one,
  so every step adds exactly one unit of mass over a sequence's positions).
* Positions at or beyond L_b are untouched; a row starts from zero when its
  sequence starts (the caller zeroes it).
* Probabilities are the same ones decode attention weights values with
  (oracle.attention / oracle.quant definitions), computed in float64.
"""

from __future__ import annotations

import numpy as np

from .attention import gather_indices, to_f64
from .quant import code_values


def softmax_probs(q_vec: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """The decode softmax over ``keys`` ([L][D]) for one query, float64."""
    if keys.shape[0] == 0:
        return np.zeros(0)
    s = scale * (keys @ q_vec)
    w = np.exp(s - s.max())
    return w / w.sum()


def attention_probs(q, k_pool, block_tables, seq_lens, dtype: str, scale=None, k_scales=None, fmt=None) -> list:
    """Per sequence, the ``[H][L_b]`` softmax probabilities of its decode step.

    ``k_pool`` in the layout of the cache; for an 8-bit cache pass its
    ``k_scales`` pool and ``fmt`` ("i8" / "fp8"), and keys are read back as
    code x scale exactly.
    """
    nb, bs, nh, d = k_pool.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qf = to_f64(q, dtype)
    kflat = k_pool.reshape(nb * bs, nh, d)
    out = []
    for b in range(qf.shape[0]):
        length = int(seq_lens[b])
        idx = gather_indices(block_tables[b], length, bs) if length > 0 else np.zeros(0, dtype=np.int64)
        probs = np.zeros((nh, length))
        for h in range(nh):
            if fmt is None:
                keys = to_f64(kflat[idx, h, :], dtype)
            else:
                keys = code_values(kflat[idx, h, :], fmt) * \
                    k_scales[idx // bs, h, idx % bs].astype(np.float64)[:, None]
            probs[h] = softmax_probs(qf[b, h], keys, scale)
        out.append(probs)
    return out


def cumulative_update(scores: np.ndarray, probs: list, decay: float) -> np.ndarray:
    """``scores`` ([B][stride], float64 copy returned): decay every position the
    step attended to and add the head-mean probability it received."""
    new = np.array(scores, dtype=np.float64, copy=True)
    for b, p in enumerate(probs):
        length = p.shape[1]
        if length == 0:
            continue
        new[b, :length] = decay * new[b, :length] + p.mean(axis=0)
    return new
