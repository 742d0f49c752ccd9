"""Seeded synthetic inputs for paged-KV decode attention.

This module only draws inputs: sequence lengths, which sequences share a
prefix, the initial order of the free list (which scatters blocks through the
pool), and the query/key/value values.  It holds none of the method's
arithmetic: no slot mapping, no allocation, no attention.  Both the HIP path
and the oracle take their inputs from here.

Recipes (one per workload; ``numpy.random.default_rng(seed)`` with the draw
order lengths -> sharer set -> free-list permutation -> Q -> K -> V; values
are float32 standard normal cast to the storage dtype with round-to-nearest-
even):

* ``tiny``: 1 layer, batch 4, 4 heads x 64, fp32, block 16, lengths
  {1, 17, 64, 100}, pool of 64 blocks, scale 1/sqrt(64).
* ``llama7b_layer``: one layer of a 7B-shaped model (32 heads x 128, fp16),
  block 16, batch 32, lengths uniform on the integers [128, 2048], pool =
  ceil(1.3 x blocks needed), blocks scattered by a random free order.  The
  shapes follow the 7B example of icman.com.cn/news/78786 §1.1 and the
  Llama-2-7B configuration of m.lqnn.cn/news/240480 §3.1; the 1.3 redundancy
  factor is hnwysp.cn/news/103996 §3.2.
* ``prefix_cow``: 32 x 128 fp16, block 16, batch 64 all sharing one 520-token
  prefix, unique suffix lengths geometric with mean 300 (support >= 1).
* ``long13b``: 13B-shaped (40 heads x 128), bf16, batch 16, length 4096 each,
  block 8, 16 or 32 (hnwysp.cn/news/103996 §1.2 gives the 13B shape).
* ``full7b_step``: 32 layers x 32 heads x 128, fp16, block 16, batch 256,
  lognormal lengths (median 300, sigma 1) clipped to [1, 4096], 30 % of
  sequences sharing a 256-token prefix; pool sized by the caller from free
  device memory (85 %, icman.com.cn/news/78786 §2.3).  Its K/V are drawn on the
  device from ``torch.Generator`` seeded ``5000 + layer``.

The pages measure whole serving stacks on public suites and private traffic;
none of that is available or needed here, and these synthetic inputs of the
same shapes stand in for it.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float32 values to their storage form with round-to-nearest-even.

    fp32 stays float32, fp16 becomes numpy float16, bf16 becomes the uint16 bit
    pattern (numpy has no bfloat16 type).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        bits = x.view(np.uint32)
        rounding = ((bits >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        return ((bits + rounding) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def nan_storage(dtype: str):
    """Quiet-NaN storage value used to poison never-written pool slots."""
    return {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}[dtype]


def storage_np_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


@dataclass
class Workload:
    key: str
    title: str
    num_layers: int
    batch: int
    num_heads: int
    head_dim: int
    dtype: str
    block_size: int
    seq_lens: np.ndarray           # int32 [B]: attended length incl. this step's token
    prefix_len: int                # tokens of the shared prefix (0 = none)
    sharers: np.ndarray            # indices of sequences that share the prefix
    num_blocks: int                # pool size in blocks
    free_order: np.ndarray         # int32 permutation of 0..num_blocks-1
    scale: float
    seed: int
    rng: np.random.Generator = field(repr=False, default=None)

    @property
    def dtype_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0

    def max_blocks_per_seq(self, extra_tokens: int = 0) -> int:
        return -(-(self.max_seq_len + extra_tokens) // self.block_size)

    def private_len(self, b: int) -> int:
        """Tokens of sequence b that are its own (not the shared prefix)."""
        shared = self.prefix_len if b in set(int(s) for s in self.sharers) else 0
        return int(self.seq_lens[b]) - shared

    def draw_values(self):
        """Draw Q and all K/V token rows (storage dtype), continuing this workload's stream.

        Returns a dict: ``q`` [B][H][D]; ``k_prefix``/``v_prefix`` [prefix][H][D];
        ``k_seq``/``v_seq``: lists of [private_len(b)][H][D] in sequence order.
        """
        rng = self.rng
        h, d, dt = self.num_heads, self.head_dim, self.dtype
        q = to_storage(rng.standard_normal((self.batch, h, d), dtype=np.float32), dt)
        counts = [self.private_len(b) for b in range(self.batch)]
        out = {"q": q}
        for name in ("k", "v"):
            pre = to_storage(rng.standard_normal((self.prefix_len, h, d), dtype=np.float32), dt)
            rows = []
            for c in counts:
                rows.append(to_storage(rng.standard_normal((c, h, d), dtype=np.float32), dt))
            out[name + "_prefix"] = pre
            out[name + "_seq"] = rows
        return out


def _finish(key, title, layers, lens, h, d, dtype, bs, prefix_len, sharers, rng, seed, num_blocks, scale=None):
    order = rng.permutation(num_blocks).astype(np.int32)
    return Workload(key=key, title=title, num_layers=layers, batch=len(lens), num_heads=h, head_dim=d,
                    dtype=dtype, block_size=bs, seq_lens=np.asarray(lens, dtype=np.int32),
                    prefix_len=prefix_len, sharers=np.asarray(sharers, dtype=np.int64), num_blocks=num_blocks,
                    free_order=order, scale=(1.0 / math.sqrt(d)) if scale is None else scale,
                    seed=seed, rng=rng)


def _pool_for(lens, bs, factor=1.3):
    # Pool sized to the redundancy factor times the blocks the lengths occupy.
    return int(math.ceil(factor * sum(-(-int(x) // bs) for x in lens)))


def tiny(seed: int = 1) -> Workload:
    rng = np.random.default_rng(seed)
    lens = [1, 17, 64, 100]
    return _finish("tiny", "Tiny: 1 layer, batch 4, 4 heads x 64, fp32, block 16, lengths {1,17,64,100}",
                   1, lens, 4, 64, "f32", 16, 0, [], rng, seed, 64, scale=1.0 / 8.0)


def llama7b_layer(seed: int = 2, batch: int = 32, lo: int = 128, hi: int = 2048) -> Workload:
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, size=batch, endpoint=True)
    return _finish("llama7b_layer",
                   f"7B-shaped single-layer decode: 32 heads x 128, fp16, block 16, batch {batch}, "
                   f"lengths U[{lo},{hi}]",
                   1, lens, 32, 128, "f16", 16, 0, [], rng, seed, _pool_for(lens, 16))


def prefix_cow(seed: int = 3, batch: int = 64, prefix: int = 520, mean_suffix: float = 300.0) -> Workload:
    rng = np.random.default_rng(seed)
    suffix = rng.geometric(1.0 / mean_suffix, size=batch)
    lens = prefix + suffix
    sharers = np.arange(batch)
    # Pool: the redundancy factor over the blocks an unshared layout would need.
    return _finish("prefix_cow",
                   f"Prefix sharing + copy-on-write: 32 heads x 128, fp16, block 16, batch {batch} sharing "
                   f"a {prefix}-token prefix, suffix ~ Geometric(mean {mean_suffix:g})",
                   1, lens, 32, 128, "f16", 16, prefix, sharers, rng, seed, _pool_for(lens, 16))


def long13b(block_size: int = 16, seed: int = 4, batch: int = 16, length: int = 4096) -> Workload:
    rng = np.random.default_rng(seed)
    lens = np.full(batch, length)
    return _finish(f"long13b_bs{block_size}",
                   f"13B-shaped long context: 40 heads x 128, bf16, batch {batch}, length {length}, "
                   f"block {block_size}",
                   1, lens, 40, 128, "bf16", block_size, 0, [], rng, seed, _pool_for(lens, block_size))


def full7b_step_lengths(seed: int = 5, batch: int = 256, median: float = 300.0, sigma: float = 1.0,
                        lo: int = 1, hi: int = 4096, prefix: int = 256, share_frac: float = 0.3):
    """Lengths and sharer set of the full 32-layer step (drawn before the pool size is known)."""
    rng = np.random.default_rng(seed)
    lens = np.clip(np.rint(np.exp(rng.normal(math.log(median), sigma, size=batch))), lo, hi).astype(np.int64)
    n_share = int(round(share_frac * batch))
    sharers = np.sort(rng.permutation(batch)[:n_share])
    lens[sharers] = np.maximum(lens[sharers], prefix + 1)
    return rng, lens, sharers


def full7b_step(num_blocks: int, seed: int = 5, batch: int = 256, layers: int = 32) -> Workload:
    rng, lens, sharers = full7b_step_lengths(seed=seed, batch=batch)
    return _finish("full7b_step",
                   f"Full 7B decode step: {layers} layers x 32 heads x 128, fp16, block 16, batch {batch}, "
                   f"lognormal lengths (median 300, sigma 1) in [1,4096], 30% share a 256-token prefix",
                   layers, lens, 32, 128, "f16", 16, 256, sharers, rng, seed, int(num_blocks))


def custom(seq_lens, num_heads=4, head_dim=64, dtype="f32", block_size=16, seed=0, pool_factor=1.3,
           num_blocks=None, prefix_len=0, sharers=(), num_layers=1) -> Workload:
    """Small parity cases: given lengths, random free order over a 1.3x pool."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(seq_lens, dtype=np.int64)
    nb = num_blocks if num_blocks is not None else max(1, _pool_for(lens, block_size, pool_factor))
    return _finish("custom", f"custom lengths {list(lens)[:8]}...", num_layers, lens, num_heads, head_dim, dtype,
                   block_size, prefix_len, list(sharers), rng, seed, nb)


CONFIGS = {
    1: tiny,
    2: llama7b_layer,
    3: prefix_cow,
    4: long13b,
}
