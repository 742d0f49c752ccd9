"""8-bit K/V cache: quantisation on write, exact dequantisation on read (oracle).

Test infrastructure only.  Storing K/V in 8 bits instead of 16 halves the
bytes per token (hnwysp.cn/news/103996 §5.4; m.lqnn.cn/news/240480 §6.2 gives
8,192 bytes per token for the 7B shape), and it stacks with paging without
changing it (icman.com.cn/news/78786 §1.3): block tables, slots and block
copies are the same; only what a slot holds changes.

The pages fix no scale granularity, rounding or 8-bit format.  Readings taken
here (each listed in the design notes):

* Formats: ``"i8"`` = signed 8-bit integers, symmetric, codes in
  [-127, 127]; ``"fp8"`` = OCP FP8 E4M3 ("e4m3fn": bias 7, subnormals, no
  infinities, 0x7F/0xFF NaN, largest finite 448), the 8-bit float format
  MI355X converts natively.
* One scale per (token, head) row of ``head_dim`` values: a row is quantised
  once, when its token is written, and never again (a per-block scale would
  have to be fixed before the block's later tokens exist).
* The scale maps the row's largest magnitude onto the format's largest code:
  ``scale = amax / QMAX`` (QMAX = 127 or 448); a row of zeros gets scale 0 and
  zero codes.
* Codes: ``r = x / scale``; int8 rounds ``r`` to the nearest integer, ties to
  even, then clamps to [-127, 127]; fp8 clamps ``r`` to [-448, 448] and rounds
  to the nearest E4M3 value, ties to the even code.
* These steps decide integers, so they are carried out in float32 exactly as
  written (IEEE float32 ``max``, division and rounding), the precision the
  kernel works in; the input is its stored value widened to float32, which is
  exact for fp16, bf16 and fp32.
* Reading a row gives ``code_value * scale`` exactly (float64 holds the
  product of an 8-bit code and a float32 scale without rounding); attention
  then runs on those values by its plain definition.

Storage: code pools ``[num_blocks][block_size][H][D]`` (uint8 bytes), scale
pools ``[num_blocks][H][block_size]`` float32, one each for K and V.
"""

from __future__ import annotations

import numpy as np

from .attention import attend_one, gather_indices, to_f64

QMAX = {"i8": 127.0, "fp8": 448.0}


def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 code from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)       # subnormal: 0.m x 2^(1 - bias)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)      # normal: 1.m x 2^(e - bias)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
_POS = E4M3_TABLE[:0x7F]   # codes 0x00..0x7E: the non-negative finite values, ascending


def e4m3_encode(r: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each finite value in [-448, 448]; a tie goes to the even code.

    The sign bit is the sign bit of ``r`` (so -0.0 and values that round to
    zero from below give 0x80).
    """
    r = np.asarray(r, dtype=np.float32)
    if np.any(~np.isfinite(r)) or np.any(np.abs(r) > 448.0):
        raise ValueError("e4m3_encode takes finite values within [-448, 448]")
    a = np.abs(r).astype(np.float64).ravel()
    hi = np.searchsorted(_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick = np.where(dlo < dhi, lo, hi)
    tie = dlo == dhi
    pick = np.where(tie & (lo != hi), np.where(lo % 2 == 0, lo, hi), pick)
    codes = pick.astype(np.uint8).reshape(r.shape)
    return codes | (np.signbit(r).astype(np.uint8) << 7)


def code_values(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Float64 value of each stored code byte."""
    codes = np.asarray(codes, dtype=np.uint8)
    if fmt == "i8":
        return codes.view(np.int8).astype(np.float64)
    if fmt == "fp8":
        return E4M3_TABLE[codes]
    raise ValueError(f"unknown 8-bit format {fmt}")


def quantize_rows(x: np.ndarray, dtype: str, fmt: str):
    """Quantise rows along the last axis; returns ``(codes uint8, scales float32)``.

    ``x``: stored values (bf16 as uint16 bits) of shape ``[..., D]``; codes
    have the same shape, scales drop the last axis.
    """
    x32 = to_f64(x, dtype).astype(np.float32)            # exact: stored values widen to float32
    amax = np.max(np.abs(x32), axis=-1)
    scale = (amax / np.float32(QMAX[fmt])).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    r = (x32 / safe[..., None]).astype(np.float32)
    if fmt == "i8":
        q = np.clip(np.rint(r), -127, 127).astype(np.int8)
        codes = q.view(np.uint8)
    elif fmt == "fp8":
        codes = e4m3_encode(np.clip(r, np.float32(-448.0), np.float32(448.0)))
    else:
        raise ValueError(f"unknown 8-bit format {fmt}")
    codes = np.where(scale[..., None] > 0, codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    """``code_value * scale`` for every element, float64 (exact)."""
    return code_values(codes, fmt) * np.asarray(scales, dtype=np.float64)[..., None]


def append(k_pool, v_pool, k_scales, v_scales, k_new, v_new, slots, dtype: str, fmt: str) -> None:
    """Quantise token t's K/V rows and store codes and scales at flat slot ``slots[t]``.

    Negative slots are skipped.  Code pools are ``[NB][bs][H][D]`` uint8; scale
    pools ``[NB][H][bs]`` float32.
    """
    nb, bs, h, d = k_pool.shape
    kf = k_pool.reshape(nb * bs, h, d)
    vf = v_pool.reshape(nb * bs, h, d)
    kc, ks = quantize_rows(k_new, dtype, fmt)
    vc, vs = quantize_rows(v_new, dtype, fmt)
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        if s >= nb * bs:
            raise IndexError(f"slot {s} outside a pool of {nb * bs} slots")
        kf[s] = kc[t]
        vf[s] = vc[t]
        k_scales[s // bs, :, s % bs] = ks[t]
        v_scales[s // bs, :, s % bs] = vs[t]


def decode_attention(q, k_pool, v_pool, k_scales, v_scales, block_tables, seq_lens, q_dtype: str, fmt: str,
                     scale: float | None = None, heads=None) -> np.ndarray:
    """Decode attention over a quantised paged cache; float64 ``[B][H][D]``.

    Each attended row is read back as ``code_value * scale`` and attention is
    the same plain softmax average as for an unquantised cache.
    """
    nb, bs, nh, d = k_pool.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qf = to_f64(q, q_dtype)
    kflat = k_pool.reshape(nb * bs, nh, d)
    vflat = v_pool.reshape(nb * bs, nh, d)
    out = np.zeros((qf.shape[0], nh, d), dtype=np.float64)
    head_list = range(nh) if heads is None else heads
    for b in range(qf.shape[0]):
        length = int(seq_lens[b])
        if length == 0:
            continue
        idx = gather_indices(block_tables[b], length, bs)
        blk, pos = idx // bs, idx % bs
        for h in head_list:
            keys = code_values(kflat[idx, h, :], fmt) * k_scales[blk, h, pos].astype(np.float64)[:, None]
            vals = code_values(vflat[idx, h, :], fmt) * v_scales[blk, h, pos].astype(np.float64)[:, None]
            out[b, h] = attend_one(qf[b, h], keys, vals, scale)
    return out
