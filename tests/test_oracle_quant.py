"""Pins of the 8-bit K/V oracle (oracle.quant).

Checked against things other than itself: torch's float8_e4m3fn type (a
library decoding and rounding of the same OCP format), rows whose scale is
exactly 1 so every code follows by hand from the rounding rule, invariants of
symmetric absmax quantisation (largest element -> largest code, error within
half a step, zero rows), and the reduction of quantised attention to the
already pinned dense oracle on the dequantised values.  Planted mistakes in
copies of the oracle must each fail at least one pin.
"""

import math
import types

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oat
from oracle import pool as opool
from oracle import quant as oq


def _torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_e4m3_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _sweep():
    """Every E4M3 value, every midpoint between neighbours, one float32 step either side, random values."""
    vals = oq.E4M3_TABLE[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    down = np.nextafter(pts, np.float32(-np.inf))
    rng = np.random.default_rng(3)
    rnd = (rng.standard_normal(4000) * np.exp(rng.uniform(-12, 6, 4000))).astype(np.float32)
    allp = np.concatenate([pts, up, down, rnd, [0.0, 2.0 ** -10, 3 * 2.0 ** -11]]).astype(np.float32)
    allp = np.clip(allp, -448, 448).astype(np.float32)
    return np.concatenate([allp, -allp, np.array([-0.0], dtype=np.float32)])


# Rows with amax equal to QMAX, so scale = 1 exactly and r = x: every code is
# read off the rounding rule by hand.
I8_ROW = np.array([127.0, 63.5, -0.5, 1.5, 2.5, -2.5, 0.25, -127.0], dtype=np.float32)
I8_CODES = [127, 64, 0, 2, 2, -2, 0, -127]          # nearest integer, ties to even
FP8_ROW = np.array([448.0, 1.0625, 1.1875, -0.001, 240.0, 2.0 ** -10, -448.0, 3.0], dtype=np.float32)
# 448 = 1.75 x 2^8 -> 0x7E; 1.0625 is halfway 1.0 (0x38) / 1.125 (0x39) -> even 0x38;
# 1.1875 halfway 1.125 (0x39) / 1.25 (0x3A) -> 0x3A; -0.001 nearest -2^-9 -> 0x81;
# 240 = 1.875 x 2^7 -> 0x77; 2^-10 halfway 0 / 2^-9 -> even 0x00; -448 -> 0xFE;
# 3 = 1.5 x 2^1 -> 0x44.
FP8_CODES = [0x7E, 0x38, 0x3A, 0x81, 0x77, 0x00, 0xFE, 0x44]


def _dense_pool_from_codes(codes, scales, fmt, table_values):
    """K/V values a quantised pool holds, element by element (independent loops)."""
    nb, bs, h, d = codes.shape
    out = np.zeros((nb, bs, h, d), dtype=np.float64)
    for blk in range(nb):
        for p in range(bs):
            for hh in range(h):
                s = float(scales[blk, hh, p])
                for e in range(d):
                    c = int(codes[blk, p, hh, e])
                    v = (c - 256 if c > 127 else c) if fmt == "i8" else table_values[c]
                    out[blk, p, hh, e] = v * s   # exact in float64: an 8-bit code times a float32
    return out


def run_quant_pins(impl):
    """Apply every pin to ``impl`` (an object with the oracle.quant functions); return failures."""
    failures = []
    tv = _torch_e4m3_values()
    # (1) the code table equals torch's decoding of the same format
    t = impl.E4M3_TABLE
    same = np.array_equal(np.isnan(t), np.isnan(tv)) and np.array_equal(t[~np.isnan(t)], tv[~np.isnan(tv)])
    if not (same and t[0x7E] == 448.0 and t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x38] == 1.0):
        failures.append("e4m3-table")
    # (2) rounding to E4M3 equals torch's cast on values, midpoints and their neighbours
    x = _sweep()
    try:
        if not np.array_equal(impl.e4m3_encode(x), _torch_e4m3_encode(x)):
            failures.append("e4m3-encode")
    except Exception:
        failures.append("e4m3-encode raised")
    # (3) hand-derived rows with scale exactly 1
    try:
        c, s = impl.quantize_rows(I8_ROW[None, :], "f32", "i8")
        if not (s[0] == 1.0 and c[0].view(np.int8).tolist() == I8_CODES):
            failures.append("i8-row")
        c, s = impl.quantize_rows(FP8_ROW[None, :], "f32", "fp8")
        if not (s[0] == 1.0 and c[0].tolist() == FP8_CODES):
            failures.append("fp8-row")
    except Exception:
        failures.append("rows raised")
    # (4) invariants on random rows of every input dtype
    rng = np.random.default_rng(5)
    for dt in ("f32", "f16", "bf16"):
        raw = (rng.standard_normal((64, 3, 32)) * np.exp(rng.uniform(-4, 4, (64, 3, 1)))).astype(np.float32)
        raw[0, 1] = 0.0                                           # a zero row
        xs = workloads.to_storage(raw, dt)
        xf = oat.to_f64(xs, dt)
        for fmt in ("i8", "fp8"):
            try:
                c, s = impl.quantize_rows(xs, dt, fmt)
            except Exception:
                failures.append(f"{fmt}-{dt} raised")
                continue
            amax = np.max(np.abs(xf), axis=-1)
            if not np.array_equal(s, (amax.astype(np.float32) / np.float32(oq.QMAX[fmt])).astype(np.float32)):
                failures.append(f"{fmt}-{dt}-scale")
            if not (s[0, 1] == 0 and np.all(c[0, 1] == 0)):
                failures.append(f"{fmt}-{dt}-zero-row")
            vals = impl.code_values(c, fmt)
            top = np.argmax(np.abs(xf), axis=-1)
            picked = np.take_along_axis(vals, top[..., None], axis=-1)[..., 0]
            nz = s > 0
            if not np.all(np.abs(picked[nz]) == oq.QMAX[fmt]):
                failures.append(f"{fmt}-{dt}-amax-code")
            deq = vals * s.astype(np.float64)[..., None]
            err = np.abs(deq - xf)
            # half a code step, plus the float32 rounding of x / scale (|r| <= QMAX)
            sd = s.astype(np.float64)[..., None]
            if fmt == "i8":
                bound = sd * (0.5 + 128 * 2.0 ** -24)
            else:
                bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * sd) + np.abs(xf) * 2.0 ** -23
            if not np.all(err <= bound):
                failures.append(f"{fmt}-{dt}-error-bound")
    # (5) quantised attention = dense attention over the dequantised pool
    h, d, bs = 3, 16, 4
    lens = [1, 6, 13]
    nblk = [-(-L // bs) for L in lens]
    nb = sum(nblk) + 2
    perm = rng.permutation(nb)
    tables = np.zeros((len(lens), max(nblk)), dtype=np.int32)
    k = 0
    for b in range(len(lens)):
        for j in range(nblk[b]):
            tables[b, j] = perm[k]
            k += 1
    q = workloads.to_storage(rng.standard_normal((len(lens), h, d), dtype=np.float32), "f16")
    for fmt in ("i8", "fp8"):
        kc = rng.integers(0, 256, (nb, bs, h, d)).astype(np.uint8)
        vc = rng.integers(0, 256, (nb, bs, h, d)).astype(np.uint8)
        if fmt == "fp8":
            kc[(kc & 0x7F) == 0x7F] = 0x10   # no NaN codes
            vc[(vc & 0x7F) == 0x7F] = 0x22
        ks = rng.uniform(0.001, 0.02, (nb, h, bs)).astype(np.float32)
        vs = rng.uniform(0.001, 0.02, (nb, h, bs)).astype(np.float32)
        kd = _dense_pool_from_codes(kc, ks, fmt, tv)
        vd = _dense_pool_from_codes(vc, vs, fmt, tv)
        want = oat.decode_attention(oat.to_f64(q, "f16").astype(np.float32), kd, vd, tables, lens, "f32", 0.3)
        try:
            got = impl.decode_attention(q, kc, vc, ks, vs, tables, lens, "f16", fmt, 0.3)
            if not np.allclose(got, want, rtol=0, atol=1e-12):
                failures.append(f"{fmt}-attention")
        except Exception:
            failures.append(f"{fmt}-attention raised")
    return failures


def test_quant_oracle_passes_all_pins():
    assert run_quant_pins(oq) == []


def _impl(**over):
    ns = types.SimpleNamespace(E4M3_TABLE=oq.E4M3_TABLE, e4m3_encode=oq.e4m3_encode, quantize_rows=oq.quantize_rows,
                               code_values=oq.code_values, decode_attention=oq.decode_attention)
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def _quantize_variant(kind):
    def qr(x, dtype, fmt):
        x32 = oat.to_f64(x, dtype).astype(np.float32)
        amax = np.max(np.abs(x32), axis=-1)
        qmax = np.float32(128.0 if kind == "qmax-128" else oq.QMAX[fmt])
        if kind == "eps-floor":
            amax = np.maximum(amax, np.float32(1e-6))
        scale = (amax / qmax).astype(np.float32)
        safe = np.where(scale > 0, scale, np.float32(1))
        with np.errstate(invalid="ignore", divide="ignore"):
            r = (x32 / safe[..., None]).astype(np.float32)
        if fmt == "i8":
            if kind == "half-away":
                rr = np.sign(r) * np.floor(np.abs(r) + 0.5)
            else:
                rr = np.rint(r)
            codes = np.clip(np.nan_to_num(rr), -127, 127).astype(np.int8).view(np.uint8)
        else:
            codes = oq.e4m3_encode(np.clip(np.nan_to_num(r), -448, 448).astype(np.float32))
        codes = np.where(scale[..., None] > 0, codes, np.uint8(0)).astype(np.uint8)
        return codes, scale
    return qr


def _fnuz_table():
    t = np.array([oq.e4m3_value(c) for c in range(256)]) / 2.0   # bias 8 instead of 7
    return t


def _encode_ties_up(r):
    r = np.asarray(r, dtype=np.float32)
    a = np.abs(r).astype(np.float64)
    pos = oq.E4M3_TABLE[:0x7F]
    hi = np.minimum(np.searchsorted(pos, a, side="left"), len(pos) - 1)
    lo = np.maximum(hi - 1, 0)
    pick = np.where(a - pos[lo] < pos[hi] - a, lo, hi)
    return pick.astype(np.uint8) | (np.signbit(r).astype(np.uint8) << 7)


def _attention_variant(kind):
    def attn(q, kp, vp, ks, vs, tables, lens, q_dtype, fmt, scale=None, heads=None):
        nb, bs, nh, d = kp.shape
        qf = oat.to_f64(q, q_dtype)
        out = np.zeros((qf.shape[0], nh, d))
        kf, vf = kp.reshape(-1, nh, d), vp.reshape(-1, nh, d)
        for b in range(qf.shape[0]):
            idx = oat.gather_indices(tables[b], int(lens[b]), bs)
            blk, pos = idx // bs, idx % bs
            for h in range(nh):
                hs = (h + 1) % nh if kind == "scale-head-mixup" else h
                ksc = (vs if kind == "v-scale-for-k" else ks)[blk, hs, pos]
                keys = oq.code_values(kf[idx, h], fmt) * ksc[:, None]
                vals = oq.code_values(vf[idx, h], fmt) * vs[blk, hs, pos][:, None]
                if kind == "scale-position-reversed":
                    keys = oq.code_values(kf[idx, h], fmt) * ks[blk, h, bs - 1 - pos][:, None]
                out[b, h] = oat.attend_one(qf[b, h], keys, vals, scale)
        return out
    return attn


MUTANTS = {
    "half-away": lambda: _impl(quantize_rows=_quantize_variant("half-away")),
    "qmax-128": lambda: _impl(quantize_rows=_quantize_variant("qmax-128")),
    "eps-floor": lambda: _impl(quantize_rows=_quantize_variant("eps-floor")),
    "fnuz-bias": lambda: _impl(E4M3_TABLE=_fnuz_table()),
    "ties-up": lambda: _impl(e4m3_encode=_encode_ties_up),
    "v-scale-for-k": lambda: _impl(decode_attention=_attention_variant("v-scale-for-k")),
    "scale-head-mixup": lambda: _impl(decode_attention=_attention_variant("scale-head-mixup")),
    "scale-position-reversed": lambda: _impl(decode_attention=_attention_variant("scale-position-reversed")),
}


@pytest.mark.parametrize("kind", sorted(MUTANTS))
def test_quant_pins_catch_planted_mistakes(kind):
    with np.errstate(all="ignore"):
        assert run_quant_pins(MUTANTS[kind]()), f"mutant {kind} passed every pin"


def test_append_writes_codes_and_scales_at_slots():
    # Scatter of quantised rows: codes at [block][pos][h][:], scale at [block][h][pos];
    # slots < 0 skipped; other slots untouched.
    rng = np.random.default_rng(9)
    nb, bs, h, d = 5, 4, 2, 8
    kp = np.full((nb, bs, h, d), 0xAB, dtype=np.uint8)
    vp = kp.copy()
    ks = np.full((nb, h, bs), np.nan, dtype=np.float32)
    vs = ks.copy()
    kn = workloads.to_storage(rng.standard_normal((4, h, d), dtype=np.float32), "bf16")
    vn = workloads.to_storage(rng.standard_normal((4, h, d), dtype=np.float32), "bf16")
    slots = [7, -1, 0, 19]
    oq.append(kp, vp, ks, vs, kn, vn, slots, "bf16", "fp8")
    kc, kscale = oq.quantize_rows(kn, "bf16", "fp8")
    vc, vscale = oq.quantize_rows(vn, "bf16", "fp8")
    for t, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(kp[s // bs, s % bs], kc[t]) and np.array_equal(vp[s // bs, s % bs], vc[t])
        assert np.array_equal(ks[s // bs, :, s % bs], kscale[t]) and np.array_equal(vs[s // bs, :, s % bs], vscale[t])
    written = {(s // bs, s % bs) for s in slots if s >= 0}
    for blk in range(nb):
        for p in range(bs):
            if (blk, p) not in written:
                assert np.all(kp[blk, p] == 0xAB) and np.all(np.isnan(ks[blk, :, p]))
    # The dense pool oracle scatters the same bytes when given the codes.
    kp2 = np.full_like(kp, 0xAB)
    vp2 = np.full_like(vp, 0xAB)
    opool.append(kp2, vp2, kc, vc, slots)
    assert np.array_equal(kp2, kp) and np.array_equal(vp2, vp)


def test_quantised_attention_tracks_unquantised():
    # Sanity of the format choice: on N(0,1) rows the 8-bit cache changes the
    # attention output by far less than the output's own spread.
    rng = np.random.default_rng(21)
    L, h, d = 200, 2, 64
    k = rng.standard_normal((L, h, d)).astype(np.float32)
    v = rng.standard_normal((L, h, d)).astype(np.float32)
    q = rng.standard_normal((1, h, d)).astype(np.float32)
    ref = oat.contiguous_attention(q, [k], [v], "f32")
    for fmt, tol in (("i8", 0.01), ("fp8", 0.03)):
        kc, ks = oq.quantize_rows(k, "f32", fmt)
        vc, vs = oq.quantize_rows(v, "f32", fmt)
        kd = oq.dequantize(kc, ks, fmt).astype(np.float32)
        vd = oq.dequantize(vc, vs, fmt).astype(np.float32)
        got = oat.contiguous_attention(q, [kd], [vd], "f32")
        assert np.max(np.abs(got - ref)) < tol, (fmt, np.max(np.abs(got - ref)))
    assert math.isclose(oq.e4m3_value(0x7E), 448.0)
