"""Pins of the attention oracle and the pool oracle.

The attention oracle is checked against things other than itself: a library
routine (torch's scaled_dot_product_attention in float64 on the CPU), closed
forms (one token, equal keys, zero query, two tokens), invariants the pages
imply (physical placement and prefix sharing change nothing), brute force on
the tiny workload, and a set of planted mistakes that the pins must catch.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oat
from oracle import pool as opool


def _paged_case(rng, lens, h, d, bs, dtype="f32", pool_extra=3, poison=True):
    """Contiguous per-sequence K/V plus the same rows scattered into a pool."""
    nblk = [-(-L // bs) for L in lens]
    nb = sum(nblk) + pool_extra
    perm = rng.permutation(nb)
    sd = workloads.storage_np_dtype(dtype)
    kp = np.zeros((nb, bs, h, d), dtype=sd)
    vp = np.zeros((nb, bs, h, d), dtype=sd)
    if poison:
        kp[:] = workloads.nan_storage(dtype)
        vp[:] = workloads.nan_storage(dtype)
    keys, vals, tables = [], [], np.zeros((len(lens), max(nblk + [1])), dtype=np.int32)
    k = 0
    for b, L in enumerate(lens):
        kb = workloads.to_storage(rng.standard_normal((L, h, d), dtype=np.float32), dtype)
        vb = workloads.to_storage(rng.standard_normal((L, h, d), dtype=np.float32), dtype)
        keys.append(kb)
        vals.append(vb)
        for j in range(nblk[b]):
            tables[b, j] = perm[k]
            k += 1
        slots = [int(tables[b, t // bs]) * bs + t % bs for t in range(L)]
        opool.append(kp, vp, kb, vb, slots)
    q = workloads.to_storage(rng.standard_normal((len(lens), h, d), dtype=np.float32), dtype)
    return q, kp, vp, tables, np.asarray(lens, dtype=np.int32), keys, vals


def _sdpa(q, keys, vals, dtype, scale):
    out = []
    for b in range(q.shape[0]):
        qt = torch.from_numpy(oat.to_f64(q[b], dtype)).unsqueeze(1)            # [H,1,D]
        kt = torch.from_numpy(oat.to_f64(keys[b], dtype)).permute(1, 0, 2).contiguous()
        vt = torch.from_numpy(oat.to_f64(vals[b], dtype)).permute(1, 0, 2).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        out.append(o[:, 0, :].numpy())
    return np.stack(out)


def run_pins(attn):
    """Apply every pin to ``attn`` (same signature as oat.decode_attention); return failures."""
    failures = []
    rng = np.random.default_rng(7)
    h, d, bs = 3, 16, 4
    # (1) library routine on random paged inputs
    lens = [1, 5, 13, 33]
    q, kp, vp, tab, L, keys, vals = _paged_case(rng, lens, h, d, bs)
    scale = 1 / math.sqrt(d)
    got = attn(q, kp, vp, tab, L, "f32", scale)
    ref = _sdpa(q, keys, vals, "f32", scale)
    if not (np.all(np.isfinite(got)) and np.max(np.abs(got - ref)) < 1e-12):
        failures.append("sdpa")
    # (2) one token: the output is that token's value row
    q1, kp1, vp1, tab1, L1, k1, v1 = _paged_case(rng, [1, 1], h, d, bs)
    got = attn(q1, kp1, vp1, tab1, L1, "f32", scale)
    if not np.array_equal(got, np.stack([v1[0][0], v1[1][0]]).astype(np.float64)):
        failures.append("one-token")
    # (3) equal keys and (4) zero query: the plain mean of the values
    q3, kp3, vp3, tab3, L3, k3, v3 = _paged_case(rng, [9], h, d, bs)
    flat = kp3.reshape(-1, h, d)
    for t in range(9):
        flat[int(tab3[0, t // bs]) * bs + t % bs] = k3[0][0]
    got = attn(q3, kp3, vp3, tab3, L3, "f32", scale)
    if not np.allclose(got[0], v3[0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-13):
        failures.append("equal-keys")
    qz = np.zeros_like(q)
    got = attn(qz, kp, vp, tab, L, "f32", scale)
    want = np.stack([vals[b].astype(np.float64).mean(axis=0) for b in range(len(lens))])
    if not np.allclose(got, want, rtol=0, atol=1e-13):
        failures.append("zero-query")
    # (5) two tokens: v0 + sigmoid(scale*(s1 - s0)) * (v1 - v0)
    q5, kp5, vp5, tab5, L5, k5, v5 = _paged_case(rng, [2], h, d, bs)
    got = attn(q5, kp5, vp5, tab5, L5, "f32", scale)
    for hh in range(h):
        qq = q5[0, hh].astype(np.float64)
        s0, s1 = scale * qq @ k5[0][0, hh], scale * qq @ k5[0][1, hh]
        sig = 1.0 / (1.0 + math.exp(-(s1 - s0)))
        want = v5[0][0, hh] + sig * (v5[0][1, hh].astype(np.float64) - v5[0][0, hh])
        if not np.allclose(got[0, hh], want, rtol=0, atol=1e-13):
            failures.append("two-token")
            break
    # (6) huge scores stay finite and pick the dominant token
    q6 = np.zeros((1, h, d), dtype=np.float32)
    q6[0, :, 0] = 1000.0
    kp6 = np.zeros((2, bs, h, d), dtype=np.float32)
    vp6 = rng.standard_normal((2, bs, h, d)).astype(np.float32)
    kp6[1, 2, :, 0] = 1.0   # logical token 6 (block 1 of the table) dominates
    tab6 = np.array([[0, 1]], dtype=np.int32)
    got = attn(q6, kp6, vp6, tab6, np.array([7], dtype=np.int32), "f32", 1.0)
    if not (np.all(np.isfinite(got)) and np.allclose(got[0], vp6[1, 2], rtol=0, atol=1e-12)):
        failures.append("stable-softmax")
    return failures


def test_oracle_passes_all_pins():
    assert run_pins(oat.decode_attention) == []


# Plausible mistakes, planted in copies of the oracle (never in the product).
def _mutant(kind):
    def attn(q, kp, vp, tables, lens, dtype, scale=None):
        nb, bs, nh, d = kp.shape
        scale = 1 / math.sqrt(d) if scale is None else scale
        out = np.zeros((q.shape[0], nh, d))
        kf, vf = kp.reshape(-1, nh, d), vp.reshape(-1, nh, d)
        for b in range(q.shape[0]):
            n = int(lens[b]) - (1 if kind == "off-by-one" and lens[b] > 1 else 0)
            t = np.arange(n)
            if kind == "swapped-index":
                row = np.asarray(tables[b])
                idx = row[np.minimum(t % bs, len(row) - 1)] * bs + np.minimum(t // bs, bs - 1)
            else:
                idx = np.asarray(tables[b])[t // bs] * bs + t % bs
            for h in range(nh):
                keys = oat.to_f64(kf[idx, h], dtype)
                vals = oat.to_f64((kf if kind == "k-for-v" else vf)[idx, h], dtype)
                qv = oat.to_f64(q[b, h], dtype)
                s = (1.0 if kind == "no-scale" else scale) * (keys @ qv)
                if kind == "sign":
                    s = -s
                w = np.exp(s - s.max())
                if kind == "no-normalise":
                    out[b, h] = w @ vals
                elif kind == "head-mixup":
                    out[b, h] = (w @ oat.to_f64(vf[idx, (h + 1) % nh], dtype)) / w.sum()
                else:
                    out[b, h] = (w @ vals) / w.sum()
        return out
    return attn


@pytest.mark.parametrize("kind", ["no-scale", "sign", "swapped-index", "k-for-v", "off-by-one",
                                  "no-normalise", "head-mixup"])
def test_pins_catch_planted_mistakes(kind):
    assert run_pins(_mutant(kind)), f"mutant {kind} passed every pin"


def test_paged_equals_contiguous_under_permutation():
    rng = np.random.default_rng(11)
    lens = [3, 16, 17, 40, 64]
    for dtype in ("f32", "f16", "bf16"):
        q, kp, vp, tab, L, keys, vals = _paged_case(rng, lens, 2, 8, 8, dtype)
        base = oat.decode_attention(q, kp, vp, tab, L, dtype)
        assert np.all(np.isfinite(base))  # the NaN-poisoned free slots were never read
        assert np.array_equal(base, oat.contiguous_attention(q, keys, vals, dtype))
        # Move every block to a new physical place: the output is bit-identical.
        nb = kp.shape[0]
        perm = rng.permutation(nb)
        kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
        kp2[perm] = kp
        vp2[perm] = vp
        tab2 = perm[tab].astype(np.int32)
        assert np.array_equal(base, oat.decode_attention(q, kp2, vp2, tab2, L, dtype))


def test_sharing_changes_nothing():
    # Two sequences reading one physical prefix block == each with a private copy.
    rng = np.random.default_rng(5)
    h, d, bs = 2, 8, 4
    kp = rng.standard_normal((6, bs, h, d)).astype(np.float32)
    vp = rng.standard_normal((6, bs, h, d)).astype(np.float32)
    q = rng.standard_normal((2, h, d)).astype(np.float32)
    shared = np.array([[0, 1], [0, 2]], dtype=np.int32)
    kp[3], vp[3] = kp[0], vp[0]
    private = np.array([[0, 1], [3, 2]], dtype=np.int32)
    L = np.array([7, 6], dtype=np.int32)
    assert np.array_equal(oat.decode_attention(q, kp, vp, shared, L, "f32"),
                          oat.decode_attention(q, kp, vp, private, L, "f32"))


def test_brute_force_tiny():
    wl = workloads.tiny()
    vals = wl.draw_values()
    bs, h, d = wl.block_size, wl.num_heads, wl.head_dim
    # Sequential layout: sequence b's blocks follow the free order.
    order = list(wl.free_order)
    tables = np.zeros((wl.batch, 8), dtype=np.int32)
    kp = np.full((wl.num_blocks, bs, h, d), np.nan, dtype=np.float32)
    vp = np.full_like(kp, np.nan)
    for b in range(wl.batch):
        L = int(wl.seq_lens[b])
        for j in range(-(-L // bs)):
            tables[b, j] = order.pop(0)
        for t in range(L):
            kp[tables[b, t // bs], t % bs] = vals["k_seq"][b][t]
            vp[tables[b, t // bs], t % bs] = vals["v_seq"][b][t]
    got = oat.decode_attention(vals["q"], kp, vp, tables, wl.seq_lens, "f32", wl.scale)
    # Pure-Python loops with math.exp and a running (online) softmax.
    for b in range(wl.batch):
        for hh in range(h):
            m, lsum, acc = -math.inf, 0.0, [0.0] * d
            for t in range(int(wl.seq_lens[b])):
                kr = vals["k_seq"][b][t][hh]
                s = sum(float(vals["q"][b, hh, i]) * float(kr[i]) for i in range(d)) * wl.scale
                if s > m:
                    c = math.exp(m - s) if m > -math.inf else 0.0
                    lsum, acc, m = lsum * c, [a * c for a in acc], s
                p = math.exp(s - m)
                lsum += p
                vr = vals["v_seq"][b][t][hh]
                acc = [a + p * float(vr[i]) for i, a in enumerate(acc)]
            want = np.array(acc) / lsum
            assert np.max(np.abs(got[b, hh] - want)) < 1e-12


def test_zero_length_gives_zero_row():
    rng = np.random.default_rng(2)
    q, kp, vp, tab, L, _, _ = _paged_case(rng, [0 + 1, 4], 2, 8, 4)
    L = np.array([0, 4], dtype=np.int32)
    out = oat.decode_attention(q, kp, vp, tab, L, "f32")
    assert np.array_equal(out[0], np.zeros_like(out[0]))


def test_pairs_match_full():
    rng = np.random.default_rng(3)
    q, kp, vp, tab, L, _, _ = _paged_case(rng, [5, 30], 3, 8, 4, "f16")
    full = oat.decode_attention(q, kp, vp, tab, L, "f16")
    part = oat.decode_attention_pairs(q, kp, vp, tab, L, "f16", [(0, 2), (1, 0)])
    assert np.array_equal(part[(0, 2)], full[0, 2]) and np.array_equal(part[(1, 0)], full[1, 0])


def test_bf16_decoding_pins():
    # bf16 bit patterns: 0x3F80 = 1.0, 0xC000 = -2.0, 0x7F80 = +inf; RNE of the cast.
    got = oat.to_f64(np.array([0x3F80, 0xC000, 0x7F80], dtype=np.uint16), "bf16")
    assert got[0] == 1.0 and got[1] == -2.0 and np.isinf(got[2])
    x = np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9], dtype=np.float32)
    bits = workloads.to_storage(x, "bf16")
    assert list(bits) == [0x3F80, 0x3F82, 0x3F80]   # ties to even, then round down


def test_pool_append_and_copy():
    rng = np.random.default_rng(9)
    nb, bs, h, d = 5, 4, 2, 8
    for dtype in ("f32", "f16", "bf16"):
        sd = workloads.storage_np_dtype(dtype)
        kp = np.full((nb, bs, h, d), workloads.nan_storage(dtype), dtype=sd)
        vp = kp.copy()
        kn = workloads.to_storage(rng.standard_normal((4, h, d), dtype=np.float32), dtype)
        vn = workloads.to_storage(rng.standard_normal((4, h, d), dtype=np.float32), dtype)
        slots = [7, -1, 0, 19]
        opool.append(kp, vp, kn, vn, slots)
        # Written rows land at (slot // bs, slot % bs); everything else keeps its poison.
        for t, s in enumerate(slots):
            if s >= 0:
                assert kp[s // bs, s % bs].tobytes() == kn[t].tobytes()
                assert vp[s // bs, s % bs].tobytes() == vn[t].tobytes()
        poison = workloads.nan_storage(dtype)
        untouched = np.ones((nb, bs), dtype=bool)
        for s in (7, 0, 19):
            untouched[s // bs, s % bs] = False
        assert all((kp[i, j] == poison).all() if dtype == "bf16" else np.isnan(kp[i, j]).all()
                   for i, j in zip(*np.nonzero(untouched)))
        with pytest.raises(IndexError):
            opool.append(kp, vp, kn[:1], vn[:1], [nb * bs])
        before = kp.copy()
        opool.copy_blocks([kp], [vp], [(1, 3), (4, 2)])
        assert kp[3].tobytes() == before[1].tobytes() and kp[2].tobytes() == before[4].tobytes()
        assert kp[0].tobytes() == before[0].tobytes()
        with pytest.raises(ValueError):
            opool.copy_blocks([kp], [vp], [(1, 3), (3, 2)])
