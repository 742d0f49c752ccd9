"""Pins of the cumulative attention-score oracle (oracle.scores).

Checked against: torch's softmax in float64 (library); the pinned attention
oracle (probabilities weight the value rows into exactly its output); closed
forms (one token, equal keys, zero query); the mass invariant (each step adds
one unit of mass per sequence, decay scales the old total); untouched
positions; the 8-bit path reducing to the dense one on dequantised keys.
Planted mistakes must each fail a pin.
"""

import math
import types

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oat
from oracle import quant as oq
from oracle import scores as osc
from tests.test_oracle_attention import _paged_case


def run_score_pins(impl):
    failures = []
    rng = np.random.default_rng(17)
    h, d, bs = 3, 16, 4
    # (1) softmax against torch in float64
    q = rng.standard_normal(d)
    keys = rng.standard_normal((23, d))
    got = impl.softmax_probs(q, keys, 0.3)
    want = torch.softmax(torch.from_numpy(0.3 * keys @ q), dim=0).numpy()
    if not np.allclose(got, want, rtol=0, atol=1e-15):
        failures.append("softmax")
    # (2) probabilities weight the values into the attention oracle's output
    lens = [1, 5, 13, 33]
    qq, kp, vp, tab, L, ks, vs = _paged_case(rng, lens, h, d, bs)
    probs = impl.attention_probs(qq, kp, tab, L, "f32", 0.25)
    ref = oat.decode_attention(qq, kp, vp, tab, L, "f32", 0.25)
    for b in range(len(lens)):
        if probs[b].shape != (h, lens[b]):
            failures.append("shape")
            break
        for hh in range(h):
            if not np.allclose(probs[b][hh] @ vs[b][:, hh].astype(np.float64), ref[b, hh], rtol=0, atol=1e-12):
                failures.append("reconstruct")
                break
    # (3) closed forms: one token -> 1; equal keys / zero query -> uniform
    q1, kp1, vp1, tab1, L1, k1, v1 = _paged_case(rng, [1, 9], h, d, bs)
    flat = kp1.reshape(-1, h, d)
    for t in range(9):
        flat[int(tab1[1, t // bs]) * bs + t % bs] = k1[1][0]
    p1 = impl.attention_probs(q1, kp1, tab1, L1, "f32", 0.5)
    if not (np.array_equal(p1[0], np.ones((h, 1))) and np.allclose(p1[1], 1 / 9, rtol=0, atol=1e-15)):
        failures.append("closed-forms")
    pz = impl.attention_probs(np.zeros_like(qq), kp, tab, L, "f32", 0.25)
    if not all(np.allclose(pz[b], 1 / lens[b], rtol=0, atol=1e-15) for b in range(len(lens))):
        failures.append("zero-query")
    # (4) mass invariant, decay, untouched tail
    prev = rng.uniform(0, 2, (len(lens), 40))
    new = impl.cumulative_update(prev, probs, 0.9)
    for b, n in enumerate(lens):
        if not math.isclose(new[b, :n].sum(), 0.9 * prev[b, :n].sum() + 1.0, rel_tol=0, abs_tol=1e-12):
            failures.append("mass")
            break
        if not np.array_equal(new[b, n:], prev[b, n:]):
            failures.append("tail")
            break
    two = impl.cumulative_update(impl.cumulative_update(np.zeros((len(lens), 40)), probs, 1.0), probs, 1.0)
    if not np.allclose(two[0, :1], 2.0, rtol=0, atol=1e-15):
        failures.append("accumulate")
    # (5) 8-bit keys read back as code x scale give the dense probabilities
    kc, kscale = oq.quantize_rows(np.nan_to_num(kp).reshape(-1, h, d), "f32", "fp8")   # poisoned slots -> 0
    kc = kc.reshape(kp.shape)
    kscale = kscale.reshape(kp.shape[0], bs, h).transpose(0, 2, 1).copy()
    deq = oq.dequantize(kc.reshape(-1, h, d), kscale.transpose(0, 2, 1).reshape(-1, h), "fp8").reshape(kp.shape)
    pq = impl.attention_probs(qq, kc, tab, L, "f32", 0.25, k_scales=kscale, fmt="fp8")
    pd = impl.attention_probs(qq, deq, tab, L, "f32", 0.25)
    if not all(np.allclose(pq[b], pd[b], rtol=0, atol=1e-14) for b in range(len(lens))):
        failures.append("quant")
    return failures


def test_oracle_passes_all_pins():
    assert run_score_pins(osc) == []


def _impl(**over):
    ns = types.SimpleNamespace(softmax_probs=osc.softmax_probs, attention_probs=osc.attention_probs,
                               cumulative_update=osc.cumulative_update)
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def _update_variant(kind):
    def upd(scores, probs, decay):
        new = np.array(scores, dtype=np.float64, copy=True)
        for b, p in enumerate(probs):
            n = p.shape[1]
            if kind == "decay-everything":
                new[b] *= decay
                new[b, :n] += p.mean(axis=0)
            elif kind == "decay-after-add":
                new[b, :n] = decay * (new[b, :n] + p.mean(axis=0))
            elif kind == "sum-heads":
                new[b, :n] = decay * new[b, :n] + p.sum(axis=0)
        return new
    return upd


def _probs_variant(kind):
    def probs(q, k_pool, tables, lens, dtype, scale=None, k_scales=None, fmt=None):
        out = osc.attention_probs(q, k_pool, tables, lens, dtype, scale, k_scales, fmt)
        if kind == "head-normalised":
            return [p / np.maximum(p.sum(axis=0, keepdims=True), 1e-300) / p.shape[0] for p in out]
        if kind == "no-scale":
            return osc.attention_probs(q, k_pool, tables, lens, dtype, 1.0, k_scales, fmt)
        if kind == "shifted":
            return [np.roll(p, 1, axis=1) for p in out]
        return out
    return probs


MUTANTS = {
    "decay-everything": lambda: _impl(cumulative_update=_update_variant("decay-everything")),
    "decay-after-add": lambda: _impl(cumulative_update=_update_variant("decay-after-add")),
    "sum-heads": lambda: _impl(cumulative_update=_update_variant("sum-heads")),
    "head-normalised": lambda: _impl(attention_probs=_probs_variant("head-normalised")),
    "no-scale": lambda: _impl(attention_probs=_probs_variant("no-scale")),
    "shifted": lambda: _impl(attention_probs=_probs_variant("shifted")),
}


@pytest.mark.parametrize("kind", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(kind):
    assert run_score_pins(MUTANTS[kind]()), f"mutant {kind} passed every pin"
