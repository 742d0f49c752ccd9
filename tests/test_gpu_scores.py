"""GPU parity of the cumulative attention scores (pkv_attention_decode_scores
and its 8-bit form) against oracle.scores.

The decode output must match the oracle within the decode bounds (the
variant is its own kernel instantiation, so it may round differently from the
plain call in the last place); the updated scores must match the oracle's float64 update within 2e-5 relative
plus 1e-6 absolute (the probabilities come from float32 logits through one
exp2 and one division), positions at or past a sequence's length and rows of
refused lengths must be untouched.
"""

import numpy as np
import pytest
import torch

import paged_attention_amd as pkv
import workloads
from oracle import scores as osc
from tests import paged_case as pc

pytestmark = pytest.mark.gpu

DEV = "cuda"
SENTINEL = -7.0


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _initial_scores(wl, stride, seed):
    rng = np.random.default_rng(seed)
    sc = np.full((wl.batch, stride), SENTINEL, dtype=np.float32)
    for b, L in enumerate(wl.seq_lens):
        sc[b, : int(L)] = rng.uniform(0, 1, int(L))
    return sc


def _oracle_scores(c, prev, decay):
    wl = c.wl
    if c.kv == "dense":
        probs = osc.attention_probs(c.vals["q"], c.ok_pool, c.tables_np, wl.seq_lens, wl.dtype, wl.scale)
    else:
        probs = osc.attention_probs(c.vals["q"], c.ok_pool, c.tables_np, wl.seq_lens, wl.dtype, wl.scale,
                                    k_scales=c.ok_scales, fmt=c.kv)
    return osc.cumulative_update(prev.astype(np.float64), probs, decay)


def _run(c, scores, decay, work_groups=0, lens=None, max_len=None):
    wl = c.wl
    out = torch.empty_like(c.q)
    lens = c.lens if lens is None else lens
    max_len = wl.max_seq_len if max_len is None else max_len
    if c.kv == "dense":
        pkv.pkv_attention_decode_scores(out, c.q, c.k_cache, c.v_cache, c.tables, lens, max_len, scores, decay,
                                        scale=wl.scale, work_groups=work_groups)
    else:
        pkv.pkv_attention_decode_quant_scores(out, c.q, c.k_cache, c.v_cache, c.k_scales, c.v_scales, c.tables,
                                              lens, max_len, c.kv, scores, decay, scale=wl.scale,
                                              work_groups=work_groups)
    torch.cuda.synchronize()
    return out


def _compare_scores(got, want, lens):
    g = got.cpu().numpy().astype(np.float64)
    for b, L in enumerate(lens):
        L = int(L)
        err = np.abs(g[b, :L] - want[b, :L])
        assert np.all(err <= 2e-5 * np.abs(want[b, :L]) + 1e-6), (b, float(err.max()))
        assert np.all(g[b, L:] == SENTINEL)


CASES = [("dense", "f16", 128, 16), ("dense", "bf16", 64, 8), ("dense", "f32", 128, 32), ("fp8", "f16", 128, 16),
         ("i8", "bf16", 64, 32)]


@pytest.mark.parametrize("kv,dtype,head_dim,block_size", CASES)
def test_scores_match_oracle(kv, dtype, head_dim, block_size):
    wl = workloads.custom([1, 7, 8, 9, 100, 333, 0], num_heads=6, head_dim=head_dim, dtype=dtype,
                          block_size=block_size, seed=head_dim + block_size + len(kv))
    c = pc.build(wl, DEV, kv=kv)
    ref_out = pc.oracle_out(c)
    stride = wl.max_seq_len + 5
    for wg, decay in ((0, 0.995), (5, 0.5), (64, 1.0)):
        prev = _initial_scores(wl, stride, wg)
        scores = torch.from_numpy(prev).to(DEV)
        out = _run(c, scores, decay, wg)
        pc.compare(c, out, ref_out)
        _compare_scores(scores, _oracle_scores(c, prev, decay), wl.seq_lens)


def test_scores_full_7b_layer_and_head_slices():
    wl = workloads.llama7b_layer()
    c = pc.build(wl, DEV)
    prev = _initial_scores(wl, wl.max_seq_len, 1)
    scores = torch.from_numpy(prev).to(DEV)
    _run(c, scores, 0.995)
    _compare_scores(scores, _oracle_scores(c, prev, 0.995), wl.seq_lens)
    wl = workloads.custom([50, 300, 1], num_heads=160, head_dim=128, dtype="bf16", block_size=16, seed=77)
    c = pc.build(wl, DEV, kv="fp8")
    prev = _initial_scores(wl, wl.max_seq_len, 2)
    scores = torch.from_numpy(prev).to(DEV)
    _run(c, scores, 0.9)
    _compare_scores(scores, _oracle_scores(c, prev, 0.9), wl.seq_lens)


def test_scores_batch_slices_and_refused_lengths():
    rng = np.random.default_rng(31)
    wl = workloads.custom(rng.integers(0, 20, size=9000), num_heads=4, head_dim=64, dtype="f32", block_size=8,
                          seed=31)
    c = pc.build(wl, DEV, check_pools=False)
    prev = _initial_scores(wl, 24, 3)
    scores = torch.from_numpy(prev).to(DEV)
    _run(c, scores, 0.99, 300)
    _compare_scores(scores, _oracle_scores(c, prev, 0.99), wl.seq_lens)
    # refused lengths (negative, beyond max_seq_len) leave their rows alone
    wl = workloads.custom([0, 1, 40, 77], num_heads=4, head_dim=64, dtype="f16", block_size=16, seed=9)
    c = pc.build(wl, DEV)
    prev = _initial_scores(wl, 80, 4)
    scores = torch.from_numpy(prev).to(DEV)
    lens = torch.tensor([-1, 78, 40, 1], dtype=torch.int32, device=DEV)
    _run(c, scores, 0.5, lens=lens, max_len=77)
    got = scores.cpu().numpy()
    assert np.array_equal(got[0], prev[0]) and np.array_equal(got[1], prev[1])
    assert not np.array_equal(got[2, :40], prev[2, :40])
