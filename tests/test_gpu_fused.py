"""GPU parity of scatter + decode attention in one launch
(pkv_append_attention_decode and its 8-bit form).

Each case is built by the usual path (every token scattered by pkv_append /
pkv_append_quant), then the slot of each sequence's newest token is poisoned
on the device and the fused call stores that token again from the decode
step's rows.  The pools must come back bit-identical to the oracle's, and
the output must match the oracle within the decode bounds and equal the
separate decode call bit for bit.
"""

import numpy as np
import pytest
import torch

import paged_attention_amd as pkv
import workloads
from tests import paged_case as pc

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _newest_slots(c):
    bs = c.wl.block_size
    out = []
    for b, L in enumerate(c.wl.seq_lens):
        L = int(L)
        if L > 0:
            out.append((b, int(c.tables_np[b, (L - 1) // bs]), (L - 1) % bs))
    return out


def _poison_newest(c):
    for _, blk, pos in _newest_slots(c):
        if c.kv == "dense":
            c.k_cache[blk, pos] = float("nan")
            c.v_cache[blk, pos] = float("nan")
        else:
            c.k_cache[blk, pos] = 0x7F
            c.v_cache[blk, pos] = 0x7F
            c.k_scales[blk, :, pos] = float("nan")
            c.v_scales[blk, :, pos] = float("nan")


def _run_fused(c, work_groups=0, tables=None, lens=None, max_len=None):
    kn = pc.to_device(c.dec_k, c.wl.dtype, DEV)
    vn = pc.to_device(c.dec_v, c.wl.dtype, DEV)
    out = torch.empty_like(c.q)
    tables = c.tables if tables is None else tables
    lens = c.lens if lens is None else lens
    max_len = c.wl.max_seq_len if max_len is None else max_len
    if c.kv == "dense":
        pkv.pkv_append_attention_decode(out, c.q, kn, vn, c.k_cache, c.v_cache, tables, lens, max_len,
                                        scale=c.wl.scale, work_groups=work_groups)
    else:
        pkv.pkv_append_attention_decode_quant(out, c.q, kn, vn, c.k_cache, c.v_cache, c.k_scales, c.v_scales,
                                              tables, lens, max_len, c.kv, scale=c.wl.scale,
                                              work_groups=work_groups)
    torch.cuda.synchronize()
    return out


def _assert_pools(c):
    if c.kv == "dense":
        assert np.array_equal(pc.to_bits(c.k_cache), pc.storage_bits(c.ok_pool))
        assert np.array_equal(pc.to_bits(c.v_cache), pc.storage_bits(c.ov_pool))
    else:
        assert np.array_equal(c.k_cache.cpu().numpy(), c.ok_pool)
        assert np.array_equal(c.v_cache.cpu().numpy(), c.ov_pool)
        assert np.array_equal(pc.to_bits(c.k_scales), pc.storage_bits(c.ok_scales))
        assert np.array_equal(pc.to_bits(c.v_scales), pc.storage_bits(c.ov_scales))


CASES = [("dense", "f32", 64, 8), ("dense", "f16", 128, 16), ("dense", "bf16", 128, 32), ("dense", "f16", 64, 32),
         ("i8", "f16", 128, 16), ("i8", "bf16", 64, 8), ("fp8", "f32", 128, 32), ("fp8", "f16", 128, 16)]


@pytest.mark.parametrize("kv,dtype,head_dim,block_size", CASES)
def test_fused_matches_oracle_and_separate_calls(kv, dtype, head_dim, block_size):
    wl = workloads.custom([1, 2, 8, 9, 16, 17, 100, 333, 0], num_heads=6, head_dim=head_dim, dtype=dtype,
                          block_size=block_size, seed=head_dim * 7 + block_size)
    c = pc.build(wl, DEV, kv=kv)
    ref = pc.oracle_out(c)
    separate = pc.run_gpu(c).clone()
    for wg in (0, 5, 64):
        _poison_newest(c)
        out = _run_fused(c, wg)
        _assert_pools(c)
        pc.compare(c, out, ref)
        if wg == 0:
            assert torch.equal(out.view(torch.uint8), separate.view(torch.uint8))


@pytest.mark.parametrize("kv", ["dense", "fp8"])
def test_fused_full_7b_layer(kv):
    wl = workloads.llama7b_layer()
    c = pc.build(wl, DEV, kv=kv)
    ref = pc.oracle_out(c)
    _poison_newest(c)
    out = _run_fused(c)
    _assert_pools(c)
    pc.compare(c, out, ref, record=f"config 2 7B layer fused append ({kv} cache)")


def test_fused_head_slices_and_batch_slices():
    # 160 heads (several head slices) and more sequences than one launch holds
    # (new rows are offset per slice).
    wl = workloads.custom([40, 3, 200], num_heads=160, head_dim=128, dtype="bf16", block_size=16, seed=3)
    c = pc.build(wl, DEV, kv="i8")
    ref = pc.oracle_out(c)
    _poison_newest(c)
    pc.compare(c, _run_fused(c), ref)
    _assert_pools(c)
    rng = np.random.default_rng(31)
    wl = workloads.custom(rng.integers(0, 20, size=9000), num_heads=4, head_dim=64, dtype="f32", block_size=8,
                          seed=31)
    c = pc.build(wl, DEV, check_pools=False)
    ref = pc.oracle_out(c)
    _poison_newest(c)
    pc.compare(c, _run_fused(c, 300), ref)
    _assert_pools(c)


def test_fused_bad_block_writes_nothing():
    wl = workloads.custom([5, 40, 77], num_heads=4, head_dim=64, dtype="f16", block_size=16, seed=9)
    c = pc.build(wl, DEV)
    tables = c.tables.clone()
    tables[1, 2] = wl.num_blocks + 7        # block of position 39: out of range
    before_k = c.k_cache.clone()
    before_v = c.v_cache.clone()
    out = _run_fused(c, tables=tables)
    assert torch.isnan(out[1]).all()
    assert torch.isfinite(out[0]).all() and torch.isfinite(out[2]).all()
    # sequences 0 and 2 rewrote their newest rows with the same bytes; nothing else moved
    assert torch.equal(c.k_cache.view(torch.int16), before_k.view(torch.int16))
    assert torch.equal(c.v_cache.view(torch.int16), before_v.view(torch.int16))


def test_prepared_fused_call():
    wl = workloads.custom([90, 1000, 3], num_heads=8, head_dim=128, dtype="f16", block_size=16, seed=22)
    c = pc.build(wl, DEV, kv="fp8")
    ref = pc.oracle_out(c)
    kn = pc.to_device(c.dec_k, "f16", DEV)
    vn = pc.to_device(c.dec_v, "f16", DEV)
    out = torch.empty_like(c.q)
    prep = pkv.PreparedAppendDecode(out, c.q, kn, vn, c.k_cache, c.v_cache, c.tables, c.lens, wl.max_seq_len,
                                    scale=wl.scale, k_scales=c.k_scales, v_scales=c.v_scales, cache_dtype="fp8")
    h_tables, h_lens = c.tables.cpu().pin_memory(), c.lens.cpu().pin_memory()
    for tb, ln in ((c.tables, c.lens), (h_tables, h_lens)):
        _poison_newest(c)
        prep.set_metadata(tb, ln)
        prep.launch(c.q, kn, vn)
        torch.cuda.synchronize()
        pc.compare(c, out, ref)
        _assert_pools(c)
