"""GPU parity of pkv_swap_blocks: blocks swapped out to pinned host memory and
back in at other ids are bit-identical to the oracle's copies, and decode
attention through the remapped tables gives the same bits as before."""

import ctypes

import numpy as np
import pytest
import torch

import paged_attention_amd as pkv
import workloads
from oracle import pool as opool
from tests import paged_case as pc

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _swap_round_trip(kv):
    wl = workloads.custom([40, 300, 17, 129], num_heads=8, head_dim=128, dtype="f16", block_size=16, seed=61,
                          num_blocks=64)
    c = pc.build(wl, DEV, kv=kv)
    before = pc.run_gpu(c).clone()
    dev_pools = [c.k_cache, c.v_cache] + ([c.k_scales, c.v_scales] if kv != "dense" else [])
    ora_pools = [c.ok_pool, c.ov_pool] + ([c.ok_scales, c.ov_scales] if kv != "dense" else [])
    # swap space: a host allocator over 32 pinned blocks per pool
    host_alloc = pkv.BlockAllocator(32, wl.block_size, list(range(31, -1, -1)))
    host = [torch.zeros((32,) + tuple(p.shape[1:]), dtype=p.dtype).pin_memory() for p in dev_pools]
    ora_host = [np.zeros((32,) + tuple(p.shape[1:]), dtype=p.dtype) for p in ora_pools]
    victim = 1                                           # preempt sequence 1 (300 tokens, 19 blocks)
    row = [int(b) for b in c.tables_np[victim, : c.nblk[victim]]]
    host_row = [host_alloc.alloc() for _ in row]
    out_pairs = list(zip(row, host_row))
    pt = torch.tensor(out_pairs, dtype=torch.int32).pin_memory()
    for group in ([0, 1], [2, 3]) if kv != "dense" else ([0, 1],):
        pkv.pkv_swap_blocks([host[i] for i in group], [dev_pools[i] for i in group], pt)
        opool.swap_blocks([ora_host[i] for i in group], [ora_pools[i] for i in group], out_pairs)
    torch.cuda.synchronize()
    for hp, op in zip(host, ora_host):
        assert np.array_equal(hp.numpy().view(np.uint8), op.view(np.uint8))
    # the device blocks go back to the pool and are overwritten by someone else
    c.palloc.release(row)
    for b in row:
        for p in dev_pools:
            p[b] = 0 if p.dtype == torch.uint8 else float("nan")
    # swap in at fresh device ids
    new_row = [c.palloc.alloc() for _ in row]
    in_pairs = list(zip(host_row, new_row))
    pt = torch.tensor(in_pairs, dtype=torch.int32, device=DEV)
    for group in ([0, 1], [2, 3]) if kv != "dense" else ([0, 1],):
        pkv.pkv_swap_blocks([dev_pools[i] for i in group], [host[i] for i in group], pt)
    torch.cuda.synchronize()
    tables = c.tables.clone()
    tables[victim, : len(new_row)] = torch.tensor(new_row, dtype=torch.int32)
    out = torch.empty_like(c.q)
    if kv == "dense":
        pkv.pkv_attention_decode(out, c.q, c.k_cache, c.v_cache, tables, c.lens, wl.max_seq_len, scale=wl.scale)
    else:
        pkv.pkv_attention_decode_quant(out, c.q, c.k_cache, c.v_cache, c.k_scales, c.v_scales, tables, c.lens,
                                       wl.max_seq_len, kv, scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), before.view(torch.int16))
    for b_old, b_new in zip(row, new_row):
        for dp, op in zip(dev_pools, ora_pools):
            assert np.array_equal(dp[b_new].cpu().numpy().view(np.uint8), op[b_old].view(np.uint8))


@pytest.mark.parametrize("kv", ["dense", "fp8"])
def test_swap_out_and_in_round_trip(kv):
    _swap_round_trip(kv)


def test_device_to_device_and_bad_ids():
    nb, bs, h, d = 12, 16, 4, 128
    rng = np.random.default_rng(4)
    src = torch.from_numpy(rng.integers(0, 256, (nb, bs, h, d)).astype(np.uint8)).to(DEV)
    dst = torch.zeros_like(src)
    pairs = [(1, 7), (4, 2), (11, 0), (nb + 3, 5), (3, -1)]
    pkv.pkv_swap_blocks([dst], [src], torch.tensor(pairs, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    want = np.zeros((nb, bs, h, d), dtype=np.uint8)
    opool.swap_blocks([want], [src.cpu().numpy()], pairs[:3])
    assert np.array_equal(dst.cpu().numpy(), want)


def test_pageable_host_memory_is_refused():
    # A plain (pageable) host buffer must be rejected on the host, never
    # handed to a kernel.
    lib = pkv._lib
    dev = torch.zeros((4, 4096), dtype=torch.uint8, device=DEV)
    pageable = np.zeros((4, 4096), dtype=np.uint8)
    pairs = torch.tensor([[0, 1]], dtype=torch.int32, device=DEV)
    darr = (ctypes.c_void_p * 1)(pageable.ctypes.data)
    sarr = (ctypes.c_void_p * 1)(dev.data_ptr())
    st = lib.pkv_swap_blocks(darr, sarr, 1, ctypes.c_void_p(pairs.data_ptr()), 1, 4, 4, 4096,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == pkv.PKV_ERR_INVALID
    assert "pinned" in lib.pkv_last_error().decode()
    with pytest.raises(pkv.InvalidArgument):
        pkv.pkv_swap_blocks([torch.zeros((4, 4096), dtype=torch.uint8)], [dev], pairs)
