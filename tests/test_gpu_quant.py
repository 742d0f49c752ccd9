"""GPU parity of the 8-bit K/V cache (int8, OCP FP8 E4M3) through the C interface.

Codes and scales written by pkv_append_quant must equal the oracle's bit for
bit (the quantisation decisions are made in float32 on both sides); decode
attention over the 8-bit cache must match the oracle's attention over the
exactly dequantised rows within the same bounds as a 16/32-bit cache (1e-5
fp32, 2e-3 fp16, 2e-3 plus output rounding for bf16).
"""

import numpy as np
import pytest
import torch

import paged_attention_amd as pkv
import workloads
from oracle import pool as opool
from oracle import quant as oq
from tests import paged_case as pc

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _log(msg):
    print(msg, flush=True)


def _append_both(rows_k, rows_v, slots, nb, bs, h, d, dt, fmt):
    """Quantising scatter on the GPU and in the oracle from the same stored rows."""
    okp = np.full((nb, bs, h, d), 0x55, dtype=np.uint8)
    ovp = okp.copy()
    oks = np.full((nb, h, bs), np.nan, dtype=np.float32)
    ovs = oks.copy()
    kc = torch.full((nb, bs, h, d), 0x55, dtype=torch.uint8, device=DEV)
    vc = torch.full_like(kc, 0x55)
    ks = torch.full((nb, h, bs), float("nan"), dtype=torch.float32, device=DEV)
    vs = torch.full_like(ks, float("nan"))
    pkv.pkv_append_quant(pc.to_device(rows_k, dt, DEV), pc.to_device(rows_v, dt, DEV),
                         torch.tensor(slots, dtype=torch.int64, device=DEV), kc, vc, ks, vs, fmt)
    torch.cuda.synchronize()
    keep = [s if 0 <= s < nb * bs else -1 for s in slots]
    oq.append(okp, ovp, oks, ovs, rows_k, rows_v, keep, dt, fmt)
    return (kc, vc, ks, vs), (okp, ovp, oks, ovs)


def _assert_same(dev, ora):
    kc, vc, ks, vs = dev
    okp, ovp, oks, ovs = ora
    assert np.array_equal(kc.cpu().numpy(), okp)
    assert np.array_equal(vc.cpu().numpy(), ovp)
    assert np.array_equal(pc.to_bits(ks), pc.storage_bits(oks))
    assert np.array_equal(pc.to_bits(vs), pc.storage_bits(ovs))


@pytest.mark.parametrize("fmt", ["i8", "fp8"])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_append_quant_bit_exact(fmt, dt, d):
    rng = np.random.default_rng(100 + d)
    nb, bs, h, T = 7, 8, 3, 40
    scale = np.exp(rng.uniform(-8, 8, (T, h, 1))) if dt == "f32" else np.exp(rng.uniform(-4, 4, (T, h, 1)))
    raw = (rng.standard_normal((T, h, d)) * scale).astype(np.float32)
    raw[3] = 0.0                                  # zero rows: scale 0, codes 0
    raw[4, 1, :] = -0.0
    qmax = oq.QMAX[fmt]
    # Rows whose largest magnitude is QMAX: scale 1, codes straight from the
    # rounding rule, ties included.
    ties = np.array([qmax, 63.5, -0.5, 1.5, 2.5, -2.5, 1.0625, 1.1875, 0.0009765625, -3.0], dtype=np.float32)
    raw[5, 0, : len(ties)] = ties
    raw[5, 0, len(ties):] = 0.25
    raw[6, 2, 0] = -qmax
    if dt == "f32":                               # magnitudes only float32 holds
        raw[9] = rng.standard_normal((h, d)) * 1e30
        raw[10] = rng.standard_normal((h, d)) * 1e-30
    kn = workloads.to_storage(raw, dt)
    vn = workloads.to_storage((raw[::-1] * 0.5).copy(), dt)
    slots = list(rng.permutation(nb * bs)[:T].astype(np.int64))
    slots[7] = -1                                 # skipped
    slots[8] = nb * bs + 3                        # out of range: skipped
    dev, ora = _append_both(kn, vn, slots, nb, bs, h, d, dt, fmt)
    _assert_same(dev, ora)


@pytest.mark.parametrize("fmt", ["i8", "fp8"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("head_dim,block_size", [(64, 8), (128, 16), (64, 32), (128, 32)])
def test_small_cases(fmt, dtype, head_dim, block_size):
    wl = workloads.custom([1, 7, 8, 9, 33, 100, 257], num_heads=5, head_dim=head_dim, dtype=dtype,
                          block_size=block_size, seed=head_dim + block_size)
    c = pc.build(wl, DEV, kv=fmt)
    ref = pc.oracle_out(c)
    for wg in (0, 7, 64):
        pc.compare(c, pc.run_gpu(c, work_groups=wg), ref)


# Two chunk streams per work-group: where both sets of wavefronts fit a
# work-group of 8 (32 heads of 128, 64 of 64), a range's chunks alternate
# between them and stream 1 hands its state to stream 0 at every segment's
# end; 33 heads of 128 (5 wavefronts) keep one stream.  Lengths put the last
# chunk of a segment on either stream and give segments of one chunk (stream
# 1 idle); counts from one range (every sequence a segment of it) up.  The
# fused append+decode call must store each new row from the stream that
# reads it back: the pools come back bit-identical to the oracle's.
DUAL_LENS = [1, 8, 9, 16, 17, 24, 25, 40, 333, 1000, 2, 64]


@pytest.mark.parametrize("fmt,dtype,num_heads,head_dim", [("fp8", "f16", 32, 128), ("i8", "bf16", 64, 64),
                                                         ("fp8", "f32", 32, 64), ("i8", "f16", 33, 128)])
def test_two_chunk_streams_per_work_group(fmt, dtype, num_heads, head_dim):
    from tests.test_gpu_fused import _assert_pools, _poison_newest, _run_fused
    wl = workloads.custom(DUAL_LENS, num_heads=num_heads, head_dim=head_dim, dtype=dtype, block_size=16,
                          seed=num_heads + head_dim)
    c = pc.build(wl, DEV, kv=fmt)
    ref = pc.oracle_out(c)
    for wg in (1, 2, 3, 5, 24, 448, 512, 0):
        _log(f"two streams {fmt} {dtype} H={num_heads} D={head_dim} work_groups={wg}")
        pc.compare(c, pc.run_gpu(c, work_groups=wg), ref)
        _poison_newest(c)
        out = _run_fused(c, work_groups=wg)
        _assert_pools(c)
        pc.compare(c, out, ref)


@pytest.mark.parametrize("fmt", ["i8", "fp8"])
def test_many_heads_span_head_slices(fmt):
    # 160 heads x 128 at 8 heads per wavefront = 20 wavefronts: 3 head slices.
    wl = workloads.custom([50, 300, 1], num_heads=160, head_dim=128, dtype="bf16", block_size=16, seed=77)
    c = pc.build(wl, DEV, kv=fmt)
    pc.compare(c, pc.run_gpu(c))


@pytest.mark.parametrize("fmt", ["i8", "fp8"])
def test_llama7b_layer_full_size(fmt):
    wl = workloads.llama7b_layer()
    c = pc.build(wl, DEV, kv=fmt)
    err = pc.compare(c, pc.run_gpu(c), record=f"config 2 7B layer {fmt} cache")
    _log(f"7B layer {fmt} max err {err:.2e}")


def test_prefix_cow_full_size_fp8():
    wl = workloads.prefix_cow()
    c = pc.build(wl, DEV, kv="fp8")
    assert len(c.cow_pairs) == wl.batch - 1
    err = pc.compare(c, pc.run_gpu(c), record="config 3 prefix+CoW fp8 cache")
    _log(f"prefix+CoW fp8 max err {err:.2e}")


def test_long13b_full_size_i8():
    wl = workloads.long13b(16)
    c = pc.build(wl, DEV, kv="i8")
    err = pc.compare(c, pc.run_gpu(c), record="config 4 13B long bf16 block 16 i8 cache")
    assert err <= 2e-3
    _log(f"13B long i8 max err {err:.2e}")


def test_edge_lengths_and_bad_entries_quant():
    wl = workloads.custom([0, 1, 40, 77], num_heads=4, head_dim=64, dtype="f16", block_size=16, seed=9)
    c = pc.build(wl, DEV, kv="fp8")
    out = pc.run_gpu(c)
    assert torch.count_nonzero(out[0]) == 0
    pc.compare(c, out)
    lens = torch.tensor([-1, 78, 40, 1], dtype=torch.int32, device=DEV)
    out = torch.zeros_like(c.q)
    pkv.pkv_attention_decode_quant(out, c.q, c.k_cache, c.v_cache, c.k_scales, c.v_scales, c.tables, lens, 77,
                                   "fp8", scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.isnan(out[0]).all() and torch.isnan(out[1]).all()
    assert torch.isfinite(out[2]).all() and torch.isfinite(out[3]).all()
    tables = c.tables.clone()
    tables[2, 1] = wl.num_blocks + 5
    tables[3, 0] = -3
    out = torch.zeros_like(c.q)
    pkv.pkv_attention_decode_quant(out, c.q, c.k_cache, c.v_cache, c.k_scales, c.v_scales, tables, c.lens,
                                   wl.max_seq_len, "fp8", scale=wl.scale, work_groups=5)
    torch.cuda.synchronize()
    assert torch.isnan(out[2]).all() and torch.isnan(out[3]).all()
    ref = pc.oracle_out(c)
    got = out[:2].float().cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - ref[:2])) <= 2e-3


def test_quant_copy_blocks_moves_codes_and_scales():
    # Copy-on-write of an 8-bit cache: one pkv_copy_blocks call for the code
    # pools, one for the scale pools, bit-exact.
    nl, nb, bs, h, d = 3, 9, 16, 4, 128
    rng = np.random.default_rng(8)
    kp = [rng.integers(0, 256, (nb, bs, h, d)).astype(np.uint8) for _ in range(nl)]
    vp = [rng.integers(0, 256, (nb, bs, h, d)).astype(np.uint8) for _ in range(nl)]
    ksc = [rng.standard_normal((nb, h, bs)).astype(np.float32) for _ in range(nl)]
    vsc = [rng.standard_normal((nb, h, bs)).astype(np.float32) for _ in range(nl)]
    dk = [torch.from_numpy(x).to(DEV) for x in kp]
    dv = [torch.from_numpy(x).to(DEV) for x in vp]
    dks = [torch.from_numpy(x).to(DEV) for x in ksc]
    dvs = [torch.from_numpy(x).to(DEV) for x in vsc]
    pairs = [(1, 7), (4, 2), (8, 0)]
    pt = torch.tensor(pairs, dtype=torch.int32, device=DEV)
    pkv.pkv_copy_blocks(dk, dv, pt)
    pkv.pkv_copy_blocks(dks, dvs, pt)
    torch.cuda.synchronize()
    opool.copy_blocks(kp, vp, pairs)
    opool.copy_blocks(ksc, vsc, pairs)
    for i in range(nl):
        assert np.array_equal(dk[i].cpu().numpy(), kp[i]) and np.array_equal(dv[i].cpu().numpy(), vp[i])
        assert np.array_equal(dks[i].cpu().numpy(), ksc[i]) and np.array_equal(dvs[i].cpu().numpy(), vsc[i])


def test_prepared_quant_calls_match_direct_calls():
    wl = workloads.custom([90, 1000, 3], num_heads=8, head_dim=128, dtype="f16", block_size=16, seed=22)
    c = pc.build(wl, DEV, kv="i8")
    ref = pc.run_gpu(c).clone()
    out = torch.empty_like(c.q)
    prep = pkv.PreparedDecodeQuant(out, c.q, c.k_cache, c.v_cache, c.k_scales, c.v_scales, c.tables, c.lens,
                                   wl.max_seq_len, "i8", scale=wl.scale)
    h_tables, h_lens = c.tables.cpu().pin_memory(), c.lens.cpu().pin_memory()
    for tb, ln in ((c.tables, c.lens), (h_tables, h_lens)):
        out.fill_(float("nan"))
        prep.set_metadata(tb, ln)
        prep.launch()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
