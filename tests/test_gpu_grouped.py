"""GPU parity of grouped decode (pkv_attention_decode_grouped) through the C interface.

Shared prefixes are attended once per tile of up to 16 sequences with the
matrix cores and each sequence's own positions by the decode kernel; the
merge kernel combines the prefix's partial softmax states with the
sequence's pieces.  The output must match the oracle's attention
within the bounds of pkv_attention_decode (2e-3 fp16; bf16 adds its output
rounding).  Pools are NaN outside written slots, so any read of a wrong
position shows in the output.
"""

import numpy as np
import pytest
import torch

import paged_attention_amd as pkv
import workloads
from oracle import attention as oatt
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


def _grouped(c, work_groups=0, spb=None, tiles=None, min_sharers=2):
    if spb is None:
        spb, tiles = pkv.prefix_tiles(c.tables_np, c.wl.seq_lens, c.wl.block_size, min_sharers)
    out = torch.empty_like(c.q)
    pkv.pkv_attention_decode_grouped(out, c.q, c.k_cache, c.v_cache, c.tables, c.lens, c.wl.max_seq_len,
                                     torch.from_numpy(np.ascontiguousarray(spb)).to(DEV),
                                     torch.from_numpy(np.ascontiguousarray(tiles)).to(DEV), scale=c.wl.scale,
                                     work_groups=work_groups)
    torch.cuda.synchronize()
    return out, spb, tiles


LENS = [41, 60, 45, 9, 100, 77, 41, 300, 2]
SHARERS = [0, 1, 2, 4, 5, 6, 7]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("block_size", [8, 16, 32])
def test_small_groups_match_oracle(dtype, head_dim, block_size):
    wl = workloads.custom(LENS, num_heads=5, head_dim=head_dim, dtype=dtype, block_size=block_size,
                          seed=head_dim + block_size, prefix_len=40, sharers=SHARERS)
    c = pc.build(wl, DEV)
    ref = pc.oracle_out(c)
    for wg in (0, 3, 50):
        out, spb, tiles = _grouped(c, wg)
        assert len(tiles) == 1 and spb[SHARERS].min() == 40 // block_size
        pc.compare(c, out, ref)


def test_no_tiles_is_the_plain_call_bit_for_bit():
    wl = workloads.custom(LENS, num_heads=5, head_dim=128, dtype="f16", block_size=16, seed=3, prefix_len=40,
                          sharers=SHARERS)
    c = pc.build(wl, DEV)
    out, _, _ = _grouped(c, spb=np.zeros(wl.batch, dtype=np.int32), tiles=np.zeros((0, 18), dtype=np.int32))
    plain = pc.run_gpu(c).clone()
    assert torch.equal(out, plain)


def test_group_of_forty_spans_three_tiles():
    rng = np.random.default_rng(5)
    lens = (200 + rng.integers(1, 300, size=44)).tolist()
    wl = workloads.custom(lens, num_heads=8, head_dim=128, dtype="f16", block_size=16, seed=5, prefix_len=200,
                          sharers=list(range(2, 42)))
    c = pc.build(wl, DEV)
    out, spb, tiles = _grouped(c)
    assert tiles[:, 1].tolist() == [16, 16, 8] and spb[2:42].min() == 12
    pc.compare(c, out)


def test_prefix_cow_full_size():
    wl = workloads.prefix_cow()
    c = pc.build(wl, DEV)
    out, spb, tiles = _grouped(c)
    assert len(tiles) == 4 and spb.min() == 32
    err = pc.compare(c, out, record="config 3 prefix+CoW f16 grouped")
    plain = pc.run_gpu(c)
    _log(f"prefix+CoW grouped max err {err:.2e}; grouped vs plain max diff "
         f"{(out.float() - plain.float()).abs().max().item():.2e}")


def test_short_member_is_attended_ungrouped_and_bad_prefix_block_gives_nan():
    bs = 16
    wl = workloads.custom([70, 70, 70, 70, 90], num_heads=4, head_dim=64, dtype="f16", block_size=bs, seed=8,
                          prefix_len=64, sharers=[0, 1, 2, 3])
    c = pc.build(wl, DEV)
    spb, tiles = pkv.prefix_tiles(c.tables_np, wl.seq_lens, bs)
    assert spb.tolist() == [4, 4, 4, 4, 0]
    # member 3 attends only its first 33 positions this call: not longer than the
    # tile's 4-block prefix, so both kernels leave it to the plain path
    lens = np.array([70, 70, 70, 33, 90], dtype=np.int32)
    ref = oatt.decode_attention(c.vals["q"], c.ok_pool, c.ov_pool, c.tables_np, lens, wl.dtype, wl.scale)
    c.lens = torch.from_numpy(lens).to(DEV)
    out, _, _ = _grouped(c, spb=spb, tiles=tiles)
    pc.compare(c, out, ref)
    # a prefix block id outside the pool in the row the tile reads: the tile's members are NaN
    lead = int(tiles[0, 2])
    bad_tables = c.tables_np.copy()
    bad_tables[lead, 1] = wl.num_blocks + 5
    c.tables = torch.from_numpy(bad_tables).to(DEV)
    spb3, tiles3 = spb.copy(), tiles.copy()
    spb3[3] = 0                                      # member 3 (33 positions) stays off the tile
    tiles3[0, 1] = 3
    tiles3[0, 5] = -1
    out, _, _ = _grouped(c, spb=spb3, tiles=tiles3)
    members = tiles3[0, 2:2 + tiles3[0, 1]].tolist()
    assert torch.isnan(out[members].float()).all()
    others = [b for b in range(wl.batch) if b not in members]
    got = out[others].float().cpu().numpy()
    assert np.all(np.abs(got - ref[others]) <= pc.tolerance(wl.dtype, ref[others]))


def test_batch_slices_with_groups():
    rng = np.random.default_rng(12)
    lens = rng.integers(1, 40, size=9000)
    lens[:300] = 33 + rng.integers(1, 20, size=300)
    wl = workloads.custom(lens, num_heads=4, head_dim=64, dtype="bf16", block_size=8, seed=12, prefix_len=32,
                          sharers=list(range(300)))
    c = pc.build(wl, DEV, check_pools=False)
    out, spb, tiles = _grouped(c, work_groups=300)
    assert spb[:300].min() == 4 and len(tiles) == 19
    pc.compare(c, out)


# ---- decode ranges and prefix units in one launch ----------------------------
# A 16-bit grouped call whose decode work-groups are fewer than the compute
# units, hold 4 or 8 wavefronts and whose batch fits one launch runs its
# prefix units in the same grid, after the ranges; otherwise (and always for
# 8-bit caches) the prefix has a launch of its own.  Both must meet the
# decode bound against the oracle.  Counts below the compute units take the
# one-launch path (with more parts per tile and head the more units are
# free); counts at or above it the other.  Shapes with an odd head count in
# three tiles give an odd number of units at one part: with 8 wavefronts the
# last work-group holds one unit and an idle half.  The 8-bit shapes run the
# same counts through the two-launch path.

ONE_LAUNCH_SHAPES = [("dense", "f16", 32, 128, 16), ("dense", "bf16", 16, 128, 8), ("dense", "f16", 32, 64, 32),
                     ("dense", "bf16", 31, 128, 16), ("fp8", "f16", 32, 128, 16), ("i8", "bf16", 64, 64, 8),
                     ("fp8", "bf16", 61, 128, 32), ("i8", "f16", 29, 128, 16)]


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("kv,dtype,num_heads,head_dim,block_size", ONE_LAUNCH_SHAPES)
def test_one_launch_grouped_matches_oracle(kv, dtype, num_heads, head_dim, block_size):
    lens = LENS + [200 + 7 * i for i in range(30)]
    sharers = SHARERS + list(range(len(LENS), len(LENS) + 30))  # 37 sharers: three tiles
    wl = workloads.custom(lens, num_heads=num_heads, head_dim=head_dim, dtype=dtype, block_size=block_size,
                          seed=num_heads + head_dim + block_size, prefix_len=40, sharers=sharers)
    c = pc.build(wl, DEV, kv=kv)
    ref = pc.oracle_out(c)
    spb, tiles = pkv.prefix_tiles(c.tables_np, wl.seq_lens, block_size)
    assert len(tiles) == 3 and spb[sharers].min() == 40 // block_size
    cus = _cus()
    run = _grouped if kv == "dense" else _grouped_quant
    for wg in (0, 3, 50, cus - 8, cus - 1, cus, cus + 44):
        _log(f"one-launch grouped {kv} {dtype} H={num_heads} D={head_dim} BS={block_size} work_groups={wg}")
        out, _, _ = run(c, wg, spb, tiles)
        pc.compare(c, out, ref)
        _poison_newest(c)
        out = _grouped_fused(c, wg, spb, tiles)
        _assert_pools(c)
        pc.compare(c, out, ref)


@pytest.mark.parametrize("kv,dtype", [("dense", "f16"), ("fp8", "bf16")])
@pytest.mark.parametrize("batch", [1024, 1025])
def test_one_launch_grouped_batch_limit(kv, dtype, batch):
    # Up to 1024 sequences per head slice the prefix units share the decode
    # launch; one more and the prefix has a launch of its own.  Both sides of
    # the limit, 32 heads of 128 (8 wavefronts per work-group), against the
    # oracle: groups of 40 sequences share a 32-token prefix.
    rng = np.random.default_rng(batch)
    lens = (33 + rng.integers(1, 40, size=batch)).tolist()
    sharers = [b for b in range(batch) if b % 50 < 40]
    wl = workloads.custom(lens, num_heads=32, head_dim=128, dtype=dtype, block_size=16, seed=batch,
                          prefix_len=32, sharers=sharers)
    c = pc.build(wl, DEV, kv=kv, check_pools=False)
    spb, tiles = pkv.prefix_tiles(c.tables_np, wl.seq_lens, 16)
    assert spb[sharers].min() == 2 and len(tiles) >= 2
    run = _grouped if kv == "dense" else _grouped_quant
    out, _, _ = run(c, 0, spb, tiles)
    pc.compare(c, out)


def test_one_launch_grouped_is_deterministic_and_reads_no_stale_state():
    # Two calls with the same arguments give the same bytes; a call after one
    # with other lengths (a different prefix share and parts) as well.
    wl = workloads.custom(LENS + [150] * 12, num_heads=32, head_dim=128, dtype="f16", block_size=16, seed=31,
                          prefix_len=40, sharers=SHARERS + list(range(len(LENS), len(LENS) + 12)))
    c = pc.build(wl, DEV)
    spb, tiles = pkv.prefix_tiles(c.tables_np, wl.seq_lens, 16)
    first, _, _ = _grouped(c, 0, spb, tiles)
    first = first.clone()
    other = workloads.custom([90] * 40, num_heads=32, head_dim=128, dtype="f16", block_size=16, seed=32,
                             prefix_len=80, sharers=list(range(40)))
    co = pc.build(other, DEV)
    out_o, _, _ = _grouped(co, 0)
    pc.compare(co, out_o)
    again, _, _ = _grouped(c, 0, spb, tiles)
    assert torch.equal(first.view(torch.uint8), again.view(torch.uint8))


# ---- 8-bit caches (pkv_attention_decode_grouped_quant) -----------------------

def _grouped_quant(c, work_groups=0, spb=None, tiles=None, min_sharers=2):
    if spb is None:
        spb, tiles = pkv.prefix_tiles(c.tables_np, c.wl.seq_lens, c.wl.block_size, min_sharers)
    out = torch.empty_like(c.q)
    pkv.pkv_attention_decode_grouped_quant(out, c.q, c.k_cache, c.v_cache, c.k_scales, c.v_scales, c.tables, c.lens,
                                           c.wl.max_seq_len, torch.from_numpy(np.ascontiguousarray(spb)).to(DEV),
                                           torch.from_numpy(np.ascontiguousarray(tiles)).to(DEV), c.kv,
                                           scale=c.wl.scale, work_groups=work_groups)
    torch.cuda.synchronize()
    return out, spb, tiles


@pytest.mark.parametrize("fmt", ["i8", "fp8"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("head_dim,block_size", [(64, 8), (128, 16), (64, 32), (128, 8)])
def test_small_groups_quant_match_oracle(fmt, dtype, head_dim, block_size):
    # The oracle attends over the exactly dequantised rows; the grouped call
    # meets the same bound as pkv_attention_decode_quant.
    wl = workloads.custom(LENS, num_heads=5, head_dim=head_dim, dtype=dtype, block_size=block_size,
                          seed=head_dim + block_size + 1, prefix_len=40, sharers=SHARERS)
    c = pc.build(wl, DEV, kv=fmt)
    ref = pc.oracle_out(c)
    for wg in (0, 3, 50):
        out, spb, tiles = _grouped_quant(c, wg)
        assert len(tiles) == 1 and spb[SHARERS].min() == 40 // block_size
        pc.compare(c, out, ref)


def test_quant_no_tiles_is_the_plain_call_bit_for_bit():
    wl = workloads.custom(LENS, num_heads=5, head_dim=128, dtype="f16", block_size=16, seed=4, prefix_len=40,
                          sharers=SHARERS)
    c = pc.build(wl, DEV, kv="fp8")
    out, _, _ = _grouped_quant(c, spb=np.zeros(wl.batch, dtype=np.int32), tiles=np.zeros((0, 18), dtype=np.int32))
    plain = pc.run_gpu(c).clone()
    assert torch.equal(out, plain)


@pytest.mark.parametrize("fmt", ["fp8", "i8"])
def test_prefix_cow_full_size_grouped_quant(fmt):
    wl = workloads.prefix_cow()
    c = pc.build(wl, DEV, kv=fmt)
    out, spb, tiles = _grouped_quant(c)
    assert len(tiles) == 4 and spb.min() == 32
    err = pc.compare(c, out, record=f"config 3 prefix+CoW {fmt} cache grouped")
    _log(f"prefix+CoW {fmt} grouped max err {err:.2e}")


def test_quant_bad_prefix_block_gives_nan_and_refuses_f32_queries():
    bs = 16
    wl = workloads.custom([70, 70, 70, 90], num_heads=4, head_dim=64, dtype="f16", block_size=bs, seed=18,
                          prefix_len=64, sharers=[0, 1, 2])
    c = pc.build(wl, DEV, kv="i8")
    ref = pc.oracle_out(c)
    spb, tiles = pkv.prefix_tiles(c.tables_np, wl.seq_lens, bs)
    assert spb.tolist() == [4, 4, 4, 0]
    out, _, _ = _grouped_quant(c, spb=spb, tiles=tiles)
    pc.compare(c, out, ref)
    lead = int(tiles[0, 2])
    bad_tables = c.tables_np.copy()
    bad_tables[lead, 2] = wl.num_blocks + 1
    c.tables = torch.from_numpy(bad_tables).to(DEV)
    out, _, _ = _grouped_quant(c, spb=spb, tiles=tiles)
    members = tiles[0, 2:2 + tiles[0, 1]].tolist()
    assert torch.isnan(out[members].float()).all()
    got = out[3].float().cpu().numpy()
    assert np.all(np.abs(got - ref[3]) <= pc.tolerance(wl.dtype, ref[3]))
    # f32 queries have no matrix-core path
    q32 = c.q.float()
    with pytest.raises(pkv.InvalidArgument):
        pkv.pkv_attention_decode_grouped_quant(torch.empty_like(q32), q32, c.k_cache, c.v_cache, c.k_scales,
                                               c.v_scales, c.tables, c.lens, wl.max_seq_len,
                                               torch.from_numpy(spb).to(DEV), torch.from_numpy(tiles).to(DEV), "i8")


# ---- scatter + grouped decode in one launch ----------------------------------
# (pkv_append_attention_decode_grouped[_quant]).  As for the ungrouped fused
# call: the slot of each sequence's newest token is poisoned, the fused call
# stores the row again, and the pools must come back bit-identical to the
# oracle's; the output meets the decode bound and equals the separate grouped
# call (same kernels and schedule) bit for bit.

from tests.test_gpu_fused import _assert_pools, _poison_newest  # noqa: E402


def _grouped_fused(c, work_groups, spb, tiles):
    kn = pc.to_device(c.dec_k, c.wl.dtype, DEV)
    vn = pc.to_device(c.dec_v, c.wl.dtype, DEV)
    out = torch.empty_like(c.q)
    spb_d = torch.from_numpy(np.ascontiguousarray(spb)).to(DEV)
    tiles_d = torch.from_numpy(np.ascontiguousarray(tiles)).to(DEV)
    if c.kv == "dense":
        pkv.pkv_append_attention_decode_grouped(out, c.q, kn, vn, c.k_cache, c.v_cache, c.tables, c.lens,
                                                c.wl.max_seq_len, spb_d, tiles_d, scale=c.wl.scale,
                                                work_groups=work_groups)
    else:
        pkv.pkv_append_attention_decode_grouped_quant(out, c.q, kn, vn, c.k_cache, c.v_cache, c.k_scales, c.v_scales,
                                                      c.tables, c.lens, c.wl.max_seq_len, spb_d, tiles_d, c.kv,
                                                      scale=c.wl.scale, work_groups=work_groups)
    torch.cuda.synchronize()
    return out


FUSED_CASES = [("dense", "f16", 128, 16), ("dense", "bf16", 64, 8), ("dense", "f16", 64, 32),
               ("i8", "f16", 128, 16), ("fp8", "bf16", 128, 8), ("fp8", "f16", 64, 32)]


@pytest.mark.parametrize("kv,dtype,head_dim,block_size", FUSED_CASES)
def test_fused_grouped_matches_oracle_and_separate_calls(kv, dtype, head_dim, block_size):
    wl = workloads.custom(LENS, num_heads=5, head_dim=head_dim, dtype=dtype, block_size=block_size,
                          seed=head_dim + block_size + 2, prefix_len=40, sharers=SHARERS)
    c = pc.build(wl, DEV, kv=kv)
    ref = pc.oracle_out(c)
    spb, tiles = pkv.prefix_tiles(c.tables_np, wl.seq_lens, block_size)
    assert len(tiles) == 1 and spb[SHARERS].min() == 40 // block_size
    separate = (_grouped(c, 0, spb, tiles) if kv == "dense" else _grouped_quant(c, 0, spb, tiles))[0].clone()
    for wg in (0, 3, 50):
        _poison_newest(c)
        out = _grouped_fused(c, wg, spb, tiles)
        _assert_pools(c)
        pc.compare(c, out, ref)
        if wg == 0:
            assert torch.equal(out.view(torch.uint8), separate.view(torch.uint8))


@pytest.mark.parametrize("kv", ["dense", "fp8"])
def test_fused_grouped_prefix_cow_full_size(kv):
    wl = workloads.prefix_cow()
    c = pc.build(wl, DEV, kv=kv)
    ref = pc.oracle_out(c)
    spb, tiles = pkv.prefix_tiles(c.tables_np, wl.seq_lens, wl.block_size)
    assert len(tiles) == 4 and spb.min() == 32
    _poison_newest(c)
    out = _grouped_fused(c, 0, spb, tiles)
    _assert_pools(c)
    err = pc.compare(c, out, ref, record=f"config 3 prefix+CoW {kv} cache grouped, append fused")
    _log(f"prefix+CoW {kv} fused grouped max err {err:.2e}")


def test_fused_grouped_refuses_missing_rows():
    wl = workloads.custom([70, 70, 90], num_heads=4, head_dim=64, dtype="f16", block_size=16, seed=19,
                          prefix_len=64, sharers=[0, 1])
    c = pc.build(wl, DEV)
    spb, tiles = pkv.prefix_tiles(c.tables_np, wl.seq_lens, 16)
    out = torch.empty_like(c.q)
    spb_d, tiles_d = torch.from_numpy(spb).to(DEV), torch.from_numpy(tiles).to(DEV)
    with pytest.raises(pkv.InvalidArgument):
        pkv.pkv_append_attention_decode_grouped(out, c.q, c.q[:, :2], c.q[:, :2], c.k_cache, c.v_cache, c.tables,
                                                c.lens, wl.max_seq_len, spb_d, tiles_d)


def test_fused_grouped_bad_block_writes_nothing():
    # A member whose block for position L - 1 is outside the pool stores
    # nothing and gets a NaN row; the other sequences, grouped or not, are
    # unaffected and rewrite their newest rows with the same bytes.
    bs = 16
    wl = workloads.custom([70, 70, 70, 90], num_heads=4, head_dim=64, dtype="f16", block_size=bs, seed=23,
                          prefix_len=64, sharers=[0, 1, 2])
    c = pc.build(wl, DEV)
    ref = pc.oracle_out(c)
    spb, tiles = pkv.prefix_tiles(c.tables_np, wl.seq_lens, bs)
    assert spb.tolist() == [4, 4, 4, 0]
    tables = c.tables.clone()
    tables[1, (70 - 1) // bs] = wl.num_blocks + 3
    c.tables = tables
    before_k, before_v = c.k_cache.clone(), c.v_cache.clone()
    out = _grouped_fused(c, 0, spb, tiles)
    assert torch.isnan(out[1].float()).all()
    others = [0, 2, 3]
    got = out[others].float().cpu().numpy()
    assert np.all(np.abs(got - ref[others]) <= pc.tolerance(wl.dtype, ref[others]))
    assert torch.equal(c.k_cache.view(torch.int16), before_k.view(torch.int16))
    assert torch.equal(c.v_cache.view(torch.int16), before_v.view(torch.int16))
