"""Builds one workload on both sides for the GPU parity tests.

Product side: the libpkv block allocator on the host, device pools written by
``pkv_append`` / ``pkv_copy_blocks`` (8-bit caches: ``pkv_append_quant`` and
block copies of the code and scale pools).  Oracle side: the oracle allocator
and numpy pools written by ``oracle.pool`` / ``oracle.quant``.  Inputs come from ``workloads`` only;
nothing the HIP path produces is fed to the oracle.

Sequence of operations (the same on both sides):
  1. the first sharer reserves and writes the shared prefix; other sharers
     fork it (their tables point at the same physical blocks);
  2. every sequence reserves its remaining history (length - 1 tokens in
     total); copy-on-write pairs are copied before the new rows are written;
  3. the decode step reserves one slot per sequence (copying again where a
     shared block is written) and writes that token's K/V.
"""

from __future__ import annotations

import numpy as np
import torch

import paged_attention_amd as pkv
import workloads
from oracle import allocator as oalloc
from oracle import attention as oatt
from oracle import pool as opool
from oracle import quant as oquant

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_device(arr: np.ndarray, dtype: str, device):
    arr = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(arr).to(device)


def to_bits(t) -> np.ndarray:
    """Device tensor -> numpy raw bits (exact comparison, NaN payloads included)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.view(torch.int16).numpy()


def storage_bits(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.float32:
        return a.view(np.int32)
    return a.view(np.int16)


class Case:
    pass


def build(wl: workloads.Workload, device="cuda", extra_blocks: int = 1, check_pools: bool = True,
          kv: str = "dense") -> Case:
    """``kv``: "dense" (cache in the workload's dtype) or an 8-bit format ("i8", "fp8")
    whose codes and scales are quantised from the same rows."""
    bs, h, d, dt = wl.block_size, wl.num_heads, wl.head_dim, wl.dtype
    vals = wl.draw_values()
    B = wl.batch
    lens = wl.seq_lens.astype(np.int64)
    sharers = [int(s) for s in wl.sharers]
    shared = set(sharers)
    maxb = wl.max_blocks_per_seq() + extra_blocks

    # logical rows of every sequence: shared prefix first when it shares
    def rows_of(b, which):
        own = vals[which + "_seq"][b]
        if b in shared:
            return np.concatenate([vals[which + "_prefix"], own], axis=0)
        return own

    palloc = pkv.BlockAllocator(wl.num_blocks, bs, wl.free_order)
    oa = oalloc.OracleAllocator(wl.num_blocks, bs, wl.free_order)
    tables = np.zeros((B, maxb), dtype=np.int32)
    nblk = np.zeros(B, dtype=np.int32)
    orows = [[] for _ in range(B)]

    quant = kv != "dense"
    if quant:
        # Unwritten slots hold codes that are not valid data (E4M3 NaN, int8
        # -128) and NaN scales: any read of one shows in the output.
        poison = 0x7F if kv == "fp8" else 0x80
        okp = np.full((wl.num_blocks, bs, h, d), poison, dtype=np.uint8)
        ovp = okp.copy()
        oks = np.full((wl.num_blocks, h, bs), np.nan, dtype=np.float32)
        ovs = oks.copy()
        kc = torch.full((wl.num_blocks, bs, h, d), poison, dtype=torch.uint8, device=device)
        vc = torch.full_like(kc, poison)
        ks = torch.full((wl.num_blocks, h, bs), float("nan"), dtype=torch.float32, device=device)
        vs = torch.full_like(ks, float("nan"))
    else:
        sd = workloads.storage_np_dtype(dt)
        okp = np.full((wl.num_blocks, bs, h, d), workloads.nan_storage(dt), dtype=sd)
        ovp = okp.copy()
        tdt = TORCH_DTYPE[dt]
        kc = torch.full((wl.num_blocks, bs, h, d), float("nan"), dtype=tdt, device=device)
        vc = torch.full_like(kc, float("nan"))

    def write(slots, krows, vrows, pairs):
        if pairs:
            pt = torch.tensor(np.asarray(pairs, dtype=np.int32).reshape(-1, 2), device=device)
            pkv.pkv_copy_blocks([kc], [vc], pt)
            opool.copy_blocks([okp], [ovp], pairs)
            if quant:
                pkv.pkv_copy_blocks([ks], [vs], pt)
                opool.copy_blocks([oks], [ovs], pairs)
        if len(slots):
            st = torch.tensor(np.asarray(slots, dtype=np.int64), device=device)
            if quant:
                pkv.pkv_append_quant(to_device(krows, dt, device), to_device(vrows, dt, device), st, kc, vc, ks, vs,
                                     kv)
                oquant.append(okp, ovp, oks, ovs, krows, vrows, slots, dt, kv)
            else:
                pkv.pkv_append(to_device(krows, dt, device), to_device(vrows, dt, device), st, kc, vc)
                opool.append(okp, ovp, krows, vrows, slots)

    # 1. shared prefix
    done = np.zeros(B, dtype=np.int64)  # tokens already written per sequence
    if sharers and wl.prefix_len > 0:
        s0 = sharers[0]
        pre = wl.prefix_len
        cslots, cpairs = palloc.reserve_batch(tables[s0:s0 + 1], nblk[s0:s0 + 1], [0], [pre])
        oslots, opairs = oa.reserve(orows[s0], 0, pre)
        assert cslots.tolist() == oslots and not opairs and len(cpairs) == 0
        write(oslots, vals["k_prefix"], vals["v_prefix"], [])
        done[s0] = pre
        for s in sharers[1:]:
            row = palloc.fork(tables[s0, : nblk[s0]])
            tables[s, : len(row)] = row
            nblk[s] = len(row)
            orows[s] = oa.fork(orows[s0], len(orows[s0]))
            done[s] = pre
    # 2. remaining history, all sequences at once (ascending order)
    hist = np.maximum(lens - 1 - done, 0)
    cslots, cpairs = palloc.reserve_batch(tables, nblk, done, hist)
    oslots, opairs = oa.reserve_batch(orows, done, hist)
    assert cslots.tolist() == oslots
    assert [tuple(p) for p in cpairs.tolist()] == [tuple(p) for p in opairs]
    krows = [rows_of(b, "k")[done[b]: done[b] + hist[b]] for b in range(B)]
    vrows = [rows_of(b, "v")[done[b]: done[b] + hist[b]] for b in range(B)]
    write(oslots, np.concatenate(krows, axis=0), np.concatenate(vrows, axis=0), opairs)
    done = done + hist
    # 3. decode step: one new token per non-empty sequence
    step = (lens > 0).astype(np.int64)
    cslots, cpairs = palloc.reserve_batch(tables, nblk, done, step)
    dslots, dpairs = oa.reserve_batch(orows, done, step)
    assert cslots.tolist() == dslots
    assert [tuple(p) for p in cpairs.tolist()] == [tuple(p) for p in dpairs]
    kd = [rows_of(b, "k")[done[b]: done[b] + step[b]] for b in range(B)]
    vd = [rows_of(b, "v")[done[b]: done[b] + step[b]] for b in range(B)]
    write(dslots, np.concatenate(kd, axis=0), np.concatenate(vd, axis=0), dpairs)
    # the decode step's rows, one per sequence (zeros where length is 0)
    sd_in = workloads.storage_np_dtype(dt)
    dec_k = np.zeros((B, h, d), dtype=sd_in)
    dec_v = np.zeros((B, h, d), dtype=sd_in)
    for b in range(B):
        if step[b]:
            dec_k[b], dec_v[b] = kd[b][0], vd[b][0]
    for b in range(B):
        assert tables[b, : nblk[b]].tolist() == orows[b]

    c = Case()
    c.wl, c.vals, c.palloc, c.oalloc = wl, vals, palloc, oa
    c.tables_np, c.nblk, c.orows = tables, nblk, orows
    c.k_cache, c.v_cache, c.ok_pool, c.ov_pool = kc, vc, okp, ovp
    c.kv = kv
    c.dec_k, c.dec_v = dec_k, dec_v
    if quant:
        c.k_scales, c.v_scales, c.ok_scales, c.ov_scales = ks, vs, oks, ovs
    c.cow_pairs = [tuple(p) for p in opairs] + [tuple(p) for p in dpairs]
    c.device = device
    c.tables = torch.tensor(tables, device=device)
    c.lens = torch.tensor(lens.astype(np.int32), device=device)
    c.q = to_device(vals["q"], dt, device)
    c.out = torch.empty_like(c.q)
    if check_pools:
        if quant:
            assert np.array_equal(kc.cpu().numpy(), okp), "K codes differ from the oracle"
            assert np.array_equal(vc.cpu().numpy(), ovp), "V codes differ from the oracle"
            assert np.array_equal(to_bits(ks), storage_bits(oks)), "K scales differ from the oracle"
            assert np.array_equal(to_bits(vs), storage_bits(ovs)), "V scales differ from the oracle"
        else:
            assert np.array_equal(to_bits(kc), storage_bits(okp)), "K pool differs from the oracle"
            assert np.array_equal(to_bits(vc), storage_bits(ovp)), "V pool differs from the oracle"
    return c


def oracle_out(c: Case, heads=None) -> np.ndarray:
    wl = c.wl
    if c.kv != "dense":
        return oquant.decode_attention(c.vals["q"], c.ok_pool, c.ov_pool, c.ok_scales, c.ov_scales, c.tables_np,
                                       wl.seq_lens, wl.dtype, c.kv, wl.scale, heads=heads)
    return oatt.decode_attention(c.vals["q"], c.ok_pool, c.ov_pool, c.tables_np, wl.seq_lens, wl.dtype, wl.scale,
                                 heads=heads)


def run_gpu(c: Case, work_groups=0, out=None):
    out = c.out if out is None else out
    if c.kv != "dense":
        pkv.pkv_attention_decode_quant(out, c.q, c.k_cache, c.v_cache, c.k_scales, c.v_scales, c.tables, c.lens,
                                       c.wl.max_seq_len, c.kv, scale=c.wl.scale, work_groups=work_groups)
        torch.cuda.synchronize()
        return out
    pkv.pkv_attention_decode(out, c.q, c.k_cache, c.v_cache, c.tables, c.lens, c.wl.max_seq_len, scale=c.wl.scale,
                             work_groups=work_groups)
    torch.cuda.synchronize()
    return out


def tolerance(dtype: str, ref: np.ndarray) -> np.ndarray:
    """Per-element bound: 1e-5 for fp32, 2e-3 for fp16 and for bf16 results
    below 0.5 in magnitude.  A bf16 result of magnitude 0.5 or more is allowed
    2e-3 plus its own rounding (half a unit in the last place of the stored
    value: 2^-9 at 0.5, 2^-8 at 1), which alone exceeds 2e-3 once |out| >= 1."""
    if dtype == "f32":
        return np.full(ref.shape, 1e-5)
    if dtype == "f16":
        return np.full(ref.shape, 2e-3)
    mag = np.maximum(np.abs(ref), 2.0 ** -126)
    half_ulp = 2.0 ** (np.floor(np.log2(mag)) - 8)
    return np.where(np.abs(ref) < 0.5, 2e-3, 2e-3 + half_ulp)


def compare(c: Case, got, ref=None, heads=None, record=None):
    """Element-wise check against the oracle; returns the largest |error|.
    ``record`` names the case in the run's table of largest errors."""
    ref = oracle_out(c, heads=heads) if ref is None else ref
    g = got.detach().float().cpu().numpy().astype(np.float64)
    if heads is not None:
        g, ref = g[:, heads], ref[:, heads]
    err = np.abs(g - ref)
    tol = tolerance(c.wl.dtype, ref)
    bad = ~(err <= tol)
    assert not bad.any(), (f"max err {np.nanmax(err):.3e} at {np.unravel_index(np.nanargmax(err), err.shape)}, "
                           f"{int(bad.sum())} elements over tolerance")
    worst = float(np.max(err)) if err.size else 0.0
    if record is not None:
        record_error(record, worst, c.wl.dtype, float(np.max(np.abs(ref))) if ref.size else 0.0)
    return worst


# Largest error per named case, written out at the end of the session (see
# tests/conftest.py) so that a quiet run still leaves the achieved margins.
ERRORS: dict = {}


def record_error(name: str, err: float, dtype: str, max_abs_out: float | None = None) -> None:
    prev = ERRORS.get(name)
    if prev is None or err > prev["max_abs_err"]:
        ERRORS[name] = {"max_abs_err": err, "dtype": dtype, "max_abs_out": max_abs_out}
