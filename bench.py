"""Decode-step benchmark for paged-KV attention on one MI355X.

One step = the whole decode path for one batch: host block reservation for
the new token of every sequence (C++ allocator), staging of slots, block
tables and lengths to the device, copy-on-write block copies (when any),
scatter of the new K/V rows (pkv_append) and decode attention over the paged
cache (pkv_attention_decode).  Inputs are resident in HBM before timing.

Default workload: one layer of a 7B-shaped model (32 heads x 128, fp16,
block 16, batch 32, lengths uniform on [128, 2048], blocks scattered through
a pool of 1.3x the blocks needed).  The sequences grow by one token per step.

Prints one JSON line.  ``value`` is KV GB/s over the whole timed step (K+V
bytes attention reads / step time); ``roofline`` reports the decode-attention
launch alone, timed with HIP events on its stream; ``cpu_baseline`` times the
oracle on a bounded sample of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
METRIC = "paged-attn decode KV GB/s and % of MI355X HBM peak; tokens-steps/sec"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--work-groups", type=int, default=0, help="decode work-groups (0 = library choice)")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the oracle timing sample")
    p.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    p.add_argument("--attention-only", type=int, default=0,
                   help="after the timed steps, launch decode attention N more times back to back")
    return p.parse_args()


def cpu_baseline(wl, lens_now, k_rows_fn, target_s):
    """Time the oracle on a sample of sequences of the same workload (host cores)."""
    from oracle import attention as oatt

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: the oracle is single threaded numpy
        cores = 1
    h, d, dt = wl.num_heads, wl.head_dim, wl.dtype
    order = np.random.default_rng(99).permutation(wl.batch)
    done_bytes, spent, used = 0, 0.0, []
    for b in order:
        L = int(lens_now[b])
        q, keys, vals = k_rows_fn(int(b), L)
        t0 = time.perf_counter()
        oatt.contiguous_attention(q[None], [keys], [vals], dt, wl.scale)
        spent += time.perf_counter() - t0
        done_bytes += L * 2 * h * d * wl.dtype_bytes
        used.append(int(b))
        if spent >= target_s:
            break
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"numpy float64 oracle over {len(used)} of {wl.batch} sequences of the same workload "
                      f"({sum(int(lens_now[b]) for b in used)} tokens x {h} heads), {spent:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported on this single-GPU build "
              f"(sharding is described in the design notes)", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_attention_amd as pkv
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.llama7b_layer()
    B, H, D, bs = wl.batch, wl.num_heads, wl.head_dim, wl.block_size
    dt = torch.float16
    esz = 2
    total_steps = args.warmup + args.steps
    hist = wl.seq_lens.astype(np.int64) - 1            # tokens already cached before the first step
    max_len = int(wl.seq_lens.max()) + total_steps
    maxb = -(-max_len // bs)
    print(f"[bench] workload: {wl.title}; steps {args.steps} warmup {args.warmup}", file=sys.stderr, flush=True)

    # --- set-up (not timed): allocator, pools, history prefill ------------
    alloc = pkv.BlockAllocator(wl.num_blocks, bs, wl.free_order)
    tables = np.zeros((B, maxb), dtype=np.int32)
    nblk = np.zeros(B, dtype=np.int32)
    slots, pairs = alloc.reserve_batch(tables, nblk, np.zeros(B, dtype=np.int32), hist)
    k_cache = torch.full((wl.num_blocks, bs, H, D), float("nan"), dtype=dt, device=dev)
    v_cache = torch.full_like(k_cache, float("nan"))
    gen = torch.Generator(device=dev).manual_seed(2024)
    n_hist = int(hist.sum())
    k_hist = torch.randn((n_hist, H, D), generator=gen, device=dev, dtype=torch.float32).to(dt)
    v_hist = torch.randn((n_hist, H, D), generator=gen, device=dev, dtype=torch.float32).to(dt)
    pkv.pkv_append(k_hist, v_hist, torch.from_numpy(slots).to(dev), k_cache, v_cache)
    # per-step inputs, resident in HBM before timing
    q_all = torch.randn((total_steps, B, H, D), generator=gen, device=dev, dtype=torch.float32).to(dt)
    k_new = torch.randn((total_steps, B, H, D), generator=gen, device=dev, dtype=torch.float32).to(dt)
    v_new = torch.randn((total_steps, B, H, D), generator=gen, device=dev, dtype=torch.float32).to(dt)
    out = torch.empty((B, H, D), dtype=dt, device=dev)
    wgs = args.work_groups or pkv.pkv_decode_work_groups()
    workspace = pkv.decode_workspace(B, H, D, "f16", wgs, device=dev)
    # device metadata (double-buffered) and pinned host staging (ring)
    ring = 4
    d_tables = [torch.empty((B, maxb), dtype=torch.int32, device=dev) for _ in range(2)]
    d_lens = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(2)]
    d_slots = [torch.empty(B, dtype=torch.int64, device=dev) for _ in range(2)]
    d_pairs = torch.empty((B, 2), dtype=torch.int32, device=dev)
    h_tables = [torch.empty((B, maxb), dtype=torch.int32, pin_memory=True) for _ in range(ring)]
    h_lens = [torch.empty(B, dtype=torch.int32, pin_memory=True) for _ in range(ring)]
    h_slots = [torch.empty(B, dtype=torch.int64, pin_memory=True) for _ in range(ring)]
    h_pairs = [torch.empty((B, 2), dtype=torch.int32, pin_memory=True) for _ in range(ring)]
    h_done = [None] * ring
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    cur = hist.astype(np.int32).copy()
    ones = np.ones(B, dtype=np.int32)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(total_steps)]
    kv_bytes = []
    table_entries = []

    def step(i):
        r, d = i % ring, i % 2
        if h_done[r] is not None:
            h_done[r].synchronize()          # host buffer free again (its copy has run)
        sl, pr = alloc.reserve_batch(tables, nblk, cur, ones)   # a1: host reservation
        cur[:] += 1
        h_tables[r].numpy()[:] = tables
        h_lens[r].numpy()[:] = cur
        h_slots[r].numpy()[:] = sl
        d_tables[d].copy_(h_tables[r], non_blocking=True)           # a2: stage metadata
        d_lens[d].copy_(h_lens[r], non_blocking=True)
        d_slots[d].copy_(h_slots[r], non_blocking=True)
        if len(pr):                                                 # a3: copy-on-write
            h_pairs[r].numpy()[: len(pr)] = pr
            d_pairs[: len(pr)].copy_(h_pairs[r][: len(pr)], non_blocking=True)
            pkv.pkv_copy_blocks([k_cache], [v_cache], d_pairs[: len(pr)])
        e = torch.cuda.Event()
        e.record(stream)
        h_done[r] = e
        pkv.pkv_append(k_new[i], v_new[i], d_slots[d], k_cache, v_cache)   # a4: scatter
        ev[i][0].record(stream)
        pkv.pkv_attention_decode(out, q_all[i], k_cache, v_cache, d_tables[d], d_lens[d], max_len,   # a5, a6
                                 scale=wl.scale, work_groups=wgs, workspace=workspace)
        ev[i][1].record(stream)
        kv_bytes.append(int(cur.astype(np.int64).sum()) * 2 * H * D * esz)
        table_entries.append(int(((cur.astype(np.int64) + bs - 1) // bs).sum()))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    kv_bytes.clear()
    table_entries.clear()
    t0 = time.perf_counter()
    for i in range(args.warmup, total_steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    lens_end = cur.copy()
    attn_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.warmup, total_steps)]
    attn_avg_s = float(np.mean(attn_ms)) / 1e3
    kv_total = float(sum(kv_bytes))
    value = kv_total / elapsed / 1e9
    # algorithmic bytes of one decode-attention launch (average over the timed steps):
    # K+V rows + q in + out + block-table entries + lengths
    mean_len_sum = float(np.mean(kv_bytes)) / (2 * H * D * esz)
    algo = float(np.mean(kv_bytes)) + 2 * B * H * D * esz + 4 * float(np.mean(table_entries)) + 4 * B
    achieved = algo / attn_avg_s / 1e9

    extra = {}
    if args.attention_only:
        # Back-to-back launches of the dominant kernel alone (profiling aid).
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(args.attention_only):
            pkv.pkv_attention_decode(out, q_all[-1], k_cache, v_cache, d_tables[(total_steps - 1) % 2],
                                     d_lens[(total_steps - 1) % 2], max_len, scale=wl.scale, work_groups=wgs,
                                     workspace=workspace)
        s1.record(stream)
        torch.cuda.synchronize()
        extra["attention_only_avg_us"] = round(s0.elapsed_time(s1) * 1e3 / args.attention_only, 2)
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        bcopy = torch.empty_like(a)
        bcopy.copy_(a)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = 1 << 30

    cpu = None
    if not args.no_cpu:
        k_cpu, v_cpu = None, None

        def rows(b, L):
            # The same logical rows the GPU attends: history rows then this
            # run's appended rows, all drawn by torch's generator above.
            start = int(hist[:b].sum())
            kh = k_hist[start: start + int(hist[b])]
            vh = v_hist[start: start + int(hist[b])]
            kk = torch.cat([kh, k_new[:total_steps, b]], 0)[:L].cpu().numpy()
            vv = torch.cat([vh, v_new[:total_steps, b]], 0)[:L].cpu().numpy()
            return q_all[total_steps - 1, b].cpu().numpy(), kk, vv

        cpu = cpu_baseline(wl, lens_end, rows, args.cpu_seconds)

    ms_per_step = elapsed / args.steps * 1e3
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; K/V/Q ~ N(0,1) in fp16)",
        "config": {"workload": wl.title, "batch": B, "heads": H, "head_dim": D, "block_size": bs,
                   "pool_blocks": wl.num_blocks, "work_groups": wgs,
                   "mean_seq_len": round(mean_len_sum / B, 1)},
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "token_steps_per_s": round(B * args.steps / elapsed, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "pkv_attention_decode", "avg_launch_us": round(attn_avg_s * 1e6, 2),
                     "algorithmic_bytes_per_launch": int(algo)},
        "cpu_baseline": cpu,
    }
    rec.update(extra)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
