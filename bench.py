"""Decode-step benchmark for paged-KV attention on one MI355X.

One step = the whole decode path for one batch:
  1. host block reservation for every sequence's new token (C++ allocator),
  2. hand-over of slots, block tables and lengths: the kernels read them in
     place from pinned host memory, with no copy on the queue (``--metadata
     device`` stages them with one asynchronous copy per step instead),
  3. copy-on-write block copies (pkv_copy_blocks) when a reservation produced any,
  4. scatter of the new K/V rows and
  5. decode attention over the paged cache, 4 and 5 in one launch per layer
     (pkv_append_attention_decode; ``--separate``: pkv_append, then
     pkv_attention_decode),
with 4-5 repeated per layer.  Every layer has its own cache; the single-layer
workloads read the caches of 4 layers in turn by default, so that no call
finds the previous call's rows in the 256 MB Infinity Cache (a model's next
decode of a layer comes 31 layers later).  Inputs are resident in HBM before
timing; sequences grow by one token per step.

Default workload: one layer of a 7B-shaped model (32 heads x 128, fp16, block
16, batch 32, lengths uniform on [128, 2048], blocks scattered through a pool
of 1.3x the blocks needed).  ``--workload full7b_step`` runs the 32-layer step
(batch 256, lognormal lengths, 30 % sharing a 256-token prefix, pool = 85 % of
free HBM); ``--workload long13b`` the 40-head bf16 4096-token case;
``--workload tiny`` the 4-sequence fp32 case (launch-bound).

``--kv-dtype i8|fp8`` stores K/V as 8-bit codes plus one float32 scale per
(token, head); queries and outputs stay in the workload's dtype.

Prints one JSON line.  ``value`` is KV GB/s over the whole timed step (K+V
bytes attention reads / step time).  ``roofline`` reports the decode-attention
call (decode kernel + merge kernel), each call of a separate pass timed with
HIP events that the call itself records at its first kernel's start and its
last kernel's end (pkv_time_next_decode), and the HBM traffic rocprofv3
counted for the same call, as its ratio to the algorithmic bytes, when the
recorded counters belong to the current kernel source.  ``cpu_baseline``
times the oracle on a bounded sample of the same workload on the host cores.
``host_side`` carries the host figures of the path: allocator ns per block,
reservation us per step, fragmentation, the Tiny call's us and the host CPU.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
# Host-to-device staging copies through the runtime's blit kernels on the
# compute queue: the copy engine path makes every step's kernels wait on a
# cross-engine signal (measured 20-45 us per step on MI355X).
os.environ.setdefault("HSA_ENABLE_SDMA", "0")

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
METRIC = "paged-attn decode KV GB/s and % of MI355X HBM peak; tokens-steps/sec"
KERNEL_SOURCES = [os.path.join(ROOT, "paged_attention_amd", "csrc", f)
                  for f in ("decode_common.h", "prefix_common.h", "kernels.hip", "kernels_q8.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="llama7b_layer",
                   choices=["tiny", "llama7b_layer", "prefix_cow", "long13b", "full7b_step"])
    p.add_argument("--component", default="decode", choices=["decode", "prefix_cache", "swap", "allocator"],
                   help="decode: the decode step (default, the headline line); prefix_cache: host prefix-cache "
                        "operations on a shared-system-prompt request stream; swap: preemption swap of a "
                        "request's blocks to pinned host memory and back; allocator: host block allocation and "
                        "release, ns per block")
    p.add_argument("--block-size", type=int, default=16, help="block size of the long13b workload")
    p.add_argument("--layers", type=int, default=0,
                   help="layers per step, each with its own cache read in turn (0 = the workload's default: 4 for "
                        "the single-layer 7B and prefix workloads, so that no call finds the previous call's rows "
                        "in the Infinity Cache; 1 for long13b and tiny; 32 for full7b_step)")
    p.add_argument("--work-groups", type=int, default=0,
                   help="decode chunk streams, i.e. work-groups for 16/32-bit caches and two per work-group for "
                        "8-bit ones where both fit (0 = library choice)")
    p.add_argument("--ring", type=int, default=4, help="host staging buffers (how many steps the host may run ahead)")
    p.add_argument("--metadata", choices=["pinned", "device", "staged"], default="pinned",
                   help="where kernels read step metadata: pinned host memory in place, a device copy on the "
                        "compute stream, or a device copy per ring slot made on a second stream")
    p.add_argument("--kv-dtype", choices=["auto", "i8", "fp8"], default="auto",
                   help="K/V cache storage: the workload's dtype (auto) or an 8-bit format")
    p.add_argument("--scores", action="store_true",
                   help="also update cumulative attention scores per cached token (16/32-bit caches; two launches "
                        "per layer)")
    p.add_argument("--grouped", action="store_true",
                   help="decode with pkv_append_attention_decode_grouped[_quant] (with --separate: "
                        "pkv_attention_decode_grouped[_quant] after pkv_append): shared prefixes read once per tile "
                        "of sequences (prefix, decode and merge kernels)")
    p.add_argument("--separate", action="store_true",
                   help="scatter and attend in two launches per layer (pkv_append, pkv_attention_decode) instead "
                        "of one (pkv_append_attention_decode)")
    p.add_argument("--timed-calls", type=int, default=64,
                   help="decode calls timed one by one, in a pass after the wall-clock steps (at least 50)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle timing sample")
    p.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    p.add_argument("--no-host-side", action="store_true", help="skip the host_side figures")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    return p.parse_args()


def source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(key: str):
    """(counted / algorithmic bytes) of one decode-attention call from committed
    rocprofv3 counters of the same call, if they belong to the current kernel
    sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(key)
    if not entry or entry.get("kernel_source_sha256_16") != source_hash():
        return None
    counted, algo = entry.get("counted_bytes_per_call"), entry.get("algorithmic_bytes_per_call")
    if not counted or not algo:
        return None
    return counted / algo


def host_info() -> dict:
    """The host CPU as lscpu reports it, and the CPUs this process may use."""
    info = {"logical_cpus": os.cpu_count()}
    try:
        info["usable_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    try:
        import subprocess

        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        fields = dict(line.split(":", 1) for line in out.splitlines() if ":" in line)
        for key, name in (("Model name", "cpu_model"), ("Socket(s)", "sockets"),
                          ("Core(s) per socket", "cores_per_socket"), ("Thread(s) per core", "threads_per_core")):
            if key in fields:
                v = fields[key].strip()
                info[name] = int(v) if v.isdigit() else v
    except (OSError, ValueError):
        pass
    if "cpu_model" not in info:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        info["cpu_model"] = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    return info


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # no threadpoolctl: numpy's BLAS threads unknown, report one
        return 1


def cpu_baseline(wl, sample_rows, target_s, kv):
    """Time the oracle on sequences of the same workload until ~target_s of work."""
    from oracle import attention as oatt
    from oracle import quant as oquant

    cores = blas_threads()
    h, d = wl.num_heads, wl.head_dim
    order = np.random.default_rng(99).permutation(wl.batch)
    done_bytes, spent, seqs, tokens = 0, 0.0, 0, 0
    i = 0
    while spent < target_s and i < 100 * wl.batch:
        b = int(order[i % wl.batch])
        i += 1
        rows = sample_rows(b)
        L = rows[1].shape[0]
        t0 = time.perf_counter()
        if kv == "dense":
            q, keys, vals = rows
            oatt.contiguous_attention(q[None], [keys], [vals], wl.dtype, wl.scale)
            done_bytes += L * 2 * h * d * wl.dtype_bytes
        else:
            # The sequence's rows as a pool of one-token blocks, read through
            # an identity table.
            q, kc, ks, vc, vs = rows
            oquant.decode_attention(q[None], kc[:, None], vc[:, None], ks[:, :, None], vs[:, :, None],
                                    np.arange(L, dtype=np.int64)[None], [L], wl.dtype, kv, wl.scale)
            done_bytes += L * 2 * h * (d + 4)
        spent += time.perf_counter() - t0
        seqs += 1
        tokens += L
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"numpy float64 oracle, {seqs} sequence decodes of this workload ({tokens} tokens x {h} heads, "
                      f"one layer), {spent:.1f} s of oracle time",
            "host": host_info()}


# The pages' allocation latencies (context, not targets: other systems,
# hardware unstated).
PAGE_ALLOC_FIGURES = [
    "fixed-size page pool: 0.18 ms -> 0.003 ms per allocation once the free list replaces a scan "
    "(m.lqnn.cn/news/240480 §5.2 tip 1)",
    "variable-size pool: 15 ms -> 0.5 ms per allocation (l189.com/news/1438543 §2.3)",
]


def allocator_figures(n_blocks: int = 4096, seconds: float = 0.5) -> dict:
    """ns per block of one allocation plus one release: the library (a batch of
    n_blocks taken by pkv_blocks_alloc and returned by pkv_seq_release, so
    that the Python call costs nothing per block) and the oracle allocator
    (one Python call per block)."""
    import paged_attention_amd as pkv
    from oracle import allocator as oalloc

    order = np.random.default_rng(13).permutation(n_blocks).astype(np.int32)
    a = pkv.BlockAllocator(n_blocks, 16, order)
    ids = np.zeros(n_blocks, dtype=np.int32)
    reps, t0 = 0, time.perf_counter()
    while True:
        a.alloc_n(n_blocks, ids)
        a.release(ids)
        reps += 1
        el = time.perf_counter() - t0
        if el > seconds:
            break
    lib_ns = el / (reps * n_blocks) * 1e9
    o = oalloc.OracleAllocator(n_blocks, 16, order.tolist())
    oreps, t0 = 0, time.perf_counter()
    while True:
        got = [o.alloc() for _ in range(n_blocks)]
        for b in got:
            o.decref(b)
        oreps += 1
        oel = time.perf_counter() - t0
        if oel > seconds:
            break
    return {"library_ns_per_block": round(lib_ns, 2), "oracle_ns_per_block": round(oel / (oreps * n_blocks) * 1e9, 1),
            "what": f"one allocation + one release per block, pool of {n_blocks} blocks (library: batches of "
                    f"{n_blocks} through pkv_blocks_alloc / pkv_seq_release; oracle: Python calls)",
            "pages": PAGE_ALLOC_FIGURES}


def full7b_reservation(num_blocks: int, steps: int = 100) -> dict:
    """Host reservation of the full 7B step (256 sequences, one token each)
    after its history is in place, us per step; and its fragmentation."""
    import paged_attention_amd as pkv
    import workloads
    from oracle import sizes

    wl = workloads.full7b_step(num_blocks)
    B, bs = wl.batch, wl.block_size
    lens = wl.seq_lens.astype(np.int64)
    maxb = -(-(int(lens.max()) + steps) // bs) + 1
    alloc = pkv.BlockAllocator(wl.num_blocks, bs, wl.free_order)
    tables = np.zeros((B, maxb), dtype=np.int32)
    nblk = np.zeros(B, dtype=np.int32)
    done = np.zeros(B, dtype=np.int64)
    sharers = [int(x) for x in wl.sharers]
    s0 = sharers[0]
    alloc.reserve_batch(tables[s0:s0 + 1], nblk[s0:s0 + 1], [0], [wl.prefix_len])
    done[s0] = wl.prefix_len
    for x in sharers[1:]:
        row = alloc.fork(tables[s0, : nblk[s0]])
        tables[x, : len(row)] = row
        nblk[x] = len(row)
        done[x] = wl.prefix_len
    alloc.reserve_batch(tables, nblk, done, lens - 1 - done)
    cur = (lens - 1).astype(np.int32)
    ones = np.ones(B, dtype=np.int32)
    slots = np.zeros(B, dtype=np.int64)
    pairs = np.zeros((B, 2), dtype=np.int32)
    frag = sizes.fragmentation_tokens(lens, bs)
    t0 = time.perf_counter()
    for _ in range(steps):
        alloc.reserve_batch_into(tables, nblk, cur, ones, slots, pairs)
        cur += 1
    el = time.perf_counter() - t0
    return {"us_per_step": round(el / steps * 1e6, 2), "sequences": B, "pool_blocks": int(wl.num_blocks),
            "fragmentation_tokens": int(frag), "fragmentation_of_tokens": round(frag / int(lens.sum()), 5)}


def tiny_call_us(dev, calls: int = 200) -> dict:
    """The Tiny workload's decode call (4 sequences, 4 heads x 64, fp32): us
    per call from its kernel timestamps, and back to back on the stream."""
    import torch

    import paged_attention_amd as pkv
    import workloads

    wl = workloads.tiny()
    bs, H, D = wl.block_size, wl.num_heads, wl.head_dim
    vals = wl.draw_values()
    alloc = pkv.BlockAllocator(wl.num_blocks, bs, wl.free_order)
    tables = np.zeros((wl.batch, wl.max_blocks_per_seq()), dtype=np.int32)
    nblk = np.zeros(wl.batch, dtype=np.int32)
    lens = wl.seq_lens.astype(np.int32)
    slots, _ = alloc.reserve_batch(tables, nblk, np.zeros(wl.batch), lens)
    kc = torch.zeros((wl.num_blocks, bs, H, D), dtype=torch.float32, device=dev)
    vc = torch.zeros_like(kc)
    pkv.pkv_append(torch.from_numpy(np.concatenate(vals["k_seq"])).to(dev),
                   torch.from_numpy(np.concatenate(vals["v_seq"])).to(dev), torch.from_numpy(slots).to(dev), kc, vc)
    q = torch.from_numpy(vals["q"]).to(dev)
    out = torch.empty_like(q)
    call = pkv.PreparedDecode(out, q, kc, vc, torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev),
                              int(lens.max()), scale=wl.scale)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for e0, e1 in evs:
        e0.record(stream)
        e1.record(stream)
    for _ in range(20):
        call.launch()
    torch.cuda.synchronize()
    for e0, e1 in evs:
        pkv.pkv_time_next_decode(e0, e1)
        call.launch()
    torch.cuda.synchronize()
    kern = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
    t0 = time.perf_counter()
    for _ in range(calls):
        call.launch()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / calls * 1e6
    return {"call_us_p50": round(float(np.median(kern)), 2), "call_us_p10": round(float(np.percentile(kern, 10)), 2),
            "call_us_p90": round(float(np.percentile(kern, 90)), 2), "back_to_back_us_per_call": round(wall, 2),
            "workload": wl.title, "bound": "launch latency (no roofline claim)"}


def run_prefix_cache(args):
    """Host prefix-cache throughput: requests that share a 1500-token system
    prompt and add ~100 tokens of their own (the example of
    icman.com.cn/news/78786 §3.1), block 16.  One request = match its prompt,
    reserve the unmatched tail, record its full blocks, release it later (a
    sliding window of 64 live requests).  Reports requests/s of the C++
    cache and, beside it, of the oracle doing the same operations."""
    import paged_attention_amd as pkv
    from oracle import prefix_cache as opc

    bs, n_req, window, prompt_len = 16, 4000, 64, 1500
    rng = np.random.default_rng(11)
    prompt = rng.integers(0, 32000, prompt_len).astype(np.int32)
    reqs = [np.concatenate([prompt, rng.integers(0, 32000, int(rng.integers(50, 151))).astype(np.int32)])
            for _ in range(n_req)]
    num_blocks = (window + 2) * (-(-(prompt_len + 150) // bs)) * 2

    def drive(alloc, match, reserve, register, release, count):
        live, hit_blocks, need_blocks = [], 0, 0
        t0 = time.perf_counter()
        for i in range(count):
            toks = reqs[i]
            row = match(toks)
            hits = len(row)
            hit_blocks += hits
            need_blocks += len(toks) // bs
            row = reserve(row, hits * bs, len(toks) - hits * bs)
            register(toks, row, hits)
            live.append(row)
            if len(live) > window:
                release(live.pop(0))
        return time.perf_counter() - t0, hit_blocks, need_blocks

    a = pkv.BlockAllocator(num_blocks, bs)
    a.enable_prefix_cache()

    def lib_reserve(row, cur, n):
        a.reserve(row, cur, n)
        return row

    dt, hits, need = drive(a, lambda t: a.prefix_match(t, 1 << 20), lib_reserve,
                           lambda t, r, first: a.prefix_register(t, r, len(r), first), a.release, n_req)
    o = opc.OracleCachingAllocator(num_blocks, bs)

    def o_reserve(row, cur, n):
        o.reserve(row, cur, n)
        return row

    n_oracle = 400
    dto, _, _ = drive(o, lambda t: o.match(t, 1 << 20), o_reserve,
                      lambda t, r, first: o.register(t, r, len(r), first), lambda r: o.release(r, len(r)), n_oracle)
    prefill_saved = hits * bs / sum(len(r) for r in reqs)
    rec = {
        "metric": "prefix-cache host operations (match + reserve + register + release) per second",
        "value": round(n_req / dt, 1), "unit": "requests/s", "n_gpus": 0, "steps": n_req, "warmup": 0,
        "ms_per_step": round(dt / n_req * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32 token ids, SHA-256 keys", "data": "synthetic (seeded token ids)",
        "config": {"workload": f"{n_req} requests sharing a {prompt_len}-token system prompt plus U[50,150] own "
                               f"tokens, block {bs}, {window} live requests", "pool_blocks": num_blocks},
        "hit_blocks_per_request": round(hits / n_req, 2),
        "full_blocks_per_request": round(need / n_req, 2),
        "prefill_tokens_saved_frac": round(prefill_saved, 4),
        "us_per_request_block": round(dt / max(1, need) * 1e6, 3),
        "cpu_baseline": {"value": round(n_oracle / dto, 1), "unit": "requests/s", "cores": 1, "kind": "oracle",
                         "sample": f"the Python oracle (hashlib SHA-256) on the first {n_oracle} requests"},
    }
    print(json.dumps(rec), flush=True)


HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction (MI355X host interface)


def run_swap(args):
    """Preemption swap of one 2048-token request of the 7B shape (32 layers,
    K and V, fp16, block 16: 128 blocks x 64 pools of 128 KiB = 1 GiB) to
    pinned host memory and back with pkv_swap_blocks, timed with HIP events."""
    import torch

    import paged_attention_amd as pkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers, bs, H, D = 32, 16, 32, 128
    n_dev, n_host, n_swap = 512, 128, 128
    pools = [torch.randn((n_dev, bs, H, D), device=dev, dtype=torch.float32).half() for _ in range(2 * layers)]
    host = [torch.empty((n_host, bs, H, D), dtype=torch.float16).pin_memory() for _ in range(2 * layers)]
    rng = np.random.default_rng(5)
    dev_ids = rng.permutation(n_dev)[:n_swap].astype(np.int32)      # the request's scattered blocks
    host_ids = rng.permutation(n_host)[:n_swap].astype(np.int32)
    out_pairs = torch.from_numpy(np.stack([dev_ids, host_ids], 1).copy()).to(dev)
    in_ids = rng.permutation(n_dev)[:n_swap].astype(np.int32)       # swapped back in elsewhere
    in_pairs = torch.from_numpy(np.stack([host_ids, in_ids], 1).copy()).to(dev)
    nbytes = n_swap * len(pools) * bs * H * D * 2
    stream = torch.cuda.current_stream()
    times = {"out": [], "in": []}
    for it in range(args.warmup + args.steps):
        for name, dst, src, pr in (("out", host, pools, out_pairs), ("in", pools, host, in_pairs)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pkv.pkv_swap_blocks(dst, src, pr)
            e1.record(stream)
            e1.synchronize()
            if it >= args.warmup:
                times[name].append(e0.elapsed_time(e1) / 1e3)
    # the round trip is exact
    ok = all(torch.equal(pools[i][in_ids[j]], pools[i][dev_ids[j]]) for i in (0, 63) for j in (0, 77))
    # reference: one contiguous 1 GiB pinned <-> device copy through the runtime
    big_d = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    big_h = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    ref = {}
    for name, (dst, src) in (("out", (big_h, big_d)), ("in", (big_d, big_h))):
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src, non_blocking=True)
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        ref[name] = round(nbytes / min(ts) / 1e9, 2)
    # oracle on the host: the same block copies between numpy pools, bounded sample
    from oracle import pool as opool
    hp = [np.zeros((n_host, bs, H, D), dtype=np.float16) for _ in range(4)]
    dp = [pools[i].cpu().numpy() for i in range(4)]
    t0 = time.perf_counter()
    opool.swap_blocks(hp, dp, list(zip(dev_ids.tolist(), host_ids.tolist())))
    cpu_s = time.perf_counter() - t0
    cpu_bytes = n_swap * 4 * bs * H * D * 2
    gbs = {k: nbytes / float(np.median(v)) / 1e9 for k, v in times.items()}
    rec = {
        "metric": "preemption swap GB/s (device <-> pinned host, whole blocks)",
        "value": round(min(gbs.values()), 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(float(np.median(times["out"]) + np.median(times["in"])) * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (random K/V rows)",
        "config": {"workload": f"swap out and back in one request of {n_swap * bs} tokens, 7B shape: {layers} layers "
                               f"x K,V x {n_swap} blocks of {bs * H * D * 2 // 1024} KiB ({nbytes / 2**30:.2f} GiB "
                               "each way)", "round_trip_exact": bool(ok)},
        "swap_out_gbs": round(gbs["out"], 2), "swap_in_gbs": round(gbs["in"], 2),
        "runtime_copy_1gib_gbs": ref,
        "roofline": {"bound": "host-link", "achieved": round(min(gbs.values()), 2), "peak": HOST_LINK_PEAK_GBS,
                     "unit": "GB/s", "frac": round(min(gbs.values()) / HOST_LINK_PEAK_GBS, 4), "traffic": None,
                     "kernel": "swap_blocks_kernel"},
        "cpu_baseline": {"value": round(cpu_bytes / cpu_s / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                         "sample": f"oracle.pool.swap_blocks of the same {n_swap} blocks for 4 of the 64 pools "
                                   "(numpy host copies)"},
    }
    print(json.dumps(rec), flush=True)


def run_allocator(args):
    """Host block allocation and release, ns per block, beside the oracle's
    and the pages' figures (no GPU)."""
    fig = allocator_figures(seconds=2.0)
    rec = {
        "metric": "host block allocation + release, ns per block",
        "value": fig["library_ns_per_block"], "unit": "ns/block", "n_gpus": 0, "steps": 0, "warmup": 0,
        "ms_per_step": None, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32 block ids", "data": "synthetic (seeded free-list order)",
        "config": {"workload": fig["what"]},
        "cpu_baseline": {"value": fig["oracle_ns_per_block"], "unit": "ns/block", "cores": 1, "kind": "oracle",
                         "sample": "the oracle allocator (Python deque and list) on the same operations",
                         "host": host_info()},
        "pages": fig["pages"],
    }
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (how the path would shard "
              f"across GPUs is described in the design notes)", file=sys.stderr)
        sys.exit(2)
    if args.component == "prefix_cache":
        run_prefix_cache(args)
        return
    if args.component == "swap":
        run_swap(args)
        return
    if args.component == "allocator":
        run_allocator(args)
        return
    import torch

    import paged_attention_amd as pkv
    import workloads
    from oracle import sizes

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    full7b_blocks = None
    if args.workload == "tiny":
        wl = workloads.tiny()
    elif args.workload == "llama7b_layer":
        wl = workloads.llama7b_layer()
    elif args.workload == "long13b":
        wl = workloads.long13b(args.block_size)
    elif args.workload == "prefix_cow":
        wl = workloads.prefix_cow()
    if args.workload == "full7b_step" or not args.no_host_side:
        # 32 layers; the pool takes 85 % of the free device memory.
        free, _ = torch.cuda.mem_get_info()
        per_block = 32 * 2 * 16 * 32 * 128 * 2
        full7b_blocks = int(0.85 * free) // per_block
    if args.workload == "full7b_step":
        wl = workloads.full7b_step(full7b_blocks)
    layers = args.layers or {"llama7b_layer": 4, "prefix_cow": 4}.get(args.workload, wl.num_layers)
    if layers != wl.num_layers:
        wl = dataclasses.replace(wl, num_layers=layers,
                                 title=f"{wl.title}; the caches of {layers} layers read in turn")
    B, H, D, bs, NL = wl.batch, wl.num_heads, wl.head_dim, wl.block_size, wl.num_layers
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[wl.dtype]
    esz = wl.dtype_bytes
    kv = "dense" if args.kv_dtype == "auto" else args.kv_dtype
    if args.scores and kv != "dense":
        print("--scores runs with a 16/32-bit cache", file=sys.stderr)
        sys.exit(2)
    if args.grouped and (args.scores or wl.dtype not in ("f16", "bf16")):
        print("--grouped runs with fp16/bf16 queries and no scores", file=sys.stderr)
        sys.exit(2)
    fused = not (args.separate or args.scores)
    timed_steps = -(-max(50, args.timed_calls) // NL)
    total_steps = args.warmup + args.steps + timed_steps
    # K/V bytes one token adds to one layer's cache (codes and scales for 8-bit)
    tok_bytes = 2 * H * D * esz if kv == "dense" else 2 * H * (D + 4)
    lens0 = wl.seq_lens.astype(np.int64)
    max_len = int(lens0.max()) + total_steps
    maxb = -(-max_len // bs)
    print(f"[bench] {wl.title}; pool {wl.num_blocks} blocks; steps {args.steps} warmup {args.warmup} "
          f"+ {timed_steps} timed", file=sys.stderr, flush=True)

    # --- set-up (not timed): allocator, pools, history ---------------------
    alloc = pkv.BlockAllocator(wl.num_blocks, bs, wl.free_order)
    tables = np.zeros((B, maxb), dtype=np.int32)
    nblk = np.zeros(B, dtype=np.int32)
    done = np.zeros(B, dtype=np.int64)
    sharers = [int(s) for s in wl.sharers]
    history = []  # slots of each reservation, in order
    if sharers and wl.prefix_len:
        s0 = sharers[0]
        sl, _ = alloc.reserve_batch(tables[s0:s0 + 1], nblk[s0:s0 + 1], [0], [wl.prefix_len])
        history.append(sl)
        done[s0] = wl.prefix_len
        for s in sharers[1:]:
            row = alloc.fork(tables[s0, : nblk[s0]])
            tables[s, : len(row)] = row
            nblk[s] = len(row)
            done[s] = wl.prefix_len
    hist = np.maximum(lens0 - 1 - done, 0)
    sl, hist_pairs = alloc.reserve_batch(tables, nblk, done, hist)
    history.append(sl)
    cur = (done + hist).astype(np.int32)
    # A shared prefix that ends inside a block is copied for every sharer but
    # the last at its first private token: rows of the prefix are written,
    # then those blocks copied, then the private rows.
    n_first = len(history[0]) if len(history) > 1 else 0
    slots_hist = torch.from_numpy(np.concatenate(history)).to(dev)
    n_hist = slots_hist.numel()
    d_hist_pairs = torch.from_numpy(np.asarray(hist_pairs, dtype=np.int32).reshape(-1, 2)).to(dev)
    # Shared full blocks are read once per sharer (logical bytes) but need
    # leave HBM only once (unique bytes); sharing no longer changes once the
    # history is in place (new tokens land in private blocks).
    shared_extra_tokens = 0
    for blk_id in {int(x) for b in range(B) for x in tables[b, : nblk[b]]}:
        r = alloc.refcount(blk_id)
        if r > 1:
            shared_extra_tokens += (r - 1) * bs
    k_caches, v_caches, k_scales, v_scales = [], [], [], []
    gen = torch.Generator(device=dev)
    for layer in range(NL):
        kc = torch.empty((wl.num_blocks, bs, H, D), dtype=tdt if kv == "dense" else torch.uint8, device=dev)
        vc = torch.empty_like(kc)
        if kv != "dense":
            k_scales.append(torch.empty((wl.num_blocks, H, bs), dtype=torch.float32, device=dev))
            v_scales.append(torch.empty_like(k_scales[-1]))
        gen.manual_seed(5000 + layer)
        cuts = sorted({0, n_first, n_hist} | set(range(0, n_hist, 1 << 16)))
        for a0, a1 in zip(cuts[:-1], cuts[1:]):   # history rows drawn on the device, in slices
            if a0 == n_first and n_first > 0 and len(hist_pairs):
                pkv.pkv_copy_blocks([kc], [vc], d_hist_pairs)
                if kv != "dense":
                    pkv.pkv_copy_blocks([k_scales[-1]], [v_scales[-1]], d_hist_pairs)
            kr = torch.randn((a1 - a0, H, D), generator=gen, device=dev, dtype=torch.float32).to(tdt)
            vr = torch.randn((a1 - a0, H, D), generator=gen, device=dev, dtype=torch.float32).to(tdt)
            if kv == "dense":
                pkv.pkv_append(kr, vr, slots_hist[a0:a1], kc, vc)
            else:
                pkv.pkv_append_quant(kr, vr, slots_hist[a0:a1], kc, vc, k_scales[-1], v_scales[-1], kv)
        k_caches.append(kc)
        v_caches.append(vc)
    del slots_hist
    # Queries and new rows: a few steps' worth, used in turn (their values do
    # not change the work).
    nq = min(total_steps, 8)
    gen.manual_seed(7)
    q_all = torch.randn((nq, NL, B, H, D), generator=gen, device=dev, dtype=torch.float32).to(tdt)
    k_new = torch.randn((nq, NL, B, H, D), generator=gen, device=dev, dtype=torch.float32).to(tdt)
    v_new = torch.randn((nq, NL, B, H, D), generator=gen, device=dev, dtype=torch.float32).to(tdt)
    out = torch.empty((B, H, D), dtype=tdt, device=dev)
    wgs = args.work_groups or pkv.pkv_decode_work_groups(wl.dtype if kv == "dense" else kv)
    workspace = pkv.decode_workspace(B, H, D, wl.dtype if kv == "dense" else kv, wgs, device=dev)
    prefix = None
    if args.grouped:
        # Groups from the tables and the first step's lengths.  New tokens land
        # in private blocks, so the shared prefixes (capped by each length) stay
        # valid for every later step.
        spb, tiles = pkv.prefix_tiles(tables, (cur + 1).astype(np.int32), bs)
        prefix = (torch.from_numpy(spb).to(dev), torch.from_numpy(tiles).to(dev))
        workspace = torch.empty(pkv.pkv_decode_grouped_workspace_bytes(B, H, D, wl.dtype if kv == "dense" else kv,
                                                                       wgs), dtype=torch.uint8,
                                device=dev)
    # Step metadata is one packed buffer: slots (int64), lengths and block
    # tables (int32).  Host side: a ring of pinned buffers, so the host can
    # prepare step i+1 while step i's kernels still read (or copy) slot i.
    off_lens = 8 * B
    off_tab = off_lens + 4 * B
    nbytes = off_tab + 4 * B * maxb
    mode = args.metadata

    def split(buf):
        return (buf[:off_lens].view(torch.int64), buf[off_lens:off_tab].view(torch.int32),
                buf[off_tab:].view(torch.int32).view(B, maxb))

    ring = args.ring
    h_meta = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(ring)]
    h_views = []
    for hm in h_meta:
        raw = hm.numpy()
        h_views.append((raw[:off_lens].view(np.int64), raw[off_lens:off_tab].view(np.int32),
                        raw[off_tab:].view(np.int32).reshape(B, maxb)))
    h_pairs = [torch.empty((B, 2), dtype=torch.int32, pin_memory=True) for _ in range(ring)]
    d_pairs = torch.empty((B, 2), dtype=torch.int32, device=dev)
    h_done = [None] * ring
    stream = torch.cuda.current_stream()
    # Calls checked once; each step only swaps the per-step row pointers.  In
    # pinned mode every ring slot has its own set of calls pointing into it.
    copy_stream, d_slots = None, None
    if mode == "device":
        d_meta = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        metas = [split(d_meta)] * ring
    elif mode == "staged":
        # one device copy per ring slot, made on a second stream (default
        # priority) so that it runs beside the previous step's kernels
        d_meta = None
        d_slots = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(ring)]
        metas = [split(dm) for dm in d_slots]
        copy_stream = torch.cuda.Stream(device=dev)
        copied = [torch.cuda.Event() for _ in range(ring)]
        slot_read = [None] * ring          # event after the kernels that last read device slot r
    else:
        d_meta = None
        metas = [split(hm) for hm in h_meta]
    per_slot = {}
    score_bufs = []
    for r in range(ring):
        key = metas[r][0].data_ptr()
        if key not in per_slot:
            sl_t, ln_t, tb_t = metas[r]
            if fused:
                qk = {} if kv == "dense" else {"k_scales": None, "v_scales": None, "cache_dtype": kv}
                calls_l = []
                for l in range(NL):
                    if kv != "dense":
                        qk["k_scales"], qk["v_scales"] = k_scales[l], v_scales[l]
                    calls_l.append(pkv.PreparedAppendDecode(out, q_all[0, l], k_new[0, l], v_new[0, l], k_caches[l],
                                                            v_caches[l], tb_t, ln_t, max_len, scale=wl.scale,
                                                            work_groups=wgs, workspace=workspace, prefix=prefix,
                                                            **qk))
                per_slot[key] = (None, calls_l)
            elif kv == "dense" and args.scores:
                if not score_bufs:
                    score_bufs.extend([torch.zeros((B, max_len), dtype=torch.float32, device=dev) for _ in range(NL)])
                per_slot[key] = (
                    [pkv.PreparedAppend(k_new[0, l], v_new[0, l], sl_t, k_caches[l], v_caches[l])
                     for l in range(NL)],
                    [pkv.PreparedDecode(out, q_all[0, l], k_caches[l], v_caches[l], tb_t, ln_t, max_len,
                                        scale=wl.scale, work_groups=wgs, workspace=workspace,
                                        scores=score_bufs[l], decay=0.995) for l in range(NL)])
            elif kv == "dense":
                per_slot[key] = (
                    [pkv.PreparedAppend(k_new[0, l], v_new[0, l], sl_t, k_caches[l], v_caches[l])
                     for l in range(NL)],
                    [pkv.PreparedDecode(out, q_all[0, l], k_caches[l], v_caches[l], tb_t, ln_t, max_len,
                                        scale=wl.scale, work_groups=wgs, workspace=workspace, prefix=prefix)
                     for l in range(NL)])
            else:
                per_slot[key] = (
                    [pkv.PreparedAppendQuant(k_new[0, l], v_new[0, l], sl_t, k_caches[l], v_caches[l],
                                             k_scales[l], v_scales[l], kv) for l in range(NL)],
                    [pkv.PreparedDecodeQuant(out, q_all[0, l], k_caches[l], v_caches[l], k_scales[l], v_scales[l],
                                             tb_t, ln_t, max_len, kv, scale=wl.scale, work_groups=wgs,
                                             workspace=workspace, prefix=prefix) for l in range(NL)])
    calls = [per_slot[metas[r][0].data_ptr()] for r in range(ring)]
    torch.cuda.synchronize()

    ones = np.ones(B, dtype=np.int32)
    released = [torch.cuda.Event() for _ in range(ring)]
    kv_bytes, table_entries, n_pairs, host_s = [], [], [0], []

    def step(i, timing=None):
        r = i % ring
        j = i % nq
        if h_done[r] is not None:                                      # ring slot r free again:
            while not h_done[r].query():                               # poll; a blocking wait sleeps and
                pass                                                   # wakes up late
        slots_v, lens_v, tab_v = h_views[r]
        t_host = time.perf_counter()
        npairs = alloc.reserve_batch_into(tables, nblk, cur, ones, slots_v, h_pairs[r].numpy())  # 1. reserve
        cur[:] += 1
        lens_v[:] = cur
        tab_v[:] = tables
        host_s.append(time.perf_counter() - t_host)
        if d_meta is not None:
            d_meta.copy_(h_meta[r], non_blocking=True)                 # 2. stage metadata (one copy)
        if d_slots is not None:                                        # 2. stage on the copy stream
            if slot_read[r] is not None:
                copy_stream.wait_event(slot_read[r])
            with torch.cuda.stream(copy_stream):
                d_slots[r].copy_(h_meta[r], non_blocking=True)
            copied[r].record(copy_stream)
            stream.wait_event(copied[r])
        if npairs:                                                     # 3. copy-on-write
            d_pairs[:npairs].copy_(h_pairs[r][:npairs], non_blocking=True)
            pkv.pkv_copy_blocks(k_caches, v_caches, d_pairs[:npairs])
            if kv != "dense":
                pkv.pkv_copy_blocks(k_scales, v_scales, d_pairs[:npairs])
            n_pairs[0] += npairs
        if d_meta is not None:                                         # slot r is free once copied
            released[r].record(stream)
        appends, decodes = calls[r]
        for layer in range(NL):
            if fused:                                                  # 4 + 5 in one launch
                if timing is not None:
                    pkv.pkv_time_next_decode(*timing[layer])
                decodes[layer].launch(q_all[j, layer], k_new[j, layer], v_new[j, layer])
            else:
                appends[layer].launch(k_new[j, layer], v_new[j, layer])    # 4. scatter new rows
                if timing is not None:
                    pkv.pkv_time_next_decode(*timing[layer])
                decodes[layer].launch(q_all[j, layer])                     # 5. decode attention
        if d_meta is None:                                             # read (in place, or the device
            released[r].record(stream)                                 # slot) until here; the copy-on-
        if d_slots is not None:                                        # write pairs too
            slot_read[r] = released[r]
        h_done[r] = released[r]
        kv_bytes.append(int(cur.astype(np.int64).sum()) * tok_bytes * NL)
        table_entries.append(int(((cur.astype(np.int64) + bs - 1) // bs).sum()))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    kv_bytes.clear()
    table_entries.clear()
    host_s.clear()
    t0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kv_total = float(sum(kv_bytes))
    host_us = float(np.mean(host_s)) * 1e6
    frag_tokens = int(sizes.fragmentation_tokens(cur, bs))
    n_wall = len(kv_bytes)

    # A separate pass: every decode call timed by its own kernel timestamps
    # (timing a call costs its step queue time, so the wall-clock steps above
    # carry none).  Each event is recorded once first so that its HIP event
    # exists.
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(NL)]
          for _ in range(timed_steps)]
    for pairs in ev:
        for e0, e1 in pairs:
            e0.record(stream)
            e1.record(stream)
    torch.cuda.synchronize()
    first_timed = args.warmup + args.steps
    for k in range(timed_steps):
        step(first_timed + k, ev[k])
    torch.cuda.synchronize()
    call_us = np.array([e0.elapsed_time(e1) * 1e3 for pairs in ev for e0, e1 in pairs])
    attn_s = float(np.mean(call_us)) / 1e6
    call_pct = {f"p{q}": round(float(np.percentile(call_us, q)), 2) for q in (10, 50, 90)}

    value = kv_total / elapsed / 1e9
    unique_total = kv_total - shared_extra_tokens * tok_bytes * NL * n_wall
    unique_gbs = unique_total / elapsed / 1e9
    # Algorithmic bytes of one decode-attention call (mean over the timed
    # pass, one layer): K+V rows read (8-bit: codes and scales) + q in + out
    # + block-table entries + lengths.  With shared blocks only the unique
    # bytes must leave HBM (the rest are cache hits), so the roofline counts
    # unique K/V bytes.
    kv_per_call = float(np.mean(kv_bytes[n_wall:])) / NL
    unique_kv_per_call = kv_per_call - shared_extra_tokens * tok_bytes
    algo = unique_kv_per_call + 2 * B * H * D * esz + 4 * float(np.mean(table_entries[n_wall:])) + 4 * B
    if fused:   # the launch also reads the new rows and writes them (8-bit: codes and scales) into the pools
        algo += 2 * B * H * D * esz + B * tok_bytes
    achieved = algo / attn_s / 1e9
    # one record per distinct call (workload, format, launches, scores, grouping)
    key = (args.workload + (f"/bs{args.block_size}" if args.workload == "long13b" and args.block_size != 16 else "")
           + ("" if kv == "dense" else f"/{kv}") + ("/fused" if fused else "") + ("/scores" if args.scores else "")
           + ("/grouped" if prefix is not None else ""))
    ratio = recorded_traffic(key)
    traffic = None if ratio is None else int(round(ratio * algo))

    extra = {}
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        bcopy = torch.empty_like(a)
        bcopy.copy_(a)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = 1 << 30

    host_side = None
    if not args.no_host_side:
        host_side = {
            "reservation_us_per_step": {"this workload": round(host_us, 2),
                                        "full 7B step (256 sequences)": full7b_reservation(full7b_blocks)},
            "fragmentation_tokens": {"this workload": frag_tokens,
                                     "this workload, fraction of tokens": round(frag_tokens / int(cur.sum()), 5)},
            "allocator": allocator_figures(),
            "tiny_decode_call": tiny_call_us(dev),
            "host": host_info(),
        }

    cpu = None
    if not args.no_cpu:
        # The oracle reads the logical rows of layer 0 that the GPU attended to
        # in the last step, gathered from the pool by position.
        def rows(b):
            L = int(cur[b])
            idx = np.arange(L)
            blocks = tables[b, idx // bs].astype(np.int64)
            flat = torch.from_numpy(blocks * bs + idx % bs).to(dev)
            qq = q_all[(total_steps - 1) % nq, 0, b].cpu()
            if tdt == torch.bfloat16:
                qq = qq.view(torch.int16).numpy().view(np.uint16)
            else:
                qq = qq.numpy()
            if kv != "dense":
                fb, fp = flat // bs, flat % bs
                return (qq, k_caches[0].view(-1, H, D)[flat].cpu().numpy(), k_scales[0][fb, :, fp].cpu().numpy(),
                        v_caches[0].view(-1, H, D)[flat].cpu().numpy(), v_scales[0][fb, :, fp].cpu().numpy())
            kk = k_caches[0].view(-1, H, D)[flat].cpu()
            vv = v_caches[0].view(-1, H, D)[flat].cpu()
            if tdt == torch.bfloat16:
                return (qq,) + tuple(x.view(torch.int16).numpy().view(np.uint16) for x in (kk, vv))
            return qq, kk.numpy(), vv.numpy()

        cpu = cpu_baseline(wl, rows, args.cpu_seconds, kv)

    ms_per_step = elapsed / args.steps * 1e3
    call_name = (("pkv_append_attention_decode_grouped" if fused else "pkv_attention_decode_grouped")
                 + ("_quant" if kv != "dense" else "")
                 + (" (grouped_decode_kernel: decode ranges and prefix units in one launch + decode_merge_kernel)"
                    if kv == "dense" and wgs < torch.cuda.get_device_properties(0).multi_processor_count else
                    " (prefix_kernel + decode_kernel + decode_merge_kernel)")
                 if prefix is not None else
                 "pkv_attention_decode_scores (decode_kernel + merge_score_kernel)" if args.scores else
                 ("pkv_append_attention_decode" if fused else "pkv_attention_decode")
                 + ("_quant" if kv != "dense" else "") + " (decode_kernel + decode_merge_kernel)")
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
        "dtype": wl.dtype if kv == "dense" else {"i8": "i8", "fp8": "fp8_e4m3"}[kv],
        "data": "synthetic (seeded; Q/K/V ~ N(0,1) cast to the storage dtype)",
        "config": {"workload": wl.title + ("" if kv == "dense" else f"; K/V cache {kv} + f32 scale per (token, head)"),
                   "kv_cache": wl.dtype if kv == "dense" else kv, "q_dtype": wl.dtype, "layers": NL, "batch": B,
                   "heads": H, "head_dim": D, "block_size": bs, "pool_blocks": wl.num_blocks, "work_groups": wgs,
                   "metadata": mode, "launches_per_layer": 1 if fused else 2,
                   "cumulative_scores": bool(args.scores),
                   "grouped_prefix_tiles": None if prefix is None else int(prefix[1].shape[0]),
                   "mean_seq_len": round(float(np.mean(kv_bytes[:n_wall])) / NL / tok_bytes / B, 1),
                   "cow_pairs": n_pairs[0]},
        "hbm_peak_frac": round(unique_gbs / HBM_PEAK_GBS, 4),
        "unique_kv_gbs": round(unique_gbs, 2),
        "token_steps_per_s": round(B * args.steps / elapsed, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_ratio": None if ratio is None else round(ratio, 4),
                     "kernel": call_name,
                     "avg_call_us": round(attn_s * 1e6, 2), "call_us_percentiles": call_pct,
                     "algorithmic_bytes_per_call": int(algo),
                     "logical_kv_bytes_per_call": int(kv_per_call), "timed_calls": int(call_us.size),
                     "timing": f"kernel timestamps of each call's first and last kernel, {call_us.size} calls "
                               f"({timed_steps} steps x {NL} layers) in a pass after the wall-clock steps",
                     "traffic_source": "rocprofv3 FETCH_SIZE + WRITE_SIZE of the same call, as a ratio to its "
                                       "algorithmic bytes (profiles/decode_traffic.json), times this run's "
                                       "algorithmic bytes"},
        "host_side": host_side,
        "cpu_baseline": cpu,
    }
    rec.update(extra)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
