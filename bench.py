#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV-cache hot path on one MI355X.

One step = the whole hot path over one batch: host bookkeeping (slot and
copy-on-write reservation in the block manager) staged to the GPU with
pkv_bm_stage_step (one kernel reads the step's record from pinned memory
and updates the device-resident block tables, lengths, slots and copy
pairs), the copy-on-write block copy (when any), then the cache append of
one token per sequence and decode attention with its log-sum-exp merge in
one call (paged_attention_decode_append; ``--separate-append`` runs them as
two calls).  Consecutive steps are real decode
steps: every sequence grows by one token per step, new blocks are taken at
block boundaries.

Default workload: the Llama-3-70B-shaped decode layer at 32k context
(16 sequences x 32768 tokens, 64 query / 8 kv heads, head_dim 128, bf16,
block 16, 40k-block pool, blocks scattered by a seeded permutation).  All
inputs are synthetic and resident in HBM before the timed region.

Prints one JSON line: ``value`` = whole-job KV throughput (algorithmic K/V
bytes of valid tokens / wall time per step), plus tokens/s, the roofline of
the decode call measured with HIP events on its stream, and the CPU oracle
timed on the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attention KV GB/s (% of HBM peak) and tokens/s, 70B-shaped layer @32k"
PREFILL_METRIC = "chunked-prefill attention TFLOP/s (causal, 70B-shaped layer)"
SWAP_METRIC = "swap to pinned host memory and back, GB/s per direction (70B-shaped 32k sequences)"
MULTITURN_METRIC = "multi-turn prompt tokens reused from cache (radix index), fraction"
HOST_LINK_PEAK = 64.0e9  # PCIe 5.0 x16, one direction, bytes/s
HBM_PEAK = 8.0e12  # MI355X HBM3E, bytes/s
MFMA_BF16_PEAK = 2.5e15  # MI355X dense bf16 matrix-core flop/s
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_cache_230_amd", "csrc", "pagedkv_kernels.hip")
DEFAULT_STEPS = {"c3_70b_32k_bf16": (200, 20), "c2_8b_bf16": (200, 20)}  # (timed, warm-up); others (30, 5)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
PREFILL_SOURCE = os.path.join(ROOT, "paged_kv_cache_230_amd", "csrc", "prefill_kernel.hip")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_c7_traffic.json")


# ------------------------------------------------------------- accounting
def decode_algorithmic_bytes(lens, num_q_heads, num_kv_heads, head_dim, block_size, elem_bytes):
    """Bytes a decode call must move at minimum: K/V of valid tokens (each
    read once, shared by the G query heads of its kv head), q and out, the
    used block-table entries and the lengths."""
    kv = sum(int(L) for L in lens) * num_kv_heads * head_dim * 2 * elem_bytes
    qo = 2 * len(lens) * num_q_heads * head_dim * elem_bytes
    tables = 4 * sum(-(-int(L) // block_size) for L in lens)
    return kv + qo + tables + 4 * len(lens)


def append_algorithmic_bytes(lens, num_kv_heads, head_dim, elem_bytes):
    """Bytes of the one-token append of a decode step: each non-empty
    sequence's new K and V rows read once and written once."""
    return sum(1 for L in lens if int(L) > 0) * num_kv_heads * head_dim * 2 * 2 * elem_bytes


def decode_kv_bytes(lens, num_kv_heads, head_dim, elem_bytes):
    return sum(int(L) for L in lens) * num_kv_heads * head_dim * 2 * elem_bytes


def decode_flops(lens, num_q_heads, head_dim):
    return sum(4 * num_q_heads * head_dim * int(L) for L in lens)


def prefill_flops(lens, chunks, num_q_heads, head_dim):
    """Causal work of one prefill call: the token at position p attends to
    p + 1 keys, 4 * H_q * d flops per key (Q K^T and P V, multiply + add)."""
    f = 0
    for L, C in zip(lens, chunks):
        L, C = int(L), int(C)
        keys = C * (L - C) + C * (C + 1) // 2  # sum over p = L-C .. L-1 of (p + 1)
        f += 4 * num_q_heads * head_dim * keys
    return f


def kernel_source_sha(path=KERNEL_SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic(workload, partition):
    """HBM bytes per decode call from committed counter runs, if they were
    taken on this workload, in the default launch, on the current kernel
    source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get("workloads", {}).get(workload)
    if t.get("kernel_source_sha256") != kernel_source_sha() or rec is None or partition != 0:
        return None
    return rec.get("hbm_bytes_per_decode_call")


def load_prefill_traffic(workload, steps, warmup):
    """Mean HBM bytes per timed prefill call from committed counter runs, if
    they were taken on this workload with the same steps (the contexts grow
    from step to step) on the current kernel source; else None."""
    try:
        with open(PREFILL_TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("kernel_source_sha256") != kernel_source_sha(PREFILL_SOURCE) or t.get("workload") != workload
            or t.get("steps") != steps or t.get("warmup") != warmup):
        return None
    return t.get("hbm_bytes_per_timed_call_mean")


def calibration_copy(dev):
    """One plain 1 GiB device copy, whose counters calibrate FETCH_SIZE and
    WRITE_SIZE (1,073,741,824 bytes read and written)."""
    import torch

    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def measured_read_peak(dev, nbytes=4 << 30, reps=6):
    """HBM read rate of the library's plain streaming probe (pkv_stream_read)
    over a buffer larger than every cache, timed with HIP events on the
    current stream: (best, median) in bytes/s over ``reps`` reads after one
    untimed read."""
    import torch

    import paged_kv_cache_230_amd as pkv

    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)  # workgroups
    pkv.stream_read(buf, sink)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for r in range(reps):
        pkv.stream_read(buf, sink)
        ev[r + 1].record()
    torch.cuda.synchronize()
    rates = sorted(nbytes / (ev[r].elapsed_time(ev[r + 1]) / 1e3) for r in range(reps))
    del buf, sink
    torch.cuda.empty_cache()
    return rates[-1], rates[len(rates) // 2]


def decode_tile_ids(tables, lens, block_size, num_kv_heads):
    """The (block, kv head) tiles a decode call reads, as tile indices
    block * num_kv_heads + head into a pool laid out [block][kv head][tile],
    in the kernel's visiting order: head by head, each head's sequences in
    order, each sequence's blocks in logical order.  Empty sequences read
    nothing."""
    import numpy as np

    nb = -(-np.asarray(lens, dtype=np.int64) // block_size)
    parts = [np.asarray(tables[s, :nb[s]], dtype=np.int64) for s in range(len(nb))]
    blocks = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    return np.concatenate([blocks * num_kv_heads + g for g in range(num_kv_heads)]).astype(np.int32)


def measured_tile_read(dev, cache, tables, lens, block_size, reps=6):
    """Rate at which the library's tile probe (pkv_tile_read) streams the
    very (block, kv head) tiles of K and V that a decode call over
    ``tables``/``lens`` reads, head by head and sequence by sequence, with
    no arithmetic: (best, median) in bytes/s over ``reps`` reads after one
    untimed read, timed with HIP events on the current stream."""
    import torch

    import paged_kv_cache_230_amd as pkv

    ids = decode_tile_ids(tables, lens, block_size, cache.k_cache.shape[1])
    tile = cache.k_cache[0, 0].numel() * cache.k_cache.element_size()
    ids_d = torch.from_numpy(ids).to(dev)
    sink = torch.empty(16384, dtype=torch.int32, device=dev)

    def read():
        pkv.tile_read(cache.k_cache, tile, ids_d, sink)
        pkv.tile_read(cache.v_cache, tile, ids_d, sink)

    read()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for r in range(reps):
        read()
        ev[r + 1].record()
    torch.cuda.synchronize()
    nbytes = 2 * ids.size * tile
    rates = sorted(nbytes / (ev[r].elapsed_time(ev[r + 1]) / 1e3) for r in range(reps))
    del ids_d, sink
    return rates[-1], rates[len(rates) // 2]


def measured_mfma_peak(dev, workgroups=2048, iters=4096, reps=5):
    """bf16 matrix-core rate of the library's probe (pkv_mfma_rate: every
    wave issues 32x32x16 products into independent register accumulators),
    timed with HIP events on the current stream: (best, median) in flop/s
    over ``reps`` runs of about 20 ms after one untimed run.  The GPU lowers
    its clock under this load, so the rate sits below the nominal peak."""
    import torch

    import paged_kv_cache_230_amd as pkv

    sink = torch.empty(workgroups * 512, dtype=torch.float32, device=dev)
    pkv.mfma_rate(sink, workgroups, iters)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    flops = 0
    for r in range(reps):
        flops = pkv.mfma_rate(sink, workgroups, iters)
        ev[r + 1].record()
    torch.cuda.synchronize()
    rates = sorted(flops / (ev[r].elapsed_time(ev[r + 1]) / 1e3) for r in range(reps))
    del sink
    return rates[-1], rates[len(rates) // 2]


def percentiles(xs, ps=(10, 50, 90)):
    """Nearest-rank percentiles of a list."""
    ys = sorted(xs)
    return {f"p{p}": ys[min(len(ys) - 1, max(0, math.ceil(p / 100 * len(ys)) - 1))] for p in ps}


def prefix_cache_report(w):
    """Host cost and effect of the prefix cache on a workload of cached
    admissions: the admissions replayed on a fresh block manager (host only,
    timed), hit counts, and blocks in use against private copies."""
    import numpy as np

    import paged_kv_cache_230_amd as pkv

    bs = w.config.block_size
    bm = pkv.BlockManager(w.num_blocks, bs, w.free_order)
    n_req = prompt_tokens = cached = 0
    t_admit = 0.0
    for op in w.setup_ops:
        if op[0] == "admit":
            _, sid, tokens, _, salt = op
            t0 = time.perf_counter()
            n = bm.add_seq_cached(sid, tokens, salt)
            bm.append_slots([sid], [len(tokens) - n], token_ids=tokens[n:])
            t_admit += time.perf_counter() - t0
            n_req += 1
            prompt_tokens += len(tokens)
            cached += n
        elif op[0] == "free":
            bm.free_seq(op[1])
        else:
            raise ValueError(f"prefix_cache_report expects admissions only, got {op[0]!r}")
    in_use = w.num_blocks - bm.num_free()
    private = sum(-(-bm.seq_len(s) // bs) for s in w.decode_seqs)
    # digest rate alone: the full prompt chain of one request, looked up
    toks = w.setup_ops[-1][2]
    t0 = time.perf_counter()
    reps = 20
    for _ in range(reps):
        bm.match_prefix(toks, 12345)  # a salt nobody uses: the first block misses, so hash all blocks below
    t_miss = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    for _ in range(reps):
        bm.match_prefix(toks, w.setup_ops[-1][4])  # every system-prompt block hits
    t_hit = (time.perf_counter() - t0) / reps
    hits = bm.match_prefix(toks, w.setup_ops[-1][4]) // bs
    return {
        "requests": n_req,
        "prompt_tokens": prompt_tokens,
        "cached_tokens": cached,
        "hit_fraction": round(cached / max(prompt_tokens, 1), 4),
        "blocks_in_use_decode_batch": int(in_use),
        "blocks_without_sharing": int(private),
        "admission_host_us_per_request": round(1e6 * t_admit / max(n_req, 1), 1),
        "lookup_us_per_block_hit": round(1e6 * t_hit / max(hits, 1), 3),
        "lookup_us_first_block_miss": round(1e6 * t_miss, 3),
        "note": "host-only; admission = digest lookups + reservation of the uncached rest with its ids",
    }


# ----------------------------------------------------------------- CPU leg
def cpu_baseline(workload_name, num_seqs):
    """The oracle (unchanged) timed on one decode step of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle.runner import OracleRun
    from workloads import Workload

    over = {} if num_seqs is None else dict(num_seqs=num_seqs)
    w = Workload(workload_name, overrides=over)
    run = OracleRun(w)  # untimed: materialise the pools for the sample
    q = w.q(0)
    t0 = time.perf_counter()
    run.step(0)
    ref = run.attention(q)
    dt = time.perf_counter() - t0
    _, lens = run.tables()
    c = w.config
    kv = decode_kv_bytes(lens, c.num_kv_heads, c.head_dim, c.elem_bytes)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    assert np.isfinite(ref).all()
    return {
        "value": kv / dt / 1e9,
        "unit": "GB/s",
        "tokens_per_s": w.num_seqs / dt,
        "seconds": dt,
        "cores": int(threads),
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"one full decode step (bookkeeping, append, fp64 gather+attention) of {w.num_seqs} "
                  f"sequences of {workload_name}, lengths {int(min(lens))}..{int(max(lens))}",
    }


# ------------------------------------------------------------ prefill leg
def run_prefill(args, w, dev):
    """Consecutive chunked-prefill steps: each appends every sequence's chunk
    (bookkeeping, slot upload, append kernel) and runs causal attention of
    the chunk over the whole cache."""
    import numpy as np
    import torch

    import paged_kv_cache_230_amd as pkv

    c = w.config
    S = w.num_seqs
    nsteps = args.warmup + args.steps
    cache = pkv.PagedKVCache(w.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.torch_dtype, dev,
                             w.free_order)
    for op in w.setup_ops:
        cache.apply(op, w.kv)
    # Two distinct sets of chunk values, alternated (values do not steer the kernels).
    kvq = []
    for k in range(2):
        kn, vn = w.kv(("chunk", k))
        kvq.append((kn.to(dev), vn.to(dev), w.prefill_q(k).to(dev)))
    T = int(sum(w.chunk_lens))
    out = torch.empty(T, c.num_q_heads, c.head_dim, dtype=c.torch_dtype, device=dev)
    qs = torch.from_numpy(w.query_start().astype(np.int32)).to(dev)
    seqs = list(w.decode_seqs)
    bs = c.block_size
    max_len = max(cache.bm.seq_len(s) for s in seqs) + nsteps * max(w.chunk_lens)
    max_blocks = -(-max_len // bs)
    tables_h = torch.empty(S, max_blocks, dtype=torch.int32, pin_memory=True)
    lens_h = torch.empty(S, dtype=torch.int32, pin_memory=True)
    slots_h = torch.empty(T, dtype=torch.int32, pin_memory=True)
    tables_d = torch.empty(S, max_blocks, dtype=torch.int32, device=dev)
    lens_d = torch.empty(S, dtype=torch.int32, device=dev)
    slots_d = torch.empty(T, dtype=torch.int32, device=dev)
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps)]
    done = [torch.cuda.Event() for _ in range(nsteps)]
    step_lens = []

    def step(k):
        if k:
            done[k - 1].synchronize()  # the pinned staging buffers are free again
        slots, pairs = cache.bm.append_slots(seqs, w.chunk_lens)
        assert pairs.shape[0] == 0
        slots_h.numpy()[:] = slots
        cache.bm.block_tables(seqs, max_blocks, tables_h.numpy(), lens_h.numpy())
        step_lens.append(lens_h.numpy().copy())
        slots_d.copy_(slots_h, non_blocking=True)
        tables_d.copy_(tables_h, non_blocking=True)
        lens_d.copy_(lens_h, non_blocking=True)
        kn, vn, q = kvq[k % 2]
        pkv.paged_kv_append(kn, vn, cache.k_cache, cache.v_cache, slots_d)
        ev0[k].record()
        pkv.paged_attention_prefill(out, q, cache.k_cache, cache.v_cache, tables_d, lens_d, qs, max(w.chunk_lens))
        ev1[k].record()
        done[k].record()

    if args.calibrate_copy:
        calibration_copy(dev)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} prefill steps)", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for k in range(args.warmup, nsteps):
        step(k)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timed = range(args.warmup, nsteps)
    call_s = [ev0[k].elapsed_time(ev1[k]) / 1e3 for k in timed]
    flops = [prefill_flops(step_lens[k], w.chunk_lens, c.num_q_heads, c.head_dim) for k in timed]
    achieved = sum(flops) / sum(call_s)
    value = sum(flops) / elapsed
    peak_mfma, median_mfma = (None, None) if args.no_read_peak else measured_mfma_peak(dev)
    return {
        "metric": PREFILL_METRIC,
        "value": round(value / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "num_seqs": S,
            "chunk_tokens_per_step": T,
            "context_first_step": [int(min(step_lens[args.warmup])), int(max(step_lens[args.warmup]))],
            "context_last_step": [int(min(step_lens[-1])), int(max(step_lens[-1]))],
            "num_q_heads": c.num_q_heads,
            "num_kv_heads": c.num_kv_heads,
            "head_dim": c.head_dim,
            "block_size": bs,
        },
        "tokens_per_s": round(T * args.steps / elapsed, 1),
        "prefill_call_ms": round(1e3 * sum(call_s) / len(call_s), 4),
        "roofline": {
            "bound": "mfma",
            "kernel": "paged_attention_prefill",
            "achieved": round(achieved / 1e12, 2),
            "peak": MFMA_BF16_PEAK / 1e12,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK, 4),
            "traffic": load_prefill_traffic(w.name, args.steps, args.warmup),
            "traffic_unit": "HBM bytes per call, mean over the timed calls",
            "algorithmic_flops_per_call_mean": int(sum(flops) / len(flops)),
            # the probe's issued bf16 matrix-core rate; the kernel issues 1.5
            # products per useful one (the probabilities' low parts)
            "measured_mfma_peak_tflops": round(peak_mfma / 1e12, 1) if peak_mfma else None,
            "measured_mfma_median_tflops": round(median_mfma / 1e12, 1) if median_mfma else None,
            "frac_of_measured_peak": round(achieved / peak_mfma, 4) if peak_mfma else None,
        },
        "cpu_baseline": None,
    }


def prefill_cpu_baseline(w, num_seqs):
    """The oracle's prefill attention timed on the host over a bounded
    sample: the first ``num_seqs`` sequences of the workload (their history
    and chunk lengths; pool materialised before timing), scaled to TFLOP/s
    with the same causal flop count."""
    from threadpoolctl import threadpool_info

    from oracle.runner import OracleRun
    from workloads import Workload

    n = num_seqs or 2
    c = w.config
    hist = [int(L) - int(C) for L, C in zip(w.lengths[:n], w.chunk_lens[:n])]
    chunks = [int(C) for C in w.chunk_lens[:n]]
    need = sum(-(-int(L) // c.block_size) for L in w.lengths[:n])
    ws = Workload(w.name, overrides=dict(histories=hist, chunks=chunks, num_blocks=need + 8))
    run = OracleRun(ws)
    run.prefill_step(0)
    q = ws.prefill_q(0)
    t0 = time.perf_counter()
    run.prefill_attention(q)
    dt = time.perf_counter() - t0
    flops = prefill_flops(ws.lengths, chunks, c.num_q_heads, c.head_dim)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "seconds": dt,
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"oracle prefill_attention (fp64) on {n} sequences shaped like the first {n} of the batch: "
                  f"chunks {chunks}, contexts {[int(L) for L in ws.lengths]}",
    }


# --------------------------------------------------------------- swap leg
def run_swap(args, w, dev):
    """Consecutive swap steps: all sequences out to the pinned host pool
    (bookkeeping, pair upload, device -> host block copies), then back in
    (host -> device).  Each direction is timed with HIP events around its
    copy kernel; the block bookkeeping runs on the host beforehand."""
    import numpy as np
    import torch

    import paged_kv_cache_230_amd as pkv

    c = w.config
    nsteps = args.warmup + args.steps
    cache = pkv.PagedKVCache(w.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.torch_dtype, dev,
                             w.free_order)
    for op in w.setup_ops:
        cache.apply(op, w.kv)
    bm = cache.bm
    bm.add_host_pool(w.host_blocks)
    hk, hv = pkv.host_pools(w.host_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.torch_dtype)
    block_bytes = 2 * c.num_kv_heads * c.block_size * c.head_dim * c.elem_bytes
    seqs = list(w.decode_seqs)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nsteps)]
    moved = []
    torch.cuda.synchronize()

    def step(k):
        out_pairs = np.concatenate([bm.swap_out(s) for s in seqs])
        d_out = torch.from_numpy(out_pairs).to(dev)
        in_pairs = np.concatenate([bm.swap_in(s) for s in seqs])
        d_in = torch.from_numpy(in_pairs).to(dev)
        ev[k][0].record()
        pkv.paged_kv_swap_blocks(cache.k_cache, cache.v_cache, hk, hv, d_out)
        ev[k][1].record()
        pkv.paged_kv_swap_blocks(hk, hv, cache.k_cache, cache.v_cache, d_in)
        ev[k][2].record()
        moved.append((len(out_pairs) * block_bytes, len(in_pairs) * block_bytes))
        torch.cuda.synchronize()  # the pair buffers are reused next step

    for k in range(args.warmup):
        step(k)
    t0 = time.perf_counter()
    for k in range(args.warmup, nsteps):
        step(k)
    elapsed = time.perf_counter() - t0
    timed = range(args.warmup, nsteps)
    out_s = [ev[k][0].elapsed_time(ev[k][1]) / 1e3 for k in timed]
    in_s = [ev[k][1].elapsed_time(ev[k][2]) / 1e3 for k in timed]
    out_b = sum(moved[k][0] for k in timed)
    in_b = sum(moved[k][1] for k in timed)
    d2h = out_b / sum(out_s)
    h2d = in_b / sum(in_s)
    slow = min(d2h, h2d)
    return {
        "metric": SWAP_METRIC,
        "value": round((out_b + in_b) / (sum(out_s) + sum(in_s)) / 1e9, 2),  # one direction at a time
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": len(seqs), "context_len": int(w.lengths[0]) - 1,
                   "bytes_each_way_per_step": moved[-1][0], "num_kv_heads": c.num_kv_heads, "head_dim": c.head_dim,
                   "block_size": c.block_size},
        "swap_out_gbps": round(d2h / 1e9, 2),
        "swap_in_gbps": round(h2d / 1e9, 2),
        "swap_out_ms": round(1e3 * sum(out_s) / len(out_s), 3),
        "swap_in_ms": round(1e3 * sum(in_s) / len(in_s), 3),
        "roofline": {
            "bound": "host_link",
            "kernel": "paged_kv_swap_blocks (slower direction: " + ("device->host" if d2h <= h2d else "host->device") + ")",
            "achieved": round(slow / 1e9, 2),
            "peak": HOST_LINK_PEAK / 1e9,
            "unit": "GB/s",
            "frac": round(slow / HOST_LINK_PEAK, 4),
            "traffic": None,
        },
        "cpu_baseline": None,
    }


# ---------------------------------------------------------- multi-turn leg
def multiturn_replay(w, kind):
    """Host-only replay of the conversation stream through the radix index
    (``kind == "radix"``) or chained block digests (``"hash"``): prompt
    tokens reused, blocks in use at the end, host time per admission and
    per insertion."""
    import paged_kv_cache_230_amd as pkv

    bs = w.config.block_size
    bm = pkv.BlockManager(w.num_blocks, bs, w.free_order)
    rx = pkv.RadixIndex(bm) if kind == "radix" else None
    toks = [w.conv_tokens(i) for i in range(w.num_convs)]
    reused = prompt = admits = inserts = 0
    t_admit = t_insert = 0.0
    for t in range(w.num_turns):
        for i in range(w.num_convs):
            sid = 100 * (t + 1) + i
            pe, te = w.prompt_end[i][t], w.turn_end[i][t]
            t0 = time.perf_counter()
            m = rx.admit(sid, toks[i][:pe]) if rx else bm.add_seq_cached(sid, toks[i][:pe], 0)
            t_admit += time.perf_counter() - t0
            admits += 1
            bm.append_slots([sid], [te - m], token_ids=toks[i][m:te])
            if rx:
                t0 = time.perf_counter()
                rx.insert(sid, toks[i][:te])
                t_insert += time.perf_counter() - t0
                inserts += 1
                rx.release(sid)
            bm.free_seq(sid)
            reused += m
            prompt += pe
    # blocks kept for reuse once every request has finished: held by radix
    # holders, or carrying a digest on the eviction list
    kept = w.num_blocks - bm.num_free() if rx else bm.num_cached()
    if rx:
        rx.close()
    return {"reused_tokens": reused, "prompt_tokens": prompt, "fraction": round(reused / prompt, 4),
            "blocks_kept_for_reuse": kept, "admit_us": round(1e6 * t_admit / admits, 2),
            "insert_us": round(1e6 * t_insert / max(inserts, 1), 2)}


def run_multiturn(args, w, dev):
    """The conversation stream on the GPU through the radix index: per turn,
    admissions, appends (copy-on-write of shared partial blocks), one decode
    over all conversations (timed with HIP events), insertions."""
    import numpy as np
    import torch

    import paged_kv_cache_230_amd as pkv

    c = w.config
    radix = multiturn_replay(w, "radix")
    hashed = multiturn_replay(w, "hash")
    cache = pkv.PagedKVCache(w.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.torch_dtype, dev,
                             w.free_order)
    rx = pkv.RadixIndex(cache.bm)
    kv = [tuple(x.to(dev) for x in w.kv(("conv", i))) for i in range(w.num_convs)]
    toks = [w.conv_tokens(i) for i in range(w.num_convs)]
    qs = [w.turn_q(t).to(dev) for t in range(w.num_turns)]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(w.num_turns)]
    kv_bytes = []
    copies = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(w.num_turns):
        sids = [100 * (t + 1) + i for i in range(w.num_convs)]
        for i, sid in enumerate(sids):
            pe, te = w.prompt_end[i][t], w.turn_end[i][t]
            m = rx.admit(sid, toks[i][:pe])
            _, pairs = cache.append([sid], [te - m], kv[i][0][m:te], kv[i][1][m:te])
            copies += pairs.shape[0]
        out = torch.empty_like(qs[t])
        tables, lens, _, lh = cache.tables(sids)
        ev[t][0].record()
        pkv.paged_attention_decode(out, qs[t], cache.k_cache, cache.v_cache, tables, lens, int(lh.max()),
                                   shared_blocks=cache.bm.num_shared() > 0)
        ev[t][1].record()
        kv_bytes.append(decode_kv_bytes(lh, c.num_kv_heads, c.head_dim, c.elem_bytes))
        for i, sid in enumerate(sids):
            rx.insert(sid, toks[i][:w.turn_end[i][t]])
            rx.release(sid)
            cache.bm.free_seq(sid)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dec_s = [a.elapsed_time(b) / 1e3 for a, b in ev]
    rx.close()
    return {
        "metric": MULTITURN_METRIC,
        "value": radix["fraction"],
        "unit": "fraction of prompt tokens",
        "n_gpus": 1,
        "steps": w.num_turns,
        "warmup": 0,
        "ms_per_step": round(elapsed / w.num_turns * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_convs": w.num_convs, "num_turns": w.num_turns,
                   "num_q_heads": c.num_q_heads, "num_kv_heads": c.num_kv_heads, "head_dim": c.head_dim,
                   "block_size": c.block_size},
        "radix": radix,
        "chained_digests": hashed,
        "partial_blocks_copied_on_write": int(copies),
        "decode_ms_per_turn": [round(1e3 * x, 4) for x in dec_s],
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_attention_decode (one call per turn over all conversations)",
            "achieved": round(sum(kv_bytes) / sum(dec_s) / 1e9, 2),
            "peak": HBM_PEAK / 1e9,
            "unit": "GB/s",
            "frac": round(sum(kv_bytes) / sum(dec_s) / HBM_PEAK, 4),
            "traffic": None,
            "note": "calls of a few MB are launch- and latency-bound; listed for completeness, not an HBM claim",
        },
        "cpu_baseline": None,
    }


def swap_cpu_baseline(w):
    """The oracle's block copy (oracle.pool.swap_copy) timed on the host for
    one sequence's blocks, device-pool format to host-pool format."""
    import numpy as np

    import oracle.pool as opool

    c = w.config
    nblk = -(-(int(w.lengths[0]) - 1) // c.block_size)
    src = opool.new_pools(nblk, c.num_kv_heads, c.head_dim, c.block_size, np.uint16, fill=1)
    dst = opool.new_pools(nblk, c.num_kv_heads, c.head_dim, c.block_size, np.uint16)
    pairs = [(b, nblk - 1 - b) for b in range(nblk)]
    t0 = time.perf_counter()
    opool.swap_copy(src[0], src[1], dst[0], dst[1], pairs)
    dt = time.perf_counter() - t0
    nbytes = nblk * 2 * c.num_kv_heads * c.block_size * c.head_dim * c.elem_bytes
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "seconds": dt, "cores": 1, "kind": "oracle",
            "sample": f"oracle swap_copy of one 32k-token sequence ({nblk} blocks, {nbytes / 1e6:.0f} MB) "
                      "between two NumPy pools"}


# -------------------------------------------------- auxiliary: paging itself
def paging_waste(lens, block_size, reserve):
    """KV slots reserved but holding no token: whole-block paging against a
    contiguous reservation of `reserve` tokens per sequence (the pages'
    fragmentation comparison)."""
    lens = [int(L) for L in lens]
    tokens = sum(lens)
    paged = sum(-(-L // block_size) * block_size for L in lens)
    reserved = len(lens) * reserve
    return {"tokens": tokens, "paged_slots": paged, "paged_waste": round((paged - tokens) / paged, 5),
            "reserved_slots": reserved, "reserved_waste": round((reserved - tokens) / reserved, 5),
            "reserve_tokens_per_seq": reserve}


def run_paging_aux(args, w, dev):
    """The decode call over the workload's shuffled pool against the same
    kernel over a pool whose blocks were handed out in order (each
    sequence's blocks contiguous), same lengths and values: the cost of the
    gather.  The two outputs must be bit-identical (the kernel reduces in
    logical order whatever the physical placement)."""
    import numpy as np
    import torch

    import paged_kv_cache_230_amd as pkv

    c = w.config
    S = w.num_seqs
    bs = c.block_size
    seqs = list(w.decode_seqs)
    res, outs = {}, {}
    for name, order in (("shuffled", w.free_order), ("contiguous", np.arange(w.num_blocks, dtype=np.int32))):
        cache = pkv.PagedKVCache(w.num_blocks, c.num_kv_heads, c.head_dim, bs, c.torch_dtype, dev, order)
        for op in w.setup_ops:
            cache.apply(op, w.kv)
        kn, vn = w.kv(("step", 0))
        slots, pairs = cache.bm.append_slots(seqs, [1] * S)
        assert len(pairs) == 0
        pkv.paged_kv_append(kn.to(dev), vn.to(dev), cache.k_cache, cache.v_cache,
                            torch.from_numpy(np.asarray(slots, np.int32)).to(dev))
        max_len = max(cache.bm.seq_len(sq) for sq in seqs)
        mb = -(-max_len // bs)
        tab = np.zeros((S, mb), np.int32)
        lens = np.zeros(S, np.int32)
        cache.bm.block_tables(seqs, mb, tab, lens)
        tab_d, lens_d = torch.from_numpy(tab).to(dev), torch.from_numpy(lens).to(dev)
        q = w.q(0).to(dev)
        out = torch.empty(S, c.num_q_heads, c.head_dim, dtype=c.torch_dtype, device=dev)
        ws = torch.empty(max(pkv.paged_attention_workspace_bytes(S, c.num_q_heads, c.num_kv_heads, c.head_dim, bs,
                                                                 max_len, args.partition), 256),
                         dtype=torch.uint8, device=dev)

        shared = cache.bm.num_shared() > 0 if args.shared_blocks == "auto" else args.shared_blocks == "on"

        def call():
            pkv.paged_attention_decode(out, q, cache.k_cache, cache.v_cache, tab_d, lens_d, max_len,
                                       partition_size=args.partition, workspace=ws, shared_blocks=shared)

        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        us = []
        for _ in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            e1.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3)
        res[name] = float(np.median(us))
        outs[name] = out.clone()
        kv_bytes = decode_kv_bytes(lens, c.num_kv_heads, c.head_dim, c.elem_bytes)
        print(f"# {name}: decode {res[name]:.1f} us ({kv_bytes / res[name] / 1e3:.1f} GB/s of KV)", file=sys.stderr,
              flush=True)
        del cache, ws
        torch.cuda.empty_cache()
    same = bool(torch.equal(outs["shuffled"].view(torch.int16) if c.dtype == "bf16" else outs["shuffled"],
                            outs["contiguous"].view(torch.int16) if c.dtype == "bf16" else outs["contiguous"]))
    lens_all = [int(L) for L in lens]
    return {
        "aux": "paging overhead and waste",
        "workload": w.name,
        "decode_us_shuffled_pool": round(res["shuffled"], 2),
        "decode_us_contiguous_pool": round(res["contiguous"], 2),
        "gather_overhead_pct": round(100.0 * (res["shuffled"] / res["contiguous"] - 1.0), 2),
        "outputs_bit_identical": same,
        "calls_timed": args.steps,
        "waste": paging_waste(lens_all, bs, -(-max(lens_all) // bs) * bs),
    }


# ----------------------------------------------------------------- GPU leg
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 200 for the 32k layer and the 8B-shaped batch, 30 for the others)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: 20 for the 32k layer and the 8B-shaped batch, 5 for the others)")
    ap.add_argument("--workload", default="c3_70b_32k_bf16")
    ap.add_argument("--partition", type=int, default=0,
                    help="about this many tokens per decode workgroup (0 = one round of resident workgroups)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-append", action="store_true",
                    help="append with paged_kv_append, then paged_attention_decode (two calls) instead of "
                         "paged_attention_decode_append")
    ap.add_argument("--cpu-seqs", type=int, default=None, help="sequences in the oracle sample (default: all)")
    ap.add_argument("--no-read-peak", action="store_true",
                    help="skip the ceiling probes: streaming and tile reads (decode), matrix-core rate (prefill); for "
                         "counter and trace runs, which would count their work too")
    ap.add_argument("--overlap-stage", action="store_true",
                    help="stage step k+1's bookkeeping on a second stream during step k's decode (two buffer sets)")
    ap.add_argument("--marked", type=int, default=50,
                    help="event-timed decode calls for the roofline, and event-bounded steps for the distribution")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--block-size", type=int, default=None, choices=(16, 32),
                    help="run the workload's batch at this block size instead of its own (for A/B runs; the "
                         "headline figure uses the workload's block size)")
    ap.add_argument("--shared-blocks", choices=("auto", "on", "off"), default="auto",
                    help="decode cache policy: auto sets PKV_DECODE_SHARED_BLOCKS when the block manager holds "
                         "shared blocks; on / off force it (results are identical, only the time differs)")
    ap.add_argument("--aux-paging", action="store_true",
                    help="instead of the benchmark: decode over the shuffled pool vs a contiguous one, and the "
                         "slot waste of paging vs max-length reservation")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU sharding of this path is a design note, not a measured configuration.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_230_amd as pkv
    from workloads import Workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = Workload(args.workload, overrides={} if args.block_size is None else {"block_size": args.block_size})
    # The 32k layer's step is 0.34 ms and the 8B-shaped batch's 0.11 ms: 200
    # timed steps keep a single host hiccup or the pipeline's start from
    # moving the mean, and 20 warm-up steps let a fresh process's host path
    # settle (a first run on a fresh box has issued steps at 3x the host time
    # of the next).  The other workloads keep 30 / 5: their pools are sized
    # for the lengths they reach in that many steps.
    d_steps, d_warmup = DEFAULT_STEPS.get(w.name, (30, 5))
    args.steps = d_steps if args.steps is None else args.steps
    args.warmup = d_warmup if args.warmup is None else args.warmup
    if args.aux_paging:
        print(json.dumps(run_paging_aux(args, w, dev)), flush=True)
        return
    if hasattr(w, "num_convs"):
        result = run_multiturn(args, w, dev)
        print(json.dumps(result), flush=True)
        return
    if hasattr(w, "host_blocks"):
        result = run_swap(args, w, dev)
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = swap_cpu_baseline(w)
        print(json.dumps(result), flush=True)
        return
    if hasattr(w, "chunk_lens"):
        result = run_prefill(args, w, dev)
        if not args.no_cpu_baseline:
            print("# cpu baseline: oracle on the host", file=sys.stderr, flush=True)
            result["cpu_baseline"] = prefill_cpu_baseline(w, args.cpu_seqs)
        print(json.dumps(result), flush=True)
        return
    c = w.config
    S = w.num_seqs
    # Warm-up steps, the timed steps (no markers between kernels: each event
    # marker costs a dispatch gap), then a pass of marked steps whose HIP
    # events time each decode call for the roofline figure, then a pass with
    # one event at each step boundary for the distribution of step times.
    n_marked = args.marked
    n_dist = args.marked
    nsteps = args.warmup + args.steps + n_marked + n_dist + 1
    print(f"# setup {w.name}: {S} sequences, pool {w.num_blocks} blocks", file=sys.stderr, flush=True)
    t_setup = time.perf_counter()
    cache = pkv.PagedKVCache(w.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.torch_dtype, dev,
                             w.free_order)
    for op in w.setup_ops:
        cache.apply(op, w.kv)
    torch.cuda.synchronize()
    print(f"# setup done in {time.perf_counter() - t_setup:.1f}s", file=sys.stderr, flush=True)

    # Per-step inputs, resident on the GPU before timing.
    step_k, step_v, step_q = [], [], []
    for k in range(nsteps):
        kn, vn = w.kv(("step", k))
        step_k.append(kn.to(dev))
        step_v.append(vn.to(dev))
        step_q.append(w.q(k).to(dev))

    step_ids = [w.step_tokens(k) for k in range(nsteps)]  # None unless the workload tracks token ids
    bm = cache.bm
    seqs = np.asarray(w.decode_seqs, np.int64)
    # Cache policy of the decode calls: read K/V through the caches when the
    # batch's sequences share blocks (prefix sharing, forks), else stream them.
    shared_blocks = bm.num_shared() > 0 if args.shared_blocks == "auto" else args.shared_blocks == "on"
    bs = c.block_size
    max_len_bound = int(max(bm.seq_len(int(s)) for s in seqs)) + nsteps
    max_blocks = -(-max_len_bound // bs)
    P = args.partition
    wph = pkv.paged_attention_workgroups_per_head(S, c.num_kv_heads, c.head_dim, bs, max_len_bound, P, c.torch_dtype)
    ws_bytes = pkv.paged_attention_workspace_bytes(S, c.num_q_heads, c.num_kv_heads, c.head_dim, bs, max_len_bound, P)
    workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty(S, c.num_q_heads, c.head_dim, dtype=c.torch_dtype, device=dev)
    # Step buffers on the device.  With --overlap-stage there are two sets,
    # used on alternate steps: the bookkeeping of step k+1 is staged into one,
    # on a stream of its own, while step k's decode still reads the other (the
    # block manager tracks both tables).  Measured slower on the 32k layer
    # (0.387 against 0.381 ms per step: the cross-stream events cost more than
    # the staging kernel they hide), so by default every step is staged on
    # the main stream, in series with its decode.
    nsets = 2 if args.overlap_stage else 1
    tables_s = [torch.empty(S, max_blocks, dtype=torch.int32, device=dev) for _ in range(nsets)]
    lens_s = [torch.empty(S, dtype=torch.int32, device=dev) for _ in range(nsets)]
    slots_s = [torch.empty(S, dtype=torch.int32, device=dev) for _ in range(nsets)]
    pairs_s = [torch.empty(S, 2, dtype=torch.int32, device=dev) for _ in range(nsets)]
    main_stream = torch.cuda.current_stream(dev)
    stage_stream = torch.cuda.Stream(dev)  # default priority
    staged_ev = [torch.cuda.Event() for _ in range(nsets)]
    released_ev = [torch.cuda.Event() for _ in range(nsets)]
    # One pinned step record per step, so the host never waits for the GPU to
    # release one (and no event is needed for that).
    stage_cap = pkv.BlockManager.stage_capacity(S, max_blocks)
    stage = [torch.zeros(stage_cap, dtype=torch.int32, pin_memory=True) for _ in range(nsteps)]
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps)]
    marked = range(args.warmup + args.steps, args.warmup + args.steps + n_marked)
    dist = range(args.warmup + args.steps + n_marked, nsteps)  # an event after each of these steps
    host_s = [0.0] * nsteps
    seg = {"wait": 0.0, "bookkeeping+stage": 0.0, "copy+append": 0.0, "decode": 0.0}
    step_lens = []
    n_cow_total = 0

    def step(k):
        nonlocal n_cow_total
        th = time.perf_counter()
        t1 = time.perf_counter()
        r = k % nsets
        tables_d, lens_d, slots_d, pairs_d = tables_s[r], lens_s[r], slots_s[r], pairs_s[r]
        if nsets == 1:
            n_cow, max_len = bm.stage_step(seqs, stage[k], tables_d, lens_d, slots_d, pairs_d, token_ids=step_ids[k])
        else:
            with torch.cuda.stream(stage_stream):
                stage_stream.wait_event(released_ev[r])  # the decode that last read this set is done
                n_cow, max_len = bm.stage_step(seqs, stage[k], tables_d, lens_d, slots_d, pairs_d,
                                               token_ids=step_ids[k])
                staged_ev[r].record(stage_stream)
            main_stream.wait_event(staged_ev[r])
        step_lens.append(stage[k].numpy()[4 + S: 4 + 2 * S].copy())  # lengths in the record
        t2 = time.perf_counter()
        if n_cow:
            pkv.paged_kv_copy_blocks(cache.k_cache, cache.v_cache, pairs_d[:n_cow])
            n_cow_total += n_cow
        if args.separate_append:
            pkv.paged_kv_append(step_k[k], step_v[k], cache.k_cache, cache.v_cache, slots_d)
        t3 = time.perf_counter()
        if k in marked:
            ev0[k].record()
        if args.separate_append:
            pkv.paged_attention_decode(out, step_q[k], cache.k_cache, cache.v_cache, tables_d, lens_d, max_len,
                                       partition_size=P, workspace=workspace, shared_blocks=shared_blocks)
        else:
            pkv.paged_attention_decode_append(out, step_q[k], step_k[k], step_v[k], cache.k_cache, cache.v_cache,
                                              tables_d, lens_d, max_len, partition_size=P, workspace=workspace,
                                              shared_blocks=shared_blocks)
        if k in marked or k in dist:
            ev1[k].record()
        if nsets > 1:
            released_ev[r].record(main_stream)
        t4 = time.perf_counter()
        host_s[k] = t4 - th
        if args.warmup <= k < args.warmup + args.steps:
            for name, dt in (("wait", t1 - th), ("bookkeeping+stage", t2 - t1), ("copy+append", t3 - t2),
                             ("decode", t4 - t3)):
                seg[name] += dt

    if args.calibrate_copy:
        calibration_copy(dev)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    gc.collect()
    gc.disable()  # no collector pause inside the timed steps
    t0 = time.perf_counter()
    for k in range(args.warmup, args.warmup + args.steps):
        step(k)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    for k in marked:
        step(k)
    for k in dist:
        step(k)
    torch.cuda.synchronize()
    print(f"# timed {args.steps} steps in {elapsed:.4f}s; host us/step by segment: "
          + ", ".join(f"{k}={1e6 * v / args.steps:.1f}" for k, v in seg.items()), file=sys.stderr, flush=True)

    # Physical K/V bytes of one call: each distinct block once (shared prefix
    # blocks are read by many sequences but held once).
    t_host, l_host = bm.block_tables(seqs, max_blocks)
    used = t_host[np.arange(max_blocks)[None, :] < -(-l_host[:, None] // bs)]
    unique_blocks = int(np.unique(used).size)
    block_bytes = 2 * bs * c.num_kv_heads * c.head_dim * c.elem_bytes

    timed = range(args.warmup, args.warmup + args.steps)
    lens_t = [step_lens[k] for k in timed]
    kv_bytes = [decode_kv_bytes(L, c.num_kv_heads, c.head_dim, c.elem_bytes) for L in lens_t]
    # roofline: the marked decode calls, each timed by its own events
    dec_ms = [ev0[k].elapsed_time(ev1[k]) for k in marked]
    lens_m = [step_lens[k] for k in marked]
    kv_bytes_m = [decode_kv_bytes(L, c.num_kv_heads, c.head_dim, c.elem_bytes) for L in lens_m]
    alg_bytes = [decode_algorithmic_bytes(L, c.num_q_heads, c.num_kv_heads, c.head_dim, bs, c.elem_bytes)
                 + (0 if args.separate_append else append_algorithmic_bytes(L, c.num_kv_heads, c.head_dim,
                                                                            c.elem_bytes))
                 for L in lens_m]
    flops = [decode_flops(L, c.num_q_heads, c.head_dim) for L in lens_m]
    mean_dec_s = sum(dec_ms) / len(dec_ms) / 1e3
    achieved = (sum(alg_bytes) / len(alg_bytes)) / mean_dec_s
    # step times between consecutive boundary events (one marker per step)
    dk = list(dist)
    step_us = [1e3 * ev1[dk[i - 1]].elapsed_time(ev1[dk[i]]) for i in range(1, len(dk))]
    step_kv = [decode_kv_bytes(step_lens[dk[i]], c.num_kv_heads, c.head_dim, c.elem_bytes) for i in range(1, len(dk))]
    step_gbps = [b / (t * 1e-6) / 1e9 for b, t in zip(step_kv, step_us)]
    dec_us = [1e3 * t for t in dec_ms]
    peak_read, median_read = (None, None) if args.no_read_peak else measured_read_peak(dev)
    tile_read, tile_median = ((None, None) if args.no_read_peak
                              else measured_tile_read(dev, cache, t_host, l_host, bs))
    ms_per_step = elapsed / args.steps * 1e3
    value = sum(kv_bytes) / elapsed / 1e9
    traffic = load_traffic(w.name, P) if not args.separate_append else None

    result = {
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
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "num_seqs": S,
            "context_len_first_step": int(lens_t[0].min()),
            "num_q_heads": c.num_q_heads,
            "num_kv_heads": c.num_kv_heads,
            "head_dim": c.head_dim,
            "block_size": bs,
            "num_blocks": w.num_blocks,
            "partition_size": P,
            "decode_workgroups": wph * c.num_kv_heads,
        },
        "tokens_per_s": round(S * args.steps / elapsed, 1),
        "pct_hbm_peak_whole_step": round(100.0 * value * 1e9 / HBM_PEAK, 2),
        "decode_call_us": round(mean_dec_s * 1e6, 2),
        "decode_kv_gbps": round((sum(kv_bytes_m) / len(kv_bytes_m)) / mean_dec_s / 1e9, 2),
        "decode_calls_marked": len(dec_ms),
        "decode_tflops": round((sum(flops) / len(flops)) / mean_dec_s / 1e12, 2),
        "cow_pairs": n_cow_total,
        # the single call writes the step's rows from inside the decode kernel
        # when there is at most one sequence per decode workgroup of a kv head
        "append_folded": (not args.separate_append) and S <= wph,
        "shared_blocks": shared_blocks,
        "host_us_per_step": round(1e6 * sum(host_s[k] for k in timed) / args.steps, 1),
        # step k+1's bookkeeping staged on a second stream during step k's decode
        "stage_overlapped": nsets > 1,
        "roofline": {
            "bound": "hbm",
            "kernel": ("paged_attention_decode (partition kernel + log-sum-exp merge)" if args.separate_append
                       else "paged_attention_decode_append (partition kernel with the step's append + "
                            "log-sum-exp merge)"),
            "achieved": round(achieved / 1e9, 2),
            "peak": HBM_PEAK / 1e9,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_call": int(sum(alg_bytes) / len(alg_bytes)),
            "unique_kv_block_bytes_last_call": unique_blocks * block_bytes,
            "calls_timed": len(dec_ms),
            "call_us": {k: round(v, 2) for k, v in percentiles(dec_us).items()},
            "measured_read_peak_gbps": round(peak_read / 1e9, 1) if peak_read else None,
            "measured_read_median_gbps": round(median_read / 1e9, 1) if median_read else None,
            "frac_of_measured_peak": round(achieved / peak_read, 4) if peak_read else None,
            # the same call's K/V tiles streamed by pkv_tile_read, no arithmetic
            "measured_tile_read_gbps": round(tile_read / 1e9, 1) if tile_read else None,
            "measured_tile_read_median_gbps": round(tile_median / 1e9, 1) if tile_median else None,
            "frac_of_tile_read": round(achieved / tile_read, 4) if tile_read else None,
        },
        "step_distribution": {
            "steps": len(step_us),
            "note": "one HIP event at each step boundary (a marker adds a dispatch gap to every step)",
            "step_us": {k: round(v, 2) for k, v in percentiles(step_us).items()},
            "kv_gbps": {k: round(v, 1) for k, v in percentiles(step_gbps).items()},
        },
        "cpu_baseline": None,
    }
    if unique_blocks < int(used.size):
        result["roofline"]["note"] = (
            "blocks shared by several sequences are read once per sequence but held once: logical bytes exceed "
            "HBM traffic, so this rate is not an HBM roofline figure")
    if any(op[0] == "admit" for op in w.setup_ops):
        result["prefix_cache"] = prefix_cache_report(w)
    del cache, step_k, step_v, step_q, workspace
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("# cpu baseline: oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seqs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
