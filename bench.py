"""Benchmark of one decode step of paged attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1] [--unfused]
    python bench.py --op stream | prefill | prefill_long | copy_blocks | swap_out | swap_in | fragmentation

A step is one pass of the hot path over one synthetic batch that is already
resident in HBM: every sequence's new token is stored in its cache slot and
decode attention runs over context_len + 1 tokens.  One-pass workloads do
both in one launch (pa_decode_append; --unfused: pa_cache_write, then
pa_decode); the long-context workload runs pa_cache_write, then
pa_decode_partitioned + pa_reduce.  Prints one JSON line.

By default the line's headline is the Llama-7B-shaped workload and
`per_config` holds the same measurement for it, the long-context, GQA and
fp8 shared-prefix workloads (--workload NAME: that one only).

value = KV tokens attended per second over the K timed steps (whole job).
roofline = the attention kernels' algorithmic HBM bytes per launch (a block
shared by several sequences counted once) / their mean duration back to
back (HIP events on the launch stream: around the whole timed region when
the step is one launch, else around the attention launches of each step:
pa_decode_partitioned + pa_reduce for long context), against 8 TB/s.
flushed = the same launches timed one by one, each after a 512 MiB read of
another buffer outside the events (3 warm-ups, 20 launches; median, min).
stream_ceiling = the read rate of a probe that streams random 4 KiB tiles
the way the decode kernels do (libpa_probe.so), the practical ceiling: the
better of equal shares per wavefront and shares weighted 6% towards the
even-numbered dies (which stream faster on this part).
cpu_baseline = the CPU oracle (test infrastructure, fp64 numpy) on a bounded
sample of the same workload, timed on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "decode attention KV tokens/s and achieved HBM GB/s (% of peak), 1×MI355X"
ELEM_BYTES = {"f16": 2, "bf16": 2, "e4m3fn": 1}
CSRC = os.path.join(ROOT, "paged_kv_cache_78_amd", "csrc")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def unique_kv_tokens(wl, cached_lens) -> int:
    """Cached tokens counted once per physical slot: a block shared by several
    block tables (a shared prefix) is read from HBM once per launch."""
    table = wl.block_table.cpu().tolist()
    BS = wl.block_size
    used = {}
    for s, L in enumerate(cached_lens):
        for j in range(-(-L // BS)):
            b = table[s][j]
            used[b] = max(used.get(b, 0), min(BS, L - j * BS))
    return sum(used.values())


def algorithmic_bytes(wl, cached_lens, append: bool, unique: bool = False) -> int:
    """Bytes one launch of the attention kernel must move: K+V of every
    cached token it reads, q in, out, block-table ids and context_lens; the
    fused step adds the new tokens' K/V (read from the inputs, written to the
    cache) and slot_mapping.  unique: K+V of a shared block counted once."""
    S, H, D, KVH, BS = wl.num_seqs, wl.num_heads, wl.head_size, wl.num_kv_heads, wl.block_size
    e_kv, e_q = ELEM_BYTES[wl.cache_dtype], ELEM_BYTES[wl.q_dtype]
    tok = unique_kv_tokens(wl, cached_lens) if unique else sum(cached_lens)
    ids = sum(-(-L // BS) for L in cached_lens)
    b = tok * KVH * D * 2 * e_kv + 2 * S * H * D * e_q + 4 * ids + 4 * S
    if append:
        b += S * KVH * D * 2 * (e_q + e_kv) + 4 * S
    return b


def recorded_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sources") != src_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_workload(name: str, device: str):
    import workloads
    if name == "long_context":
        return workloads.long_context(device=device)        # ~10.7 GB pool: draw on the GPU
    return workloads.make(name).to(device)


def cpu_baseline(wl, lens, budget_s: float = 10.0):
    """Time the CPU oracle on whole sequences of the workload (host copies of
    just those sequences' blocks) until about budget_s has been spent."""
    import numpy as np
    import torch
    import oracle
    from workloads import to_numpy_bits
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = torch.get_num_threads()
    S = wl.num_seqs
    order = list(range(S))
    done_tokens = 0
    done_seqs = 0
    t_total = 0.0
    table = wl.block_table.cpu().numpy()
    qn = to_numpy_bits(wl.q)
    i = 0
    while t_total < budget_s and i < 64 * S:
        s = order[i % S]
        i += 1
        L = int(lens[s])
        nblk = -(-L // wl.block_size)
        ids = torch.from_numpy(table[s, :nblk].astype(np.int64)).to(wl.k_cache.device)
        k = to_numpy_bits(wl.k_cache.index_select(0, ids))
        v = to_numpy_bits(wl.v_cache.index_select(0, ids))
        row = np.arange(nblk, dtype=np.int32)[None, :]
        t0 = time.perf_counter()
        oracle.paged_decode(qn[s:s + 1], k, v, row, np.array([L], dtype=np.int32), wl.scale,
                            wl.num_kv_heads, wl.block_size, wl.q_dtype, wl.cache_dtype,
                            wl.k_scale, wl.v_scale)
        t_total += time.perf_counter() - t0
        done_tokens += L
        done_seqs += 1
    return {"value": done_tokens / t_total, "unit": "KV tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done_seqs} whole sequences (all {wl.num_heads} heads, {done_tokens} "
                      f"KV tokens) of the same workload, fp64 numpy, {t_total:.1f} s"}


PEAK_HOST_LINK_GBS = 64.0   # PCIe 5.0 x16, one direction


def bench_block_copy(args, torch, pa, dev):
    """Whole-block copies on a Llama-7B-shaped pool (32 kv heads, head 128,
    block 16, f16: 128 KiB of K and 128 KiB of V per block): 2048 pairs per
    launch, inside one 8192-block GPU pool (copy-on-write) or between it and
    a 2048-block pool in pinned host memory (swap out / in)."""
    import numpy as np
    NB, KVH, BS, D, N = 8192, 32, 16, 128, 2048
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    k = torch.randn((NB, KVH, BS, D), generator=g, device=dev, dtype=torch.float32).half()
    v = torch.randn((NB, KVH, BS // 4, D, 4), generator=g, device=dev,
                    dtype=torch.float32).half()
    perm = torch.randperm(NB, generator=g, device=dev).to(torch.int32)
    if args.op == "copy_blocks":
        m = torch.stack([perm[:N], perm[N:2 * N]], 1).contiguous()
        src, dst = (k, v), (k, v)
    else:
        hk = torch.empty((N, KVH, BS, D), dtype=torch.float16).pin_memory()
        hv = torch.empty((N, KVH, BS // 4, D, 4), dtype=torch.float16).pin_memory()
        hid = torch.randperm(N, generator=g, device=dev).to(torch.int32)
        if args.op == "swap_out":
            m = torch.stack([perm[:N], hid], 1).contiguous()
            src, dst = (k, v), (hk, hv)
        else:
            m = torch.stack([hid, perm[:N]], 1).contiguous()
            src, dst = (hk, hv), (k, v)
    payload = N * 2 * KVH * BS * D * 2               # K + V bytes moved per launch

    def launch():
        pa.copy_blocks(src[0], src[1], dst[0], dst[1], m)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    ev = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        launch()
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    kern_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    if args.op == "copy_blocks":
        alg = 2 * payload                               # read + write in HBM
        roof = {"bound": "hbm", "peak": PEAK_HBM_GBS}
    else:
        alg = payload                                   # one crossing of the host link
        roof = {"bound": "host_link", "peak": PEAK_HOST_LINK_GBS}
    achieved = alg / (kern_ms * 1e-3) / 1e9
    roof.update({"kernel": "pa_copy_blocks", "achieved": achieved, "unit": "GB/s",
                 "frac": achieved / roof["peak"],
                 "traffic": recorded_traffic("pa_copy_blocks", args.op, kernel_source_hash()),
                 "algorithmic_bytes_per_launch": alg, "kernel_ms": kern_ms,
                 "kernel_sources": kernel_source_hash()})
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        hk_ = k[:256].cpu().numpy()
        hv_ = v[:256].cpu().numpy()
        mm = np.stack([np.arange(128), np.arange(128, 256)], 1).astype(np.int32)
        c0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - c0 < args.cpu_budget and reps < 200:
            oracle.copy_blocks(hk_, hv_, hk_, hv_, mm)
            reps += 1
        dt = time.perf_counter() - c0
        cpu = {"value": reps * 128 * 2 * KVH * BS * D * 2 / dt / 1e9, "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{reps} oracle copies of 128 blocks inside a 256-block host pool, "
                         f"{dt:.1f} s"}
    return {
        "metric": f"{args.op} payload GB/s (K+V of whole blocks), 1×MI355X",
        "value": payload / (ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{args.op}: {N} blocks of a Llama-7B-shaped pool "
                               f"(32 kv heads, head 128, block 16, f16)",
                   "pairs": N, "block_bytes_k_plus_v": 2 * KVH * BS * D * 2},
        "roofline": roof, "cpu_baseline": cpu,
    }


def bench_fragmentation(args, pa):
    """The simulation the how-it-works page proposes (its closing project):
    100 requests with lengths uniform in [50, 500] tokens, block size 16,
    against reserving max_len = 512 contiguous slots per request.  The paged
    side runs through the library's block manager, which grows every
    sequence token by token (append_slots, as decode steps do).  Reported:
    the share of allocated slots left unused by both schemes, how many such
    requests fit in the memory of 100 reserved ones, and the manager's
    append rate through its Python binding, one call per decode step of the
    live requests (the oracle's Python manager is the baseline)."""
    import random
    import numpy as np
    BS, MAXLEN, N = 16, 512, 100
    rng = random.Random(7)
    lens = [rng.randint(50, 500) for _ in range(N)]
    pool_slots = N * MAXLEN                          # the memory of 100 reserved requests
    bm = pa.BlockManager(pool_slots // BS, 0, BS)
    for i, L in enumerate(lens):                     # prompt of half the length, then decode
        bm.add_sequence(i, L // 2)
    t_append = 0.0
    appended = 0
    cur = [L // 2 for L in lens]
    live = list(range(N))
    while live:
        t0 = time.perf_counter()
        slots, _ = bm.append_slots(live)             # one decode step of the live requests
        t_append += time.perf_counter() - t0
        appended += len(live)
        for i in live:
            cur[i] += 1
        live = [i for i in live if cur[i] < lens[i]]
    assert all(bm.seq_len(i) == lens[i] for i in range(N))
    used_blocks = pool_slots // BS - bm.num_free()
    paged_frag = 1.0 - sum(lens) / (used_blocks * BS)
    naive_frag = 1.0 - sum(lens) / (N * MAXLEN)
    # how many requests of the same length distribution fit in the same memory
    fit, i = 0, N
    while True:
        L = rng.randint(50, 500)
        try:
            bm.add_sequence(i, L)
        except pa.BlockManager.NoFreeBlocks:
            break
        fit += 1
        i += 1
    paged_concurrency = N + fit
    # serving-sized batch: 4096 live sequences, 100 decode steps
    big = pa.BlockManager(1 << 20, 0, BS)
    ids = list(range(4096))
    for j in ids:
        big.add_sequence(j, 100)
    t0 = time.perf_counter()
    for _ in range(100):
        big.append_slots(ids)
    big_rate = 4096 * 100 / (time.perf_counter() - t0)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        ob = oracle.BlockManager(pool_slots // BS, 0, BS)
        for j, L in enumerate(lens):
            ob.add_sequence(j, L // 2)
        dt, done = 0.0, 0
        cur = [L // 2 for L in lens]
        live = list(range(N))
        while live:
            c0 = time.perf_counter()
            for j in live:
                ob.append_slot(j)
            dt += time.perf_counter() - c0
            done += len(live)
            for j in live:
                cur[j] += 1
            live = [j for j in live if cur[j] < lens[j]]
        cpu = {"value": done / dt, "unit": "slots/s", "cores": 1, "kind": "oracle",
               "sample": f"the same {done} appends through the oracle's Python manager, {dt:.2f} s"}
    return {
        "metric": "paged KV cache: unused share of allocated slots (%), how-it-works simulation",
        "value": 100.0 * paged_frag, "unit": "%", "n_gpus": 0, "steps": 1, "warmup": 0,
        "ms_per_step": t_append * 1e3, "higher_is_better": False, "scaling": "none",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": "100 requests, lengths U[50,500], prompt = half, the rest "
                               "generated token by token; block 16 vs 512 reserved per request",
                   "naive_unused_percent": 100.0 * naive_frag,
                   "requests_in_the_memory_of_100_reserved": paged_concurrency,
                   "concurrency_ratio": paged_concurrency / N,
                   "manager_append_rate_slots_per_s": appended / t_append,
                   "manager_append_rate_4096_seq_batches_slots_per_s": big_rate},
        "roofline": None, "cpu_baseline": cpu,
    }


PEAK_MFMA_F16_TFLOPS = 2500.0


def prefill_flops(b, causal: bool = True) -> int:
    """QK and PV multiply-adds of every (query, key) pair a chunk attends:
    4 * D flops per pair per query head."""
    cu = b.cu_seqlens_q.cpu().tolist()
    K = b.context_lens.cpu().tolist()
    pairs = 0
    for s in range(b.num_seqs):
        n = cu[s + 1] - cu[s]
        # causal: query i attends K - n + i + 1 keys; otherwise all K
        pairs += n * (K[s] - n + 1) + n * (n - 1) // 2 if causal else n * K[s]
    return 4 * b.head_size * b.num_heads * pairs


def bench_prefill(args, torch, pa, dev, long_prompts: bool = False):
    """One chunked-prefill step on the Llama-7B shape: 16 sequences, a
    512-token chunk each after U{0..1536} cached tokens; the chunk's K/V are
    written (pa_cache_write), then the chunk attends its context (pa_prefill,
    causal).  long_prompts: 8 whole prompts of 4096 tokens instead (no cached
    prefix), and the same attention without the causal mask timed beside it."""
    import workloads
    b = (workloads.llama7b_prefill_long if long_prompts else workloads.llama7b_prefill_chunks)(
        device=dev)
    out = torch.empty_like(b.q)
    ev = []

    def step(record):
        pa.cache_write(b.new_k, b.new_v, b.k_cache, b.v_cache, b.slot_mapping)
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        pa.prefill(b.q, b.k_cache, b.v_cache, b.block_table, b.cu_seqlens_q, b.context_lens,
                   b.scale, b.max_seqlen_q, out=out)
        if record:
            e1.record()
            ev.append((e0, e1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    kern_ms = sum(a.elapsed_time(c) for a, c in ev) / len(ev)
    flops = prefill_flops(b)
    achieved = flops / (kern_ms * 1e-3) / 1e12
    T = int(b.q.shape[0])
    non_causal = None
    if long_prompts:
        # the cache already holds every prompt: the same launches without the mask
        ev_nc = []
        for _ in range(args.steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            pa.prefill(b.q, b.k_cache, b.v_cache, b.block_table, b.cu_seqlens_q, b.context_lens,
                       b.scale, b.max_seqlen_q, causal=False, out=out)
            e1.record()
            ev_nc.append((e0, e1))
        torch.cuda.synchronize()
        nc_ms = sum(a.elapsed_time(c) for a, c in ev_nc) / len(ev_nc)
        nc_flops = prefill_flops(b, causal=False)
        non_causal = {"kernel_ms": nc_ms, "algorithmic_flops_per_launch": nc_flops,
                      "achieved": nc_flops / (nc_ms * 1e-3) / 1e12, "unit": "TFLOP/s",
                      "frac": nc_flops / (nc_ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS}
    cpu = None
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        from workloads import to_numpy_bits
        # one sequence of the same batch, two heads' worth of work: the oracle
        # loops over heads, so the time scales with the heads it is given
        cu = b.cu_seqlens_q.cpu().tolist()
        n = cu[1] - cu[0]
        K = int(b.context_lens[0])
        nblk = -(-K // b.block_size)
        ids = b.block_table[0, :nblk].long()
        row = np.arange(nblk, dtype=np.int32)[None, :]
        pairs = n * (K - n + 1) + n * (n - 1) // 2
        done, dt, heads = 0, 0.0, 0
        while dt < args.cpu_budget and heads < b.num_heads:
            h = heads
            kc = to_numpy_bits(b.k_cache.index_select(0, ids)[:, h:h + 1])
            vc = to_numpy_bits(b.v_cache.index_select(0, ids)[:, h:h + 1])
            qn = to_numpy_bits(b.q[:n, h:h + 1])
            c0 = time.perf_counter()
            oracle.paged_prefill(qn, kc, vc, row, np.array([0, n], dtype=np.int32),
                                 np.array([K], dtype=np.int32), b.scale, 1, b.block_size,
                                 "f16", "f16")
            dt += time.perf_counter() - c0
            done += 4 * b.head_size * pairs
            heads += 1
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            cores = torch.get_num_threads()
        cpu = {"value": done / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "sample": f"sequence 0 ({n} queries over {K} keys), {heads} of "
                         f"{b.num_heads} heads, fp64 numpy, {dt:.1f} s"}
    wname = "llama7b_prefill_long" if long_prompts else "llama7b_prefill_chunks"
    wdesc = ("llama7b_prefill_long: 8 prompts x 4096 tokens, no cached prefix, 32 = 32 kv heads, "
             "head 128, block 16, f16" if long_prompts else
             "llama7b_prefill_chunks: 16 seqs x 512-token chunks after U{0..1536} cached tokens, "
             "32 = 32 kv heads, head 128, block 16, f16")
    line = {
        "metric": "chunked prefill query tokens/s and achieved TFLOP/s (% of f16 MFMA peak), 1×MI355X",
        "value": T / (ms * 1e-3), "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": wdesc, "total_query_tokens": T,
                   "step": "pa_cache_write + pa_prefill"},
        "roofline": {"bound": "mfma", "kernel": "pa_prefill", "achieved": achieved,
                     "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_MFMA_F16_TFLOPS,
                     "traffic": recorded_traffic("pa_prefill", wname, kernel_source_hash()),
                     "algorithmic_flops_per_launch": flops, "kernel_ms": kern_ms,
                     "kernel_sources": kernel_source_hash()},
        "cpu_baseline": cpu,
    }
    if non_causal is not None:
        line["non_causal"] = non_causal
    return line


class StreamProbe:
    """ctypes handle on libpa_probe.so (pa_probe_stream, include/pa_probe.h)."""

    def __init__(self):
        import ctypes
        path = os.path.join(ROOT, "paged_kv_cache_78_amd", "libpa_probe.so")
        if not os.path.exists(path):
            raise SystemExit(f"{path} is missing: build with python -m paged_kv_cache_78_amd.build")
        self.lib = ctypes.CDLL(path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        self.lib.pa_probe_stream.restype = ctypes.c_int
        self.lib.pa_probe_stream.argtypes = [vp, i64, vp, i32, i32, i32, i32, i32, vp, vp]
        self.ctypes = ctypes

    def launch(self, torch, pool, num_tiles, ids, num_waves, tiles_per_wave, nontemporal, sink,
               tile_bytes=4096, in_flight=3):
        c = self.ctypes
        st = self.lib.pa_probe_stream(c.c_void_p(pool.data_ptr()), num_tiles,
                                      c.c_void_p(ids.data_ptr()), num_waves, tiles_per_wave,
                                      tile_bytes, in_flight, 1 if nontemporal else 0,
                                      c.c_void_p(sink.data_ptr()),
                                      c.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"pa_probe_stream failed ({st})")


PROBE_WAVES_PER_WORKGROUP = 4     # the probe's workgroups (stream_probe.hip)
DIES = 8                          # workgroup b runs on die (XCD) b % 8


def stream_rate(torch, probe, dev, pool_bytes: int, num_waves: int, tiles_per_wave: int,
                nontemporal: bool, reps: int = 5, seed: int = 9, tile_bytes: int = 4096,
                in_flight: int = 3, die_skew: float = 0.0) -> dict:
    """GB/s read by the probe: num_waves wavefronts x tiles_per_wave distinct
    random tiles of tile_bytes of a pool_bytes pool, in_flight tiles in flight
    per wavefront (best and median of reps launches after one warm-up).  With
    die_skew > 0 the wavefronts on even-numbered dies read (1 + die_skew) x
    tiles_per_wave tiles and those on odd dies (1 - die_skew) x as many (the
    list is padded with ids outside the pool, which the probe skips)."""
    num_tiles = pool_bytes // tile_bytes
    hi = int(round(tiles_per_wave * (1 + die_skew)))
    lo = int(round(tiles_per_wave * (1 - die_skew)))
    die = (torch.arange(num_waves, device=dev) // PROBE_WAVES_PER_WORKGROUP) % DIES
    real = torch.where(die % 2 == 0, hi, lo)
    need = int(real.sum())
    width = max(hi, lo)
    assert need <= num_tiles
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    chosen = torch.randperm(num_tiles, generator=g, device=dev)[:need].to(torch.int32)
    ids = torch.full((num_waves, width), -1, dtype=torch.int32, device=dev)
    ids[torch.arange(width, device=dev)[None, :] < real[:, None]] = chosen
    ids = ids.contiguous()
    sink = torch.empty(num_waves * 64, dtype=torch.int32, device=dev)
    args = (torch, pool, num_tiles, ids, num_waves, width, nontemporal, sink, tile_bytes,
            in_flight)
    probe.launch(*args)
    ms = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        probe.launch(*args)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del pool, ids, sink
    b = need * tile_bytes
    ms.sort()
    return {"best_gbs": b / (ms[0] * 1e-3) / 1e9, "median_gbs": b / (ms[len(ms) // 2] * 1e-3) / 1e9,
            "bytes": b, "num_waves": num_waves, "tiles_per_wave": tiles_per_wave,
            "tile_bytes": tile_bytes, "in_flight": in_flight, "nontemporal": nontemporal,
            "die_skew": die_skew}


def bench_stream(args, torch, dev):
    """The probe over launch shapes, tile sizes (4 KiB: a 16-bit K or V tile
    at block 16, head 128; 2 KiB: the same in fp8), tiles in flight and both
    cache policies."""
    probe = StreamProbe()
    rows = []
    for nt in (True, False):
        for waves, tiles in ((2048, 64), (8192, 16), (8192, 32), (16384, 16)):
            rows.append(stream_rate(torch, probe, dev, 8 << 30, waves, tiles, nt))
    for tb in (4096, 2048):
        for fl in (2, 3, 4, 6, 8):
            rows.append(stream_rate(torch, probe, dev, 8 << 30, 8192, 32 * 4096 // tb, True,
                                    tile_bytes=tb, in_flight=fl))
    rows.append(stream_rate(torch, probe, dev, 8 << 30, 12288, 32, True, tile_bytes=2048,
                            in_flight=4))
    for skew in (0.03, 0.06, 0.09):
        rows.append(stream_rate(torch, probe, dev, 8 << 30, 8192, 32, True, die_skew=skew))
    best = max(r["best_gbs"] for r in rows if r["nontemporal"])
    return {
        "metric": "HBM read GB/s of random 4 KiB tiles streamed like the decode kernels, 1×MI355X",
        "value": best, "unit": "GB/s", "n_gpus": 1, "steps": 5, "warmup": 1,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8", "data": "synthetic",
        "config": {"workload": "stream probe: distinct random 2 or 4 KiB tiles of an 8 GiB pool",
                   "sweep": rows},
        "roofline": {"bound": "hbm", "achieved": best, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": best / PEAK_HBM_GBS, "traffic": None},
        "cpu_baseline": None,
    }


FLUSH_BYTES = 512 << 20
DEFAULT_WORKLOADS = ["llama7b_mha", "long_context", "gqa", "fp8_shared_prefix"]


def bench_decode(name, args, torch, pa, dev, flush_buf, cpu_budget):
    """One decode workload: back-to-back steps, then the flushed protocol."""
    wl = make_workload(name, dev)
    lens_step = (wl.context_lens + 1).contiguous()       # the step attends the new token too
    lens_host = lens_step.cpu().tolist()
    partitioned = wl.partition_size > 0
    fused = not partitioned and not args.unfused
    P = wl.partition_size
    max_len = max(lens_host)
    out = torch.empty_like(wl.q)
    ws = pa.partition_workspace(wl.num_seqs, wl.num_heads, wl.head_size, max_len, P, dev) \
        if partitioned else None

    def attention(ev):
        """The step's attention launches; ev = (start, mid, end) events or None."""
        if ev:
            ev[0].record()
        if partitioned:
            pa.decode_partitioned_only(wl.q, wl.k_cache, wl.v_cache, wl.block_table, lens_step,
                                       wl.scale, P, max_len, ws, wl.k_scale, wl.v_scale)
            if ev:
                ev[1].record()
            pa.reduce(out, ws, lens_step, P)
        elif fused:
            pa.decode_append(wl.q, wl.new_k, wl.new_v, wl.k_cache, wl.v_cache, wl.slot_mapping,
                             wl.block_table, wl.context_lens, wl.scale, k_scale=wl.k_scale,
                             v_scale=wl.v_scale, out=out)
        else:
            pa.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, lens_step, wl.scale,
                      k_scale=wl.k_scale, v_scale=wl.v_scale, out=out)
        if ev:
            ev[2].record()

    def step(ev=None):
        if not fused:
            pa.cache_write(wl.new_k, wl.new_v, wl.k_cache, wl.v_cache, wl.slot_mapping,
                           k_scale=wl.k_scale, v_scale=wl.v_scale)
        attention(ev)

    def events():
        return tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # back to back: the fused step is one launch, so one event pair around
    # the whole timed region gives its average; multi-launch steps bracket
    # their attention launches in every step
    per_step = [] if not fused else None
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record()
    for _ in range(args.steps):
        if fused:
            step()
        else:
            ev = events()
            step(ev)
            per_step.append(ev)
    r1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    if fused:
        kern_ms = r0.elapsed_time(r1) / args.steps
        part_ms = None
    else:
        kern_ms = sum(a.elapsed_time(c) for a, _, c in per_step) / len(per_step)
        part_ms = (sum(a.elapsed_time(b) for a, b, _ in per_step) / len(per_step)
                   if partitioned else None)

    # launch by launch, each after a read of another 512 MiB buffer (outside
    # the events), so no K/V of the previous launch is left in the caches
    flushed_ms = []
    for i in range(3 + args.flush_launches):
        flush_buf.sum()                      # 512 MiB read, outside the events
        if not fused:
            pa.cache_write(wl.new_k, wl.new_v, wl.k_cache, wl.v_cache, wl.slot_mapping,
                           k_scale=wl.k_scale, v_scale=wl.v_scale)
        ev = events()
        attention(ev)
        torch.cuda.synchronize()
        if i >= 3:
            flushed_ms.append(ev[0].elapsed_time(ev[2]))
    flushed_ms.sort()

    tokens = sum(lens_host)
    # roofline bytes count a shared block once (it is read from HBM once);
    # the logical count reads it once per sequence
    cached = wl.context_lens.cpu().tolist() if fused else lens_host
    alg = algorithmic_bytes(wl, cached, fused, unique=True)
    alg_logical = algorithmic_bytes(wl, cached, fused)
    achieved = alg / (kern_ms * 1e-3) / 1e9
    kernel = ("pa_decode_partitioned + pa_reduce" if partitioned
              else ("pa_decode_append" if fused else "pa_decode"))
    src_hash = kernel_source_hash()
    traffic = recorded_traffic("pa_decode_partitioned" if partitioned else kernel, name, src_hash)
    med = flushed_ms[len(flushed_ms) // 2]
    kv_dt = {"f16": "f16", "bf16": "bf16", "e4m3fn": "e4m3fn KV / bf16 q"}[wl.cache_dtype]
    rec = {
        "workload": name,
        "num_seqs": wl.num_seqs, "num_heads": wl.num_heads, "num_kv_heads": wl.num_kv_heads,
        "head_size": wl.head_size, "block_size": wl.block_size, "kv_dtype": kv_dt,
        "context_tokens_per_step": tokens,
        "partition_size": P if partitioned else None,
        "step": ("pa_decode_append" if fused else
                 "pa_cache_write + " + ("pa_decode_partitioned + pa_reduce" if partitioned
                                        else "pa_decode")),
        "ms_per_step": ms_per_step,
        "kv_tokens_per_s": tokens / (ms_per_step * 1e-3),
        "roofline": {
            "bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
            "algorithmic_bytes_per_launch": alg, "logical_bytes_per_launch": alg_logical,
            "kernel_ms": kern_ms,
            "kernel_timing": ("HIP events around the timed region (launches back to back)"
                              if fused else "HIP events around the attention launches of each "
                                            "step (launches back to back)"),
            "kernel_sources": src_hash,
        },
        "flushed": {
            "protocol": f"3 warm-ups, {args.flush_launches} launches each after a 512 MiB read "
                        "of another buffer outside the events",
            "median_ms": med, "min_ms": flushed_ms[0],
            "achieved_median": alg / (med * 1e-3) / 1e9,
            "frac_median": alg / (med * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "frac_min_time": alg / (flushed_ms[0] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        },
        "cpu_baseline": None,
    }
    if partitioned:
        S, H, D = wl.num_seqs, wl.num_heads, wl.head_size
        parts = sum(-(-L // P) for L in lens_host)
        rec["roofline"]["partitioned_ms"] = part_ms
        rec["roofline"]["reduce_ms"] = kern_ms - part_ms
        rec["roofline"]["partial_triple_bytes"] = H * parts * (D + 2) * 4 * 2
        rec["roofline"]["frac_partitioned_alone"] = alg / (part_ms * 1e-3) / 1e9 / PEAK_HBM_GBS
    if cpu_budget > 0:
        rec["cpu_baseline"] = cpu_baseline(wl, lens_host, cpu_budget)
    del wl, out, ws
    torch.cuda.empty_cache()
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="default",
                    choices=["default", "worked_example", "llama7b_mha", "gqa", "long_context",
                             "fp8_shared_prefix"],
                    help="default: llama7b_mha (the headline) plus long_context, gqa and "
                         "fp8_shared_prefix under per_config")
    ap.add_argument("--op", default="step",
                    choices=["step", "stream", "copy_blocks", "swap_out", "swap_in", "prefill",
                             "prefill_long", "fragmentation"],
                    help="step: one decode step (default); stream: the HBM read probe; "
                         "copy_blocks: copy-on-write copies inside a pool; swap_out / swap_in: "
                         "blocks to / from a pinned host pool; prefill: one chunked-prefill "
                         "step (cache write + pa_prefill); prefill_long: 8 whole 4096-token "
                         "prompts, causal, with the unmasked attention timed beside it; "
                         "fragmentation: the host block "
                         "manager on the how-it-works page's 100-request simulation (CPU only)")
    ap.add_argument("--unfused", action="store_true",
                    help="one-pass workloads: pa_cache_write then pa_decode instead of the "
                         "single pa_decode_append launch")
    ap.add_argument("--flush-launches", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time for the headline workload's baseline "
                         "(a third of it for each other workload)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="before the warm-up, run one plain device copy of BYTES bytes "
                         "(reference dispatch for rocprofv3 FETCH_SIZE/WRITE_SIZE scaling)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(decode attention shards by sequence or kv head with no exchange).",
              file=sys.stderr)
        return 2

    import torch
    import paged_kv_cache_78_amd as pa
    if args.op == "fragmentation":
        print(json.dumps(bench_fragmentation(args, pa)))
        return 0
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (ROCm) and the built libpa.so")
    pa.lib()
    dev = "cuda:0"
    if args.copy_calibration > 0:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.op == "stream":
        print(json.dumps(bench_stream(args, torch, dev)))
        return 0
    if args.op in ("prefill", "prefill_long"):
        print(json.dumps(bench_prefill(args, torch, pa, dev, long_prompts=args.op == "prefill_long")))
        return 0
    if args.op != "step":
        print(json.dumps(bench_block_copy(args, torch, pa, dev)))
        return 0

    names = DEFAULT_WORKLOADS if args.workload == "default" else [args.workload]
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    ceiling = None
    if args.copy_calibration == 0:
        # the practical read ceiling: the probe at the decode kernels' shape
        probe = StreamProbe()
        ceiling = max((stream_rate(torch, probe, dev, 4 << 30, 8192, 32, True, die_skew=k)
                       for k in (0.0, 0.06)), key=lambda r: r["best_gbs"])
    per = []
    for i, name in enumerate(names):
        budget = 0.0 if args.no_cpu_baseline else (args.cpu_budget if i == 0 else args.cpu_budget / 3)
        print(f"[bench] {name}", file=sys.stderr, flush=True)
        rec = bench_decode(name, args, torch, pa, dev, flush_buf, budget)
        if ceiling:
            rec["roofline"]["frac_of_stream_ceiling"] = (rec["roofline"]["achieved"] /
                                                         ceiling["best_gbs"])
        per.append(rec)
    del flush_buf
    head = per[0]
    rec = {
        "metric": METRIC,
        "value": head["kv_tokens_per_s"],
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3fn" if head["kv_dtype"].startswith("e4m3fn") else head["kv_dtype"],
        "data": "synthetic",
        "config": {k: head[k] for k in ("workload", "num_seqs", "num_heads", "num_kv_heads",
                                        "head_size", "block_size", "kv_dtype",
                                        "context_tokens_per_step", "partition_size", "step")},
        "roofline": head["roofline"],
        "flushed": head["flushed"],
        "cpu_baseline": head["cpu_baseline"],
        "stream_ceiling": ceiling,
        "library": os.path.relpath(pa.binding._LIB_PATH, ROOT),
        "per_config": per,
    }
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
