"""Benchmark of the paged decode hot path on one MI355X.

One step = the whole hot path over one synthetic batch already resident in
HBM: append each sequence's new K/V token, then decode attention over the
paged cache -- by default one ``pa_decode_append`` call (slots from the
block tables), ``--separate-append`` for ``pa_kv_cache_write`` with the
slot mapping then ``pa_decode`` -- plus ``pa_decode_reduce`` when the
context is split and not merged inside the decode launch (``--partition
-2``, ``PA_PARTITION_AUTO_MERGED``).  Default workload: the
Llama-3-70B-shaped decode batch (256 sequences, 64 query / 8 KV heads, head
dim 128, 16-token blocks, bf16 KV, lognormal lengths, median 1024), the
largest bf16 configuration; ``--workload 2`` is the Llama-3-8B-shaped one.

Prints one JSON line on stdout.  ``value`` is the step's algorithmic HBM
bytes divided by the step time (GB/s), K steps back to back (timed both
eagerly and as replays of a captured HIP graph; the faster mode is the step
time and ``config.launch`` names it); ``roofline``
is the decode kernel alone and ``roofline.in_step`` the appending decode
the steps launch, each timed launch by launch with HIP events on the stream
it runs on after a cache flush (``--flush``), next to the bandwidth a plain
streaming read attains in the same run; ``cpu_baseline`` is the fp64 CPU
oracle on a bounded sample of the same batch, one process, and
``cpu_baseline_all_cores`` the same oracle in a pool of processes over the
batch's sequences.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD public spec
KERNEL_SOURCES = ["decode_mfma.hip", "decode_valu.hip", "pa_device.hpp", "pa_mfma.hpp", "pa_split.hpp",
                  "pa_internal.hpp", "pa_merge.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_253_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name: str, partition: int, launches_per_step: int):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, or
    None when there are none for this kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_sha() or rec.get("partition") != partition:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(batch, seconds: float, threads: int = 1) -> dict:
    """Time the oracle (its BLAS limited to ``threads`` threads) on whole
    sequences of the batch, in a seeded order and cycling over the batch,
    until ``seconds`` of oracle time have been spent (host copies of each
    sequence are made outside the timed part)."""
    from threadpoolctl import threadpool_limits

    from oracle import paged
    from workloads import decode_bytes, extract_sequences

    w = batch.workload
    order = np.random.default_rng(0).permutation(len(batch.context_lens))
    subs = {}
    done, spent, nbytes, tokens = 0, 0.0, 0, 0
    with threadpool_limits(limits=threads):
        while spent < seconds:
            b = int(order[done % len(order)])
            if b not in subs:
                subs[b] = extract_sequences(batch, [b])
                if len(subs) > 64:  # bound host memory on long-context batches
                    subs.pop(next(iter(subs)))
            sub = subs[b]
            t = time.perf_counter()
            paged.decode(sub["q"], sub["k_pool"], sub["v_pool"], sub["block_tables"],
                         sub["context_lens"], w.block_size, batch.scale, w.q_dtype,
                         w.cache_dtype, sub["k_scale"], sub["v_scale"])
            spent += time.perf_counter() - t
            done += 1
            acct = decode_bytes(sub["context_lens"], w.num_q_heads, w.num_kv_heads, w.head_dim,
                                w.block_size, w.cache_dtype, w.q_dtype)
            nbytes += acct["total"]
            tokens += acct["tokens"]
    distinct = min(done, len(order))
    return {"value": nbytes / spent / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "tokens_per_s": tokens / spent, "seconds": round(spent, 2),
            "sample": f"{done} sequence decodes over {distinct} of {len(order)} sequences of "
                      f"the batch ({tokens} context tokens), fp64 numpy oracle, "
                      f"{threads} BLAS thread{'s' if threads > 1 else ''}"}


def host_cores() -> int:
    """Cores this process may run on, capped by OMP_NUM_THREADS when set."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(cap)) if cap.isdigit() and int(cap) > 0 else n


def bench_copy(args) -> int:
    """Copy-on-write burst: pa_copy_blocks on half the blocks of the
    workload's pool (independent random pairs, e.g. a wide beam or parallel
    sampling fork), back-to-back launches timed with HIP events."""
    import torch

    import paged_kv_cache_253_amd as pk
    from oracle import paged
    from workloads import WORKLOADS, copy_bytes, host_view, make_batch

    w = with_cache_dtype(WORKLOADS[args.workload], args.cache_dtype)
    if w is None:
        return 2
    kw = dict(cache_dtype=w.cache_dtype, block_size=w.block_size)
    dev = "cuda"
    batch = make_batch(w, device=dev)
    nb = batch.num_blocks
    npairs = min(8192, nb // 2)
    ids = np.random.default_rng(w.seed).permutation(nb)[:2 * npairs]
    pairs_np = np.stack([ids[:npairs], ids[npairs:]], axis=1).astype(np.int64)
    pairs = torch.from_numpy(pairs_np).to(dev)
    for _ in range(args.warmup):
        pk.copy_blocks(batch.k_pool, batch.v_pool, pairs, **kw)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        pk.copy_blocks(batch.k_pool, batch.v_pool, pairs, **kw)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = copy_bytes(npairs, w.num_kv_heads, w.head_dim, w.block_size, w.cache_dtype)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] copy {npairs} block pairs ({nbytes / 1e6:.1f} MB moved): {ms * 1e3:.1f} us = "
        f"{gbs:.0f} GB/s = {100 * gbs / PEAK_HBM_GBS:.1f}% of peak")
    result = {
        "metric": "copy-on-write block copy: achieved HBM GB/s (% of peak)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.cache_dtype, "data": "synthetic",
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "config": {"workload": f"{w.name} pool, copy-on-write burst", "block_pairs": npairs,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "kv_dtype": w.cache_dtype,
                   "launch": "eager, back to back"},
        "roofline": {"bound": "hbm", "kernel": "pa_copy_blocks", "achieved": round(gbs, 1),
                     "launch_us": round(ms * 1e3, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes,
                     "traffic": None},
    }
    if not args.no_cpu:
        # the oracle's copy on a bounded sample of the same pairs
        sample = pairs_np[:64]
        used = np.unique(sample.reshape(-1))
        remap = {int(b): i for i, b in enumerate(used)}
        k_h = host_view(batch.k_pool.index_select(0, torch.from_numpy(used).to(dev)))
        v_h = host_view(batch.v_pool.index_select(0, torch.from_numpy(used).to(dev)))
        local = np.vectorize(remap.get)(sample)
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            paged.copy_blocks(k_h, v_h, local)
            n += 1
        dt = time.perf_counter() - t0
        cpu_bytes = n * copy_bytes(len(sample), w.num_kv_heads, w.head_dim, w.block_size,
                                   w.cache_dtype)
        result["cpu_baseline"] = {"value": round(cpu_bytes / dt / 1e9, 3), "unit": "GB/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": f"{n} oracle copies of 64 block pairs "
                                            f"(numpy, whole pools copied per call)"}
    print(json.dumps(result), flush=True)
    return 0


PEAK_HOST_LINK_GBS = 64.0  # PCIe 5.0 x16, one direction (MI355X host interface)


def bench_swap(args) -> int:
    """Preemption swap: pa_swap_blocks moving a quarter of the workload's
    pool to a pinned host pool and back, each direction timed separately
    (back-to-back launches, HIP events)."""
    import torch

    import paged_kv_cache_253_amd as pk
    from workloads import WORKLOADS, copy_bytes, make_batch

    w = with_cache_dtype(WORKLOADS[args.workload], args.cache_dtype)
    if w is None:
        return 2
    kw = dict(cache_dtype=w.cache_dtype, block_size=w.block_size)
    dev = "cuda"
    batch = make_batch(w, device=dev)
    n = batch.num_blocks // 4
    kh = torch.empty((n,) + tuple(batch.k_pool.shape[1:]), dtype=batch.k_pool.dtype, pin_memory=True)
    vh = torch.empty((n,) + tuple(batch.v_pool.shape[1:]), dtype=batch.v_pool.dtype, pin_memory=True)
    rng = np.random.default_rng(w.seed)
    dev_ids = rng.permutation(batch.num_blocks)[:n]
    out_map = torch.from_numpy(np.stack([dev_ids, np.arange(n)], 1).astype(np.int64)).to(dev)
    in_map = torch.from_numpy(np.stack([np.arange(n), dev_ids], 1).astype(np.int64)).to(dev)
    steps = max(1, min(args.steps, 10))

    def timed(fn):
        for _ in range(min(args.warmup, 2)):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_out = timed(lambda: pk.swap_blocks(kh, vh, batch.k_pool, batch.v_pool, out_map, **kw))
    ms_in = timed(lambda: pk.swap_blocks(batch.k_pool, batch.v_pool, kh, vh, in_map, **kw))
    moved = copy_bytes(n, w.num_kv_heads, w.head_dim, w.block_size, w.cache_dtype) // 2  # one side
    gbs_out = moved / (ms_out * 1e-3) / 1e9
    gbs_in = moved / (ms_in * 1e-3) / 1e9
    log(f"[bench] swap {n} blocks ({moved / 1e6:.1f} MB each way): out {ms_out * 1e3:.0f} us = "
        f"{gbs_out:.1f} GB/s, in {ms_in * 1e3:.0f} us = {gbs_in:.1f} GB/s")
    result = {
        "metric": "preemption swap over the host link: achieved GB/s (device to host)",
        "value": round(gbs_out, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": min(args.warmup, 2), "ms_per_step": round(ms_out, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.cache_dtype, "data": "synthetic",
        "config": {"workload": f"{w.name} pool, swap of {n} blocks", "blocks": n,
                   "bytes_each_way": moved, "host_to_device_gbs": round(gbs_in, 2),
                   "host_to_device_ms": round(ms_in, 4)},
        "roofline": {"bound": "host link", "kernel": "pa_swap_blocks", "achieved": round(gbs_out, 2),
                     "peak": PEAK_HOST_LINK_GBS, "unit": "GB/s",
                     "frac": round(gbs_out / PEAK_HOST_LINK_GBS, 4), "traffic": None},
    }
    print(json.dumps(result), flush=True)
    return 0


PEAK_MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, AMD public spec


def bench_prefill(args) -> int:
    """Several query tokens per sequence: back-to-back pa_prefill_chunk
    (+ merge) launches on a seeded batch; HBM roofline when the arithmetic
    intensity is below the bf16 ridge, matrix-core roofline above it."""
    import torch

    import paged_kv_cache_253_amd as pk
    from workloads import PREFILL_WORKLOADS, make_batch, prefill_bytes

    w, nq = PREFILL_WORKLOADS[args.case]
    w = with_cache_dtype(w, args.cache_dtype)
    if w is None:
        return 2
    dev = "cuda"
    batch = make_batch(w, device=dev)
    lens = batch.context_lens
    qlens = np.minimum(lens, nq).astype(np.int32)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    g = torch.Generator(device=dev).manual_seed(w.seed + 1)
    q = torch.randn((int(qs[-1]), w.num_q_heads, w.head_dim), generator=g,
                    device=dev).to(torch.bfloat16)
    bt = torch.from_numpy(batch.block_tables).to(dev)
    cl = torch.from_numpy(lens).to(dev)
    qs_d = torch.from_numpy(qs).to(dev)
    out = torch.empty_like(q)
    part = args.partition
    if part is None:  # the binding's own choice, made once and reused
        part = pk.prefill_partition(len(lens), w.num_q_heads, w.num_kv_heads, w.head_dim,
                                    int(qlens.max()), batch.max_context_len,
                                    w.head_dim == 128 and w.cache_dtype in ("bf16", "int4"), dev)
    ws = pk.new_workspace(int(qs[-1]), w.num_q_heads, w.num_kv_heads, w.head_dim,
                          batch.max_context_len, part, dev) if part else None

    def run():
        pk.prefill_chunk(q, batch.k_pool, batch.v_pool, bt, cl, batch.max_context_len, qs_d,
                         int(qlens.max()), batch.scale, batch.k_scale, batch.v_scale,
                         partition_size=part, out=out, workspace=ws, cache_dtype=w.cache_dtype)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    acc = prefill_bytes(lens, qlens, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                        w.cache_dtype, w.q_dtype)
    gbs = acc["total"] / (ms * 1e-3) / 1e9
    tflops = acc["flops"] / (ms * 1e-3) / 1e12
    mfma_bound = acc["flops"] / acc["total"] > PEAK_MFMA_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    log(f"[bench] prefill {args.case}: {len(lens)} seqs, {int(qs[-1])} query rows, P={part}: "
        f"{ms * 1e3:.1f} us = {gbs:.0f} GB/s, {tflops:.1f} TFLOP/s "
        f"({'matrix-core' if mfma_bound else 'HBM'} bound)")
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_BF16_TFLOPS, 4),
                "algorithmic_flops": acc["flops"]}
        value, unit, metric = tflops, "TFLOP/s", "multi-query paged attention: achieved TFLOP/s"
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": acc["total"]}
        value, unit, metric = gbs, "GB/s", "multi-query paged attention: achieved HBM GB/s"
    roof.update({"kernel": "pa_prefill_chunk" + (" + pa_prefill_reduce" if part else ""),
                 "launch_us": round(ms * 1e3, 2), "traffic": None})
    result = {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.cache_dtype,
        "data": "synthetic",
        "config": {"workload": args.case, "num_seqs": len(lens), "query_tokens_per_seq": nq,
                   "context_tokens": acc["tokens"], "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "partition_size": part,
                   "gbs": round(gbs, 1), "tflops": round(tflops, 2)},
        "roofline": roof,
    }
    if not args.no_cpu:
        from oracle import paged
        from workloads import extract_sequences, host_view
        b = int(np.argmin(lens))
        sub = extract_sequences(batch, [b])
        ns = min(int(qlens[b]), 32)  # the sequence's last ns query rows: a chunk of its own
        q_h = host_view(q[int(qs[b + 1]) - ns:int(qs[b + 1])])
        qs_1 = np.array([0, ns], np.int64)
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 8.0) or n == 0:
            paged.prefill_chunk(q_h, sub["k_pool"], sub["v_pool"], sub["block_tables"],
                                sub["context_lens"], qs_1, w.block_size, batch.scale, "bf16",
                                w.cache_dtype, sub["k_scale"], sub["v_scale"])
            n += 1
        dt = time.perf_counter() - t0
        one = prefill_bytes(lens[b:b + 1], [ns], w.num_q_heads, w.num_kv_heads,
                            w.head_dim, w.block_size, w.cache_dtype, w.q_dtype)
        result["cpu_baseline"] = {
            "value": round((one["flops"] / 1e12 if mfma_bound else one["total"] / 1e9) * n / dt, 5),
            "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"{n} oracle runs of the last {ns} query rows of sequence {b} "
                      f"({int(lens[b])} tokens)"}
    print(json.dumps(result), flush=True)
    return 0


def with_cache_dtype(w, cache_dtype):
    """The workload with another KV cache format, or None (message printed)
    when the swap makes no sense."""
    if not cache_dtype or cache_dtype == w.cache_dtype:
        return w
    import dataclasses
    if cache_dtype == "int4":
        if w.cache_dtype == "f32":
            print("--cache-dtype int4 needs a bf16 or FP8 workload (bf16 queries)", file=sys.stderr)
            return None
        return dataclasses.replace(w, cache_dtype="int4", q_dtype="bf16",
                                   name=w.name.rsplit("-", 1)[0] + "-int4")
    if not w.cache_dtype.startswith("fp8"):
        print("--cache-dtype fp8_* applies to FP8 workloads only", file=sys.stderr)
        return None
    return dataclasses.replace(w, cache_dtype=cache_dtype,
                               name=w.name + ("-e5m2" if cache_dtype == "fp8_e5m2" else ""))


FLUSH_COPY_BYTES = 512 << 20    # device-to-device copy before every timed launch
FLUSH_READ_BYTES = 1 << 30      # then a streaming read, so the copy's dirty lines leave first
ATTAINABLE_BYTES = 2 << 30      # the streaming-read buffer (more than the largest decode reads)


class Flush:
    """Run before every per-launch timing: a 512 MiB device-to-device copy,
    so the memory-side cache (256 MB) and the L2s hold none of the decode's
    data, then (mode "copy+read", the default) a 1 GiB streaming read of
    another buffer, so the lines the copy dirtied are written back during
    the read and not during the timed launch.  Both outside the timed
    events and outside any captured graph."""

    def __init__(self, torch, pk, mode: str, dev):
        self.mode, self.pk = mode, pk
        if mode == "none":
            return
        self.src = torch.zeros(FLUSH_COPY_BYTES, dtype=torch.uint8, device=dev)
        self.dst = torch.empty_like(self.src)
        if "read" in mode:
            self.rd = torch.ones(FLUSH_READ_BYTES, dtype=torch.uint8, device=dev)
            self.sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def __call__(self):
        if self.mode == "none":
            return
        self.dst.copy_(self.src)
        if "read" in self.mode:
            self.pk.stream_read(self.rd, self.sink)

    def describe(self) -> str:
        return {"none": "none (back to back)",
                "copy": "512 MiB device copy before each launch",
                "copy+read": "512 MiB device copy then a 1 GiB streaming read before each launch"
                }[self.mode]


def timed_launches(torch, fn, reps: int, flush) -> np.ndarray:
    """Milliseconds of each of ``reps`` launches of ``fn``, one HIP event pair
    around each on torch's current stream (the stream the library launches
    on), each preceded by ``flush``; one untimed flush and launch first
    (first-call costs of the flush's and the timed kernels)."""
    flush()
    fn()
    pairs = []
    for _ in range(reps):
        flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in pairs])


def dist_us(ms: np.ndarray) -> dict:
    us = np.asarray(ms) * 1e3
    return {"mean": round(float(us.mean()), 2), "median": round(float(np.median(us)), 2),
            "p10": round(float(np.percentile(us, 10)), 2),
            "p90": round(float(np.percentile(us, 90)), 2), "n": int(us.size)}


def _oracle_worker(conn):
    """One process of the CPU-baseline pool: decode its share of the batch's
    sequences with the oracle, its BLAS on one thread, ``rounds`` times when
    told to; report (seconds, bytes, tokens, decodes)."""
    from threadpoolctl import threadpool_limits

    from oracle import paged

    meta, shard = conn.recv()

    def decode(sub):
        paged.decode(sub["q"], sub["k_pool"], sub["v_pool"], sub["block_tables"],
                     sub["context_lens"], meta["block_size"], meta["scale"], meta["q_dtype"],
                     meta["cache_dtype"], sub["k_scale"], sub["v_scale"])

    with threadpool_limits(limits=1):
        if shard:
            decode(min(shard, key=lambda x: x[1])[0])  # imports and first-call costs
        conn.send("ready")
        rounds = conn.recv()
        nbytes = tokens = count = 0
        t0 = time.perf_counter()
        for _ in range(rounds):
            for sub, b_bytes, b_tokens in shard:
                decode(sub)
                nbytes += b_bytes
                tokens += b_tokens
                count += 1
        conn.send((time.perf_counter() - t0, nbytes, tokens, count))
    conn.close()


def cpu_baseline_pool(batch, seconds: float, procs: int, rate_1: float) -> dict:
    """The oracle as it stands, run by ``procs`` processes at once, each
    decoding its share of the batch's sequences (shares balanced by bytes),
    the whole batch ``rounds`` times so that the pool works about
    ``seconds``.  The value is all processes' algorithmic bytes over the
    wall time from the start signal to the last result (host copies and
    process start-up outside it)."""
    import multiprocessing as mp

    from workloads import decode_bytes, extract_sequences

    w = batch.workload
    subs = []
    for b in range(len(batch.context_lens)):
        acct = decode_bytes(batch.context_lens[b:b + 1], w.num_q_heads, w.num_kv_heads,
                            w.head_dim, w.block_size, w.cache_dtype, w.q_dtype)
        subs.append((extract_sequences(batch, [b]), acct["total"], acct["tokens"]))
    total = sum(x[1] for x in subs)
    shards = [[] for _ in range(procs)]
    load = [0] * procs
    for item in sorted(subs, key=lambda x: -x[1]):  # largest first, to the lightest share
        i = int(np.argmin(load))
        shards[i].append(item)
        load[i] += item[1]
    rounds = max(1, int(np.ceil(seconds * rate_1 * 1e9 * procs / max(total, 1))))
    meta = {"block_size": w.block_size, "scale": batch.scale, "q_dtype": w.q_dtype,
            "cache_dtype": w.cache_dtype}
    ctx = mp.get_context("spawn")  # fresh interpreters: nothing of this process's GPU state
    workers = []
    for shard in shards:
        parent, child = ctx.Pipe()
        p = ctx.Process(target=_oracle_worker, args=(child,), daemon=True)
        p.start()
        parent.send((meta, shard))
        workers.append((p, parent))

    def collect(what, timeout_s):
        got = []
        for p, conn in workers:
            if not conn.poll(timeout_s):
                for q, _ in workers:
                    q.terminate()
                raise RuntimeError(f"CPU-baseline worker gave no {what} within {timeout_s}s "
                                   f"(alive: {p.is_alive()})")
            got.append(conn.recv())
        return got

    assert all(r == "ready" for r in collect("ready signal", 300))
    t0 = time.perf_counter()
    for _, conn in workers:
        conn.send(rounds)
    results = collect("result", max(600, 20 * seconds))
    wall = time.perf_counter() - t0
    for p, _ in workers:
        p.join(timeout=30)
    nbytes = sum(r[1] for r in results)
    tokens = sum(r[2] for r in results)
    count = sum(r[3] for r in results)
    return {"value": nbytes / wall / 1e9, "unit": "GB/s", "cores": procs, "kind": "oracle",
            "tokens_per_s": tokens / wall, "seconds": round(wall, 2),
            "speedup_vs_one_process": round(nbytes / wall / 1e9 / rate_1, 2),
            "sample": f"process pool of {procs} (one BLAS thread each; "
                      f"{len(os.sched_getaffinity(0))} cores in this process's affinity), "
                      f"{count} sequence decodes = {rounds} passes over all "
                      f"{len(subs)} sequences of the batch ({tokens} context tokens), "
                      f"fp64 numpy oracle"}


def bench_step(args) -> int:
    """The hot path's step on one batch resident in HBM: ``value`` from K
    back-to-back steps (eager or graph-replayed, the faster); per-kernel times (roofline) from single launches
    each preceded by the cache flush."""
    import torch

    import paged_kv_cache_253_amd as pk
    from workloads import WORKLOADS, decode_bytes, make_batch, write_bytes

    w = with_cache_dtype(WORKLOADS[args.workload], args.cache_dtype)
    if w is None:
        return 2
    dev = "cuda"
    t_gen = time.perf_counter()
    batch = make_batch(w, device=dev)
    if args.equal_lengths:  # same token total, n equal contexts (segment-count studies)
        n = args.equal_lengths
        total = int(batch.context_lens.sum())
        batch = make_batch(w, device=dev, lens=np.full(n, max(1, total // n), np.int32))
    if args.unshare:
        from workloads import unshare
        batch = unshare(batch)
    if args.contiguous_blocks:  # block-layout studies: the unpaged order, same data
        from workloads import contiguous_layout, unshare
        batch = contiguous_layout(unshare(batch))
    torch.cuda.synchronize()
    log(f"[bench] workload {w.index} {w.name}{' (unshared)' if args.unshare else ''}"
        f"{' (blocks in sequence order)' if args.contiguous_blocks else ''}: "
        f"{len(batch.context_lens)} seqs, "
        f"{int(batch.context_lens.sum())} tokens, pool {batch.num_blocks} blocks "
        f"(generated in {time.perf_counter() - t_gen:.1f}s)")

    part = args.partition
    if part is None:
        part = w.partition_size or pk.default_partition_size(batch.max_context_len)
    bt = torch.from_numpy(batch.block_tables).to(dev)
    cl = torch.from_numpy(batch.context_lens).to(dev)
    slots = torch.from_numpy(batch.slot_mapping).to(dev)
    out = torch.empty_like(batch.q)
    s, hq, d = batch.q.shape
    ws = None
    if part:
        ws = pk.new_workspace(s, hq, w.num_kv_heads, d, batch.max_context_len, part, dev)

    one_call = not args.separate_append  # the step calls pa_decode_append
    merge_launch = part not in (0, pk.PARTITION_AUTO_MERGED)  # a pa_decode_reduce per step
    new_rows = dict(k_new=batch.k_new, v_new=batch.v_new)

    def write():
        pk.kv_cache_write(batch.k_new, batch.v_new, batch.k_pool, batch.v_pool, slots,
                          batch.k_scale, batch.v_scale, cache_dtype=w.cache_dtype)

    def attend(rows):
        """pa_decode_append (rows given) or pa_decode, without the merge."""
        if part:
            pk.decode_partitions(batch.q, batch.k_pool, batch.v_pool, bt, cl,
                                 batch.max_context_len, part, batch.scale, batch.k_scale,
                                 batch.v_scale, ws, out=out, cache_dtype=w.cache_dtype, **rows)
        else:
            pk.decode(batch.q, batch.k_pool, batch.v_pool, bt, cl, batch.max_context_len,
                      batch.scale, batch.k_scale, batch.v_scale, 0, out=out,
                      cache_dtype=w.cache_dtype, **rows)

    def reduce():
        pk.decode_reduce(out, ws, cl, batch.max_context_len, part, w.num_kv_heads)

    def step():
        if not one_call:
            write()
        attend(new_rows if one_call else {})
        if merge_launch:
            reduce()

    # ---- the step: K steps back to back, timed as a whole ----------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps (partition {part})")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    eager_ms_per_step = start.elapsed_time(end) / args.steps
    graph_ms_per_step = None
    if not args.eager:
        # The same step captured once in a HIP graph and replayed K times
        # (a fixed launch sequence on one stream, no host launch gaps; on
        # ROCm each replay adds a few microseconds of its own).  The replayed
        # result must match the eager step bit for bit.
        ref = out.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(out.view(torch.int16), ref.view(torch.int16)):
            raise RuntimeError("graph replay differs from the eager step")
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms_per_step = g0.elapsed_time(g1) / args.steps
    # the step time is that of the faster launch mode; both are reported
    graph_faster = graph_ms_per_step is not None and graph_ms_per_step < eager_ms_per_step
    ms_per_step = graph_ms_per_step if graph_faster else eager_ms_per_step
    launch = "hip graph replay" if graph_faster else "eager, back to back"
    log(f"[bench] step {ms_per_step * 1e3:.1f} us ({launch}; eager {eager_ms_per_step * 1e3:.1f} us"
        + (f", graph replay {graph_ms_per_step * 1e3:.1f} us)" if graph_ms_per_step is not None else ")"))

    # ---- each kernel alone, one launch per flush -------------------------
    flush = Flush(torch, pk, args.flush, dev)
    reps = max(args.steps, 30)
    t_write = timed_launches(torch, write, reps, flush)
    t_decode = timed_launches(torch, lambda: attend({}), reps, flush)
    t_append = timed_launches(torch, lambda: attend(new_rows), reps, flush) if one_call else None
    t_reduce = timed_launches(torch, reduce, reps, flush) if merge_launch else None
    abuf = torch.ones(ATTAINABLE_BYTES, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    t_read = timed_launches(torch, lambda: pk.stream_read(abuf, sink), reps, flush)
    del abuf
    warm = None
    if args.warm:  # back to back, no flush (a separate figure; not the roofline's)
        for _ in range(3):
            attend({})
        t_warm = timed_launches(torch, lambda: attend({}), reps, lambda: None)
        warm = dist_us(t_warm)

    dec = decode_bytes(batch.context_lens, w.num_q_heads, w.num_kv_heads, w.head_dim,
                       w.block_size, w.cache_dtype, w.q_dtype)
    wr = write_bytes(len(batch.context_lens), w.num_kv_heads, w.head_dim, w.src_dtype,
                     w.cache_dtype)
    step_bytes = dec["total"] + wr
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    decode_ms = float(t_decode.mean())
    achieved = dec["total"] / (decode_ms * 1e-3) / 1e9
    attainable = ATTAINABLE_BYTES / (float(np.median(t_read)) * 1e-3) / 1e9
    in_step_ms = float((t_append if one_call else t_decode).mean())
    in_step_bytes = dec["total"] + (wr if one_call else 0)
    in_step_gbs = in_step_bytes / (in_step_ms * 1e-3) / 1e9
    log(f"[bench] decode {decode_ms * 1e3:.1f} us = {achieved:.0f} GB/s = "
        f"{100 * achieved / PEAK_HBM_GBS:.1f}% of peak, {100 * achieved / attainable:.1f}% of the "
        f"{attainable:.0f} GB/s streaming read; "
        + (f"appending decode {in_step_ms * 1e3:.1f} us = {100 * in_step_gbs / PEAK_HBM_GBS:.1f}%; "
           if one_call else "")
        + f"write {t_write.mean() * 1e3:.1f} us"
        + (f", reduce {t_reduce.mean() * 1e3:.1f} us" if merge_launch else ""))

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 1 GiB device copies done")

    # the counters were taken on the drawn batch only
    traffic = (None if (args.equal_lengths or args.unshare or args.contiguous_blocks)
               else measured_traffic(w.name, part, 1))
    split = {0: "unsplit", -1: "balanced", -2: "balanced, merged in the decode launch"}.get(
        part, f"{part}-token partitions")
    result = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) and context tokens/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.cache_dtype,
        "data": "synthetic",
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "context_tokens_per_s": round(dec["tokens"] / (ms_per_step * 1e-3), 1),
        "config": {"workload": w.name + ("-unshared" if args.unshare else "")
                   + (f"-equal-lengths-{args.equal_lengths}" if args.equal_lengths else "")
                   + ("-contiguous-blocks" if args.contiguous_blocks else ""),
                   "num_seqs": len(batch.context_lens),
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size,
                   "kv_dtype": w.cache_dtype, "context_tokens": dec["tokens"],
                   "partition_size": part, "split": split,
                   "step": ("decode_append" if one_call else "kv_cache_write + decode")
                   + (" + reduce" if merge_launch else ""),
                   "launch": launch,
                   "eager_ms_per_step": round(eager_ms_per_step, 4),
                   "graph_ms_per_step": (round(graph_ms_per_step, 4)
                                         if graph_ms_per_step is not None else None)},
        # each kernel alone: one launch per flush, HIP events around it
        "kernels_us": {"flush": flush.describe(),
                       "kv_cache_write": dist_us(t_write),
                       "decode": dist_us(t_decode),
                       "decode_append": dist_us(t_append) if one_call else None,
                       "decode_reduce": dist_us(t_reduce) if merge_launch else None,
                       "stream_read_2GiB": dist_us(t_read),
                       "decode_warm_back_to_back": warm},
        "roofline": {"bound": "hbm", "kernel": "pa_decode", "achieved": round(achieved, 1),
                     "launch_us": round(decode_ms * 1e3, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes": dec["total"],
                     # what a kernel that only streams reads attains on this device
                     "attainable": round(attainable, 1),
                     "frac_of_attainable": round(achieved / attainable, 4),
                     # the same figures for the decode launch the steps make:
                     # pa_decode_append, the append inside the decode launch
                     # where the kernels allow (else the plain decode)
                     "in_step": {"kernel": "pa_decode_append" if one_call else "pa_decode",
                                 "launch_us": round(in_step_ms * 1e3, 2),
                                 "achieved": round(in_step_gbs, 1),
                                 "frac": round(in_step_gbs / PEAK_HBM_GBS, 4),
                                 "frac_of_attainable": round(in_step_gbs / attainable, 4),
                                 "algorithmic_bytes": in_step_bytes}},
    }
    if not args.no_cpu:
        log(f"[bench] timing the CPU oracle for about {args.cpu_seconds:.0f}s")
        one = cpu_baseline(batch, args.cpu_seconds)
        result["cpu_baseline"] = one
        procs = host_cores()
        if procs > 1 and not args.no_pool:
            log(f"[bench] timing the CPU oracle in a pool of {procs} processes")
            result["cpu_baseline_all_cores"] = cpu_baseline_pool(batch, args.cpu_seconds / 2,
                                                                 procs, one["value"])
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--partition", type=int, default=None,
                    help="context split: tokens per partition, 0 unsplit, -1 balanced with "
                         "a separate merge launch, -2 balanced merged in the decode launch "
                         "(default: the workload's own, else the library default, -1)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-pool", action="store_true",
                    help="skip the CPU baseline's process-pool leg")
    ap.add_argument("--flush", choices=["copy+read", "copy", "none"], default="copy+read",
                    help="what runs before each per-kernel timed launch")
    ap.add_argument("--warm", action="store_true",
                    help="also time the decode back to back without flushes")
    ap.add_argument("--unshare", action="store_true",
                    help="give every sequence private copies of the blocks it shares "
                         "(the shared-prefix workload without sharing)")
    ap.add_argument("--eager", action="store_true",
                    help="time the step eagerly only (no HIP graph capture and replay)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--op", choices=["step", "copy", "prefill", "swap"], default="step",
                    help="step: append + decode (+ merge); copy: a copy-on-write burst "
                         "of pa_copy_blocks on the workload's pool; prefill: several query "
                         "tokens per sequence (pa_prefill_chunk), see --case")
    ap.add_argument("--cache-dtype", choices=["fp8_e4m3", "fp8_e5m2", "int4"], default=None,
                    help="KV cache format in place of the workload's: the other FP8 format "
                         "for an FP8 workload, or INT4 (per-token scales, bf16 queries) for "
                         "any bf16 or FP8 workload")
    ap.add_argument("--separate-append", action="store_true",
                    help="step as pa_kv_cache_write + pa_decode (two launches) instead of "
                         "pa_decode_append")
    ap.add_argument("--equal-lengths", type=int, default=0, metavar="N",
                    help="replace the workload's drawn lengths by N equal contexts with the "
                         "same token total (how the decode's time depends on the number of "
                         "runs, not on the bytes)")
    ap.add_argument("--contiguous-blocks", action="store_true",
                    help="renumber the batch's blocks so each sequence's are consecutive, in "
                         "sequence order (the unpaged layout, same data): what the scattered "
                         "physical blocks cost the decode")
    ap.add_argument("--case", default="spec-verify-8b",
                    help="prefill shape: spec-verify-8b, chunked-prefill-8b or "
                         "chunked-prefill-8b-fp8")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on one GPU; it has no multi-GPU path)", file=sys.stderr)
        return 2
    if args.op == "copy":
        return bench_copy(args)
    if args.op == "prefill":
        return bench_prefill(args)
    if args.op == "swap":
        return bench_swap(args)

    return bench_step(args)


if __name__ == "__main__":
    sys.exit(main())
