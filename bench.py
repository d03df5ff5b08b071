"""Benchmark of the paged-KV decode hot path on one MI355X.

Default workload: the full decode step -- 512 sequences, cached lengths
U{64..4096}, 32 layers, bf16, Hq=32, Hkv=8, D=128, block 16. One step = for
every layer one paged_decode_attention_append launch: each sequence's new
token K/V stored at the slot its position translates to (slot mapping and
write), split decode attention (balanced pieces, 1024-position slots) and the
log-sum-exp merge. ``--write separate`` runs paged_slot_mapping once and
paged_kv_write per layer before a paged_decode_attention_merged launch;
``--merge two-launch`` the split call and paged_attention_reduce (as the
single-layer workloads do by default).
Inputs are resident in HBM before timing starts.

Multi-token workloads (``--workload spec_verify_bf16`` / ``mixed_prefill_bf16``):
one step is one paged_varlen_attention call (balanced split kernel over
(sequence, column group) units, then the merge over query rows) on one layer,
with L2/MALL evicted before it.

Block moves: ``--workload cow_fork_bf16`` times paged_kv_copy_blocks over
all 32 layers of a parallel-sampling fork (128 prompts x 4 branches, one copy
per forked branch whose prompt ends in a partly filled block);
``--workload swap_bf16`` times paged_kv_swap_out / paged_kv_swap_in of 8
sequences' blocks of the 32-layer decode step through pinned host memory.
Each is set beside a plain contiguous copy of the same bytes (device copy,
or torch's host copies) measured in the same run.

Prints one JSON line. `value` is KV-read GB/s over the whole step: the
algorithmic bytes every layer must read (2 * Hkv * D * 2 B per live
(sequence, position)) divided by the step time. The `roofline` object is for
the decode kernel alone, timed with HIP events on the stream it runs on.
The `cpu_baseline` object times the fp64 CPU oracle on a bounded sample of the
same workload (rank 0, one GPU only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode KV-read HBM GB/s (% of MI355X peak) + decoded seqs·tokens/s"
HBM_PEAK_GBS = 8000.0
DECODE_SOURCES = ["paged_kv_cache_113_amd/csrc/decode_fast.hip",
                  "paged_kv_cache_113_amd/csrc/device.h",
                  "paged_kv_cache_113_amd/csrc/mfma_tile.h",
                  "paged_kv_cache_113_amd/csrc/varlen.h"]
VARLEN_SOURCES = DECODE_SOURCES + ["paged_kv_cache_113_amd/csrc/prefill.hip",
                                   "paged_kv_cache_113_amd/csrc/decode_generic.hip"]
MOVE_SOURCES = ["paged_kv_cache_113_amd/csrc/block_ops.hip",
                "paged_kv_cache_113_amd/csrc/device.h"]


def kernel_source_hash(sources=DECODE_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kernel: str = "decode_split", sources=DECODE_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


PROBE_LIB = os.path.join(ROOT, "paged_kv_cache_113_amd", "libpkvprobe.so")
_probe = None


def probe_lib():
    """The bench-only read-stream probe library (built beside libpagedkv.so)."""
    global _probe
    if _probe is None:
        import ctypes
        if not os.path.exists(PROBE_LIB):
            raise ImportError(f"{PROBE_LIB} is missing: build with python __graft_entry__.py")
        lib = ctypes.CDLL(PROBE_LIB)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.pkvprobe_read_stream.restype = I32
        lib.pkvprobe_read_stream.argtypes = [P, P, I64, P, I64, I32, I32, I32, P, P]
        _probe = lib
    return _probe


def run_read_probe(k, v, order, heads, tiles_per_head, wg_per_cu, sink):
    import ctypes
    import torch
    nbytes = k.numel() * k.element_size()
    assert v.numel() * v.element_size() == nbytes and order.dtype == torch.int32
    rc = probe_lib().pkvprobe_read_stream(
        ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()), nbytes,
        ctypes.c_void_p(order.data_ptr()), order.numel(), heads, tiles_per_head, wg_per_cu,
        ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"pkvprobe_read_stream failed: {rc}")


def read_probe(dev, nbytes, heads, tiles_per_head, wg_per_cu, reps: int = 5):
    """Read rate of the split decode kernel's access pattern without its
    arithmetic (the bench-only probe library): nbytes of K and V read as
    whole blocks of `heads` side-by-side KV-head slabs (tiles_per_head 4 KiB
    tiles each), distinct blocks in a seeded shuffled order over pools of at
    least 2 GiB each, neighbouring waves reading the slabs of one block, the
    kernel's launch shape, load width, loads in flight and non-temporal
    hint. Median GB/s over ``reps`` calls."""
    import torch
    block = 4096 * heads * tiles_per_head
    n = max(1, int(nbytes // (2 * block)))
    pool_blocks = max(n, (2 << 30) // block)
    k = torch.empty(pool_blocks * block, dtype=torch.uint8, device=dev)
    v = torch.empty_like(k)
    k.fill_(1)
    v.fill_(2)
    order = torch.from_numpy(
        np.random.default_rng(7).permutation(pool_blocks)[:n].astype(np.int32)).to(dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(2):
        run_read_probe(k, v, order, heads, tiles_per_head, wg_per_cu, sink)
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        run_read_probe(k, v, order, heads, tiles_per_head, wg_per_cu, sink)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del k, v, order, sink
    torch.cuda.empty_cache()
    return 2.0 * block * n / (float(np.median(ts)) / 1e3) / 1e9


def kv_bytes(batch, lens) -> float:
    e = {"f32": 4, "f16": 2, "bf16": 2}[batch.dtype]
    return float(np.sum(lens, dtype=np.int64)) * 2 * batch.num_kv_heads * batch.head_size * e


def make_batch(workload, block_size=None):
    import workloads as W
    if block_size is None:
        return W.CASES[workload]()
    return W.CASES[workload](block_size=block_size)


def default_partition(workload):
    """Split size per workload: it sizes the partial slots (max_partitions =
    ceil(max ctx / P)); smaller P leaves the balanced split more freedom."""
    return {"decode_step_bf16": 1024, "long_split_bf16": 1024, "mha_fp16": 256,
            "gqa_shared_bf16": 1024, "tiny": 0, "spec_verify_bf16": 0,
            "mixed_prefill_bf16": 0}[workload]


VARLEN = ("spec_verify_bf16", "mixed_prefill_bf16")
BLOCK_MOVES = ("cow_fork_bf16", "swap_bf16")
HOST_ONLY = ("prefix_cache",)
PCIE_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction


def _events_ms(fn, reps, flush=None):
    """Mean and spread of fn's device time over ``reps`` runs (HIP events on
    torch's current stream), with an optional cache-evicting read before each."""
    import torch
    xs = []
    for _ in range(reps):
        if flush is not None:
            flush.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        xs.append(e0.elapsed_time(e1))
    return float(np.mean(xs)), float(np.percentile(xs, 10)), float(np.percentile(xs, 90))


def bench_prefix_cache(args):
    """Host-only: admissions through the library's cached block pool (hash
    the full blocks, longest cached prefix, touch, fresh blocks, cache the
    new full blocks) for 512 requests, cold and then warm after releasing
    them all; the oracle's pool timed on the same requests."""
    import paged_kv_cache_113_amd as pkv
    import workloads as W
    reqs = W.prefix_requests()
    B = 16
    need = sum(-(-len(t) // B) for t in reqs)
    n_blocks = int(math.ceil(1.1 * need))
    toks_total = int(sum(len(t) for t in reqs))
    blocks_full = int(sum(len(t) // B for t in reqs))

    def run(make_pool, admit, cache, release):
        pool = make_pool()
        times, hits = [], []
        for phase in range(2):
            tables = []
            t0 = time.perf_counter()
            cached = 0
            for t in reqs:
                table, c = admit(pool, t)
                cache(pool, table, t)
                tables.append(table)
                cached += c
            times.append(time.perf_counter() - t0)
            hits.append(cached)
            for table in tables:
                release(pool, table)
        return times, hits

    lib_t, lib_h = run(lambda: pkv.BlockPool(n_blocks, B),
                       lambda p, t: p.admit(t), lambda p, tb, t: p.cache_full_blocks(tb, t),
                       lambda p, tb: p.release(tb))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.prefix_cache as OP
        ora_t, ora_h = run(lambda: OP.CachedBlockPool(n_blocks, B),
                           lambda p, t: p.admit(t.tolist()),
                           lambda p, tb, t: p.cache_full_blocks(tb, t.tolist()),
                           lambda p, tb: p.release(tb))
        assert ora_h == lib_h, (ora_h, lib_h)
        cpu = {"value": round(toks_total * 2 / sum(ora_t), 1), "unit": "tokens/s", "cores": 1,
               "kind": "oracle",
               "sample": f"the same 512 requests, cold then warm, {sum(ora_t):.1f} s "
                         "(hashlib SHA-256, Python pool)"}
    # each block hashes a 96-byte message (parent hash + 16 int32 tokens) in
    # two 64-byte compression blocks, on both admission and caching
    value = toks_total * 2 / sum(lib_t)
    line = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 0,
            "steps": 2, "warmup": 0, "ms_per_step": round(sum(lib_t) / 2 * 1e3, 3),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
            "data": "synthetic",
            "config": {"workload": "prefix_cache", "requests": len(reqs), "block_size": B,
                       "pool_blocks": n_blocks, "tokens": toks_total, "full_blocks": blocks_full,
                       "shared_prompt_tokens": 512},
            "phases_ms": {"cold": round(lib_t[0] * 1e3, 3), "warm": round(lib_t[1] * 1e3, 3)},
            "cached_tokens": {"cold": lib_h[0], "warm": lib_h[1]},
            "blocks_hashed_per_s": round(blocks_full * 4 / sum(lib_t), 1),
            "roofline": {"bound": "host", "achieved": round(value, 1), "peak": None,
                         "unit": "tokens/s", "frac": None, "traffic": None,
                         "kernel": "pkv_pool_admit + pkv_pool_cache_full_blocks (one host thread,"
                                   " Python call overhead included)"},
            "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


def bench_block_moves(args):
    import torch
    import paged_kv_cache_113_amd as pkv
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps, warm = args.steps, args.warmup
    if args.workload == "cow_fork_bf16":
        b = W.cow_fork_bf16()
    else:
        b = W.decode_step_bf16()
    L = b.num_layers
    t0 = time.perf_counter()
    ks, vs = [], []
    for l in range(L):
        t = W.layer_tensors(b, layer=l, device=dev, poison=False)
        ks.append(t["k_cache"])
        vs.append(t["v_cache"])
        del t
    torch.cuda.synchronize()
    print(f"[bench] {args.workload}: {L} layers x {b.num_blocks} blocks generated in "
          f"{time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    slab = b.num_kv_heads * b.block_size * b.head_size * 2
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    pools = pkv.PoolSet(ks, vs)     # checked once: the timed calls only launch
    config = {"workload": args.workload, "layers": L, "num_kv_heads": b.num_kv_heads,
              "block_size": b.block_size, "head_size": b.head_size,
              "slab_bytes": slab, "blocks_per_layer": b.num_blocks}
    line = {"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warm,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": b.dtype,
            "data": "synthetic", "cpu_baseline": None}
    if args.workload == "cow_fork_bf16":
        pairs = torch.as_tensor(b.copy_pairs, dtype=torch.int64, device=dev)
        n = int(pairs.shape[0])
        run = lambda: pkv.paged_kv_copy_blocks(pools, None, pairs)   # noqa: E731
        for _ in range(warm):
            run()
        ms, p10, p90 = _events_ms(run, steps, flush)
        moved = 2.0 * n * L * 2 * slab               # K and V, read + write, per pair
        # a source shared by several pairs (the branches of one prompt) needs
        # reading once: the algorithmic bytes count it once
        n_src = len(set(int(x) for x in b.copy_pairs[:, 0]))
        unique = float(n_src + n) * L * 2 * slab
        # the same bytes as one contiguous device copy
        a = torch.empty(n * L * 2 * slab // 2, dtype=torch.bfloat16, device=dev)
        c = torch.empty_like(a)
        for _ in range(warm):
            c.copy_(a)
        cms = _events_ms(lambda: c.copy_(a), steps, flush)[0]
        del a, c
        achieved = unique / (ms / 1e3) / 1e9
        config.update({"pairs": n, "distinct_sources": n_src, "branches": b.branches,
                       "prompts": len(b.prompt_lens)})
        line.update({
            "value": round(achieved, 2), "ms_per_step": round(ms, 4), "config": config,
            "kernels_ms": {"copy_blocks_avg": round(ms, 4), "copy_blocks_p10": round(p10, 4),
                           "copy_blocks_p90": round(p90, 4),
                           "contiguous_copy_same_bytes": round(cms, 4)},
            "blocks_per_s": round(n * L / (ms / 1e3), 1),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic_for(args.workload, "move_blocks", MOVE_SOURCES),
                         "kernel": "move_blocks_kernel<16, copy>",
                         "bytes_per_launch": unique, "logical_bytes_per_launch": moved,
                         "logical_gbs": round(moved / (ms / 1e3) / 1e9, 2),
                         "contiguous_copy_gbs": round(moved / (cms / 1e3) / 1e9, 2)}})
    else:
        rng = np.random.default_rng(17)
        victims = np.sort(rng.choice(b.num_seqs, 8, replace=False))
        ids = [int(x) for s in victims for x in b.block_table[s] if x >= 0]
        keep = set(int(x) for s in range(b.num_seqs) if s not in set(victims.tolist())
                   for x in b.block_table[s] if x >= 0)
        free = np.array([x for x in range(b.num_blocks) if x not in keep], np.int64)
        fresh = rng.permutation(free)[:len(ids)]
        n = len(ids)
        ids_t = torch.as_tensor(ids, dtype=torch.int64, device=dev)
        fresh_t = torch.as_tensor(fresh, dtype=torch.int64, device=dev)
        buf = torch.empty((L, 2, n, b.num_kv_heads, b.block_size, b.head_size),
                          dtype=torch.bfloat16, pin_memory=True)
        out_fn = lambda: pkv.paged_kv_swap_out(buf, pools, None, ids_t)   # noqa: E731
        in_fn = lambda: pkv.paged_kv_swap_in(buf, pools, None, fresh_t)   # noqa: E731
        for _ in range(warm):
            out_fn()
            in_fn()
        o_ms, o10, o90 = _events_ms(out_fn, steps)
        i_ms, i10, i90 = _events_ms(in_fn, steps)
        moved = float(n) * L * 2 * slab
        d = torch.empty(buf.shape, dtype=torch.bfloat16, device=dev)
        for _ in range(warm):
            buf.copy_(d, non_blocking=True)
            d.copy_(buf, non_blocking=True)
        d2h = _events_ms(lambda: buf.copy_(d, non_blocking=True), steps)[0]
        h2d = _events_ms(lambda: d.copy_(buf, non_blocking=True), steps)[0]
        del d
        out_gbs = moved / (o_ms / 1e3) / 1e9
        in_gbs = moved / (i_ms / 1e3) / 1e9
        config.update({"swapped_sequences": int(len(victims)), "blocks": n,
                       "tokens": int(b.context_lens[victims].sum())})
        line.update({
            "value": round(moved * 2 / ((o_ms + i_ms) / 1e3) / 1e9, 2),
            "ms_per_step": round(o_ms + i_ms, 4), "config": config,
            "kernels_ms": {"swap_out_avg": round(o_ms, 4), "swap_out_p10": round(o10, 4),
                           "swap_out_p90": round(o90, 4), "swap_in_avg": round(i_ms, 4),
                           "swap_in_p10": round(i10, 4), "swap_in_p90": round(i90, 4),
                           "torch_d2h_same_bytes": round(d2h, 4),
                           "torch_h2d_same_bytes": round(h2d, 4)},
            "roofline": {"bound": "pcie", "achieved": round(out_gbs, 2), "peak": PCIE_PEAK_GBS,
                         "unit": "GB/s", "frac": round(out_gbs / PCIE_PEAK_GBS, 4),
                         "traffic": None, "kernel": "move_blocks_kernel<16, swap out>",
                         "bytes_per_launch": moved,
                         "swap_in_gbs": round(in_gbs, 2),
                         "swap_in_frac": round(in_gbs / PCIE_PEAK_GBS, 4),
                         "torch_d2h_gbs": round(moved / (d2h / 1e3) / 1e9, 2),
                         "torch_h2d_gbs": round(moved / (h2d / 1e3) / 1e9, 2)}})
    line["pct_of_peak"] = round(100.0 * line["roofline"]["frac"], 2)
    print(json.dumps(line), flush=True)


def block_utilisation(batch) -> float:
    """Live positions over the slots of the distinct blocks the tables hold
    (nxmr.cn article, section 5.2: utilisation = live tokens / (blocks x B));
    a block shared by several sequences counts once, its positions once."""
    B = batch.block_size
    live = {}
    for s, n in enumerate(batch.context_lens):
        n = int(n)
        for b in range((n + B - 1) // B):
            blk = int(batch.block_table[s, b])
            live[blk] = max(live.get(blk, 0), min(B, n - b * B))
    return round(sum(live.values()) / (len(live) * B), 4) if live else 0.0


def visible_pairs(batch) -> np.ndarray:
    """Per query row, how many positions it attends (causal, new tokens at the
    end of each context): a workload statistic for the flop count."""
    ctx = batch.context_lens.astype(np.int64)
    q = batch.query_lens.astype(np.int64)
    out = []
    for s in range(batch.num_seqs):
        out.append(ctx[s] - q[s] + 1 + np.arange(q[s], dtype=np.int64))
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def visible_pairs_of(batch, s) -> int:
    c, q = int(batch.context_lens[s]), int(batch.query_lens[s])
    return q * (c - q) + q * (q + 1) // 2


def host_topology() -> dict:
    """Logical CPUs (nproc), the CPUs this process may run on, physical cores
    and sockets (from /proc/cpuinfo, or lscpu when present), and the thread
    share the job is given (OMP_NUM_THREADS when set)."""
    import shutil
    import subprocess
    info = {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "physical_cores": None, "sockets": None, "model": None,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}
    try:
        cores, sockets, phys = set(), set(), None
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "physical id":
                    phys = val
                    sockets.add(val)
                elif key == "core id":
                    cores.add((phys, val))
                elif key == "model name" and info["model"] is None:
                    info["model"] = val
        if cores:
            info["physical_cores"] = len(cores)
        if sockets:
            info["sockets"] = len(sockets)
    except OSError:
        pass
    if shutil.which("lscpu"):
        try:
            out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
            kv = {a.strip(): b.strip() for a, _, b in
                  (line.partition(":") for line in out.splitlines())}
            per = kv.get("Core(s) per socket")
            sk = kv.get("Socket(s)")
            if per and sk and per.isdigit() and sk.isdigit():
                info["physical_cores"] = int(per) * int(sk)
                info["sockets"] = int(sk)
        except (OSError, subprocess.SubprocessError):
            pass
    return info


def cpu_baseline(batch, th, target_s: float, threads: int, topo: dict):
    """Time the fp64 oracle on layer 0 of the workload (post-write pools made
    by the oracle's own scatter), median of 3 runs per leg: all sequences with
    ``threads`` workers (the job's thread share), and one worker on a prefix of
    a seeded sequence order sized to about target_s / 6 per run."""
    import oracle
    k = oracle._raw(th["k_cache"], batch.dtype)
    v = oracle._raw(th["v_cache"], batch.dtype)
    if batch.positions is not None:
        slots = oracle.allocator.slot_mapping(
            [r[r >= 0].tolist() for r in batch.block_table], batch.positions.tolist(),
            batch.block_size)
        k = oracle.scatter.scatter(k, oracle._raw(th["k_new"], batch.dtype), slots)
        v = oracle.scatter.scatter(v, oracle._raw(th["v_new"], batch.dtype), slots)
    scale = float(np.float32(1.0 / math.sqrt(batch.head_size)))
    qsl = batch.query_start_loc

    def run(seqs, nthreads):
        if batch.query_lens is None:
            t0 = time.perf_counter()
            oracle.attention(th["q"], k, v, batch.block_table, batch.context_lens, scale,
                             batch.dtype, seqs=seqs, threads=nthreads)
            return time.perf_counter() - t0
        rows = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in seqs])
        ql = np.array([qsl[s + 1] - qsl[s] for s in seqs], np.int64)
        sub_qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        sub_q = th["q"][rows]
        t0 = time.perf_counter()
        oracle.attention_varlen(sub_q, k, v, batch.block_table[seqs], sub_qsl,
                                batch.context_lens[seqs], scale, batch.dtype, threads=nthreads)
        return time.perf_counter() - t0

    everything = np.arange(batch.num_seqs, dtype=np.int32)
    all_runs = [run(everything, threads) for _ in range(3)]
    all_s = float(np.median(all_runs))
    all_rate = kv_bytes(batch, batch.context_lens) / all_s
    order = np.random.default_rng(7).permutation(batch.num_seqs).astype(np.int32)
    # work per sequence: the positions its query rows attend
    work = batch.context_lens.astype(np.int64) if batch.query_lens is None else np.array(
        [visible_pairs_of(batch, s) for s in range(batch.num_seqs)], np.int64)
    probe = order[:2]
    dt = run(probe, 1)
    per_pos = dt / max(1, int(work[probe].sum()))
    csum = np.cumsum(work[order])
    n1 = int(max(1, min(len(order), np.searchsorted(csum, (target_s / 6) / per_pos) + 1)))
    one_runs = [run(order[:n1], 1) for _ in range(3)]
    dt1 = float(np.median(one_runs))
    one_rate = kv_bytes(batch, batch.context_lens[order[:n1]]) / dt1
    pos = float(batch.context_lens.sum())
    return {"value": round(all_rate / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"layer 0 of the workload, all {batch.num_seqs} sequences "
                      f"({int(pos)} positions), median of 3 runs "
                      f"({', '.join(f'{x:.2f}' for x in all_runs)} s); fp64 gather + attention",
            "seq_tokens_per_s": round(pos / all_s, 1),
            "threads": threads,
            "host": topo,
            "single_thread": {"value": round(one_rate / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"{n1} sequences of layer 0, median of 3 runs "
                                        f"({', '.join(f'{x:.2f}' for x in one_runs)} s)"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 10 for the 32-layer decode step, 20 otherwise)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode_step_bf16",
                    choices=["decode_step_bf16", "mha_fp16", "gqa_shared_bf16",
                             "long_split_bf16", *VARLEN, *BLOCK_MOVES, *HOST_ONLY])
    ap.add_argument("--max-partitions", type=int, default=8,
                    help="multi-token workloads: pieces per query row at most")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None, help="decode step only (default 32)")
    ap.add_argument("--block-size", type=int, default=None,
                    help="positions per physical block (block-size study; the workloads "
                         "define 16, or 32 for the long split)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--merge", choices=["auto", "one-launch", "two-launch"], default="auto",
                    help="split decode and its merge: paged_decode_attention_merged (one launch) "
                         "or paged_decode_attention + paged_attention_reduce (two); auto takes "
                         "the faster on MI355X: one launch for the 32-layer decode step (most of "
                         "its sequences finish in one piece), two for the single-layer cases "
                         "(many pieces per sequence: the in-kernel merge lengthens the kernel's "
                         "tail by about what the second launch costs)")
    ap.add_argument("--write", choices=["fused", "separate"], default="fused",
                    help="decode step with the merge in one launch: store the new tokens' K/V in "
                         "the same launch (paged_decode_attention_append) or with "
                         "paged_slot_mapping + paged_kv_write first")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured in a HIP graph (per-kernel times "
                         "still come from eager steps)")
    ap.add_argument("--no-probe", "--no-ceiling", dest="no_probe", action="store_true",
                    help="skip the read-stream probe")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    args.two_call = args.merge == "two-launch" or (
        args.merge == "auto" and args.workload != "decode_step_bf16")
    if args.steps is None:
        args.steps = 10 if args.workload == "decode_step_bf16" else 20

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(sequences and KV heads shard across GPUs with no communication)",
              file=sys.stderr)
        sys.exit(2)

    if args.workload in BLOCK_MOVES:
        bench_block_moves(args)
        return
    if args.workload in HOST_ONLY:
        bench_prefix_cache(args)
        return

    import torch
    import paged_kv_cache_113_amd as pkv
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    batch = make_batch(args.workload, args.block_size)
    if args.layers is not None:
        batch.num_layers = args.layers
    L = batch.num_layers
    P = default_partition(args.workload) if args.partition_size is None else args.partition_size
    mp = batch.max_partitions(P) if P > 0 else 1
    varlen = args.workload in VARLEN
    if varlen:
        mp = args.max_partitions
    scale = float(np.float32(1.0 / math.sqrt(batch.head_size)))
    print(f"[bench] workload {args.workload}: S={batch.num_seqs} layers={L} "
          f"blocks/layer={batch.num_blocks} P={P}", file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    layers = []
    cpu_host = None
    for l in range(L):
        t = W.layer_tensors(batch, layer=l, device=dev)
        if l == 0 and not args.no_cpu_baseline:
            cpu_host = {k: v.cpu() for k, v in t.items()}
        layers.append(t)
    torch.cuda.synchronize()
    print(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
          flush=True)

    table = torch.as_tensor(batch.block_table, device=dev)
    ctx = torch.as_tensor(batch.context_lens, device=dev)
    pos = torch.as_tensor(batch.positions, device=dev) if batch.positions is not None else None
    slots = torch.empty(batch.num_seqs, dtype=torch.int64, device=dev)
    outs = [torch.empty(batch.num_tokens, batch.num_heads, batch.head_size, device=dev)
            for _ in range(L)]
    qsl = torch.as_tensor(batch.query_start_loc, device=dev)
    if P > 0 or varlen:
        ws_shape = (batch.num_tokens, batch.num_heads, mp)
        ml = torch.empty(ws_shape, device=dev)
        es = torch.empty(ws_shape, device=dev)
        to = torch.empty(ws_shape + (batch.head_size,), device=dev)
    # arrival counters of the merged call: zeroed once, left zero by each call
    counters = torch.zeros(batch.num_seqs * batch.num_kv_heads, dtype=torch.int32, device=dev)
    flush = None
    if args.workload != "decode_step_bf16":
        # 1 GiB, written once here; each step only reads it, so the eviction
        # leaves no dirty lines to be written back inside the timed kernels
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    ev = {k: [] for k in ("decode", "reduce", "write")}

    def timed(name, record, fn):
        # HIP events on torch's current stream, which is the stream every
        # library call is enqueued on
        if name not in record:
            fn()
            return
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        ev[name].append((e0, e1))

    fused_write = pos is not None and P > 0 and not args.two_call and args.write == "fused"

    def step(record=()):
        if pos is not None and not fused_write:
            pkv.paged_slot_mapping(slots, table, pos, batch.block_size)
        for l, t in enumerate(layers):
            if fused_write:
                # the new token's K/V stored at its slot, attention and merge:
                # one launch per layer
                timed("decode", record, lambda: pkv.paged_decode_attention_append(
                    outs[l], t["q"], t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], table,
                    ctx, scale, P, mp, ml, es, to, counters))
                continue
            if pos is not None:
                timed("write", record, lambda: pkv.paged_kv_write(
                    t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], slots))
            if varlen:
                timed("decode", record, lambda: pkv.paged_varlen_attention(
                    outs[l], t["q"], t["k_cache"], t["v_cache"], table, qsl, ctx, scale, mp, ml,
                    es, to))
            elif P > 0 and not args.two_call:
                timed("decode", record, lambda: pkv.paged_decode_attention_merged(
                    outs[l], t["q"], t["k_cache"], t["v_cache"], table, ctx, scale, P, mp, ml,
                    es, to, counters))
            elif P > 0:
                timed("decode", record, lambda: pkv.paged_decode_attention(
                    None, t["q"], t["k_cache"], t["v_cache"], table, ctx, scale, P, mp, ml, es,
                    to))
                timed("reduce", record, lambda: pkv.paged_attention_reduce(
                    outs[l], ml, es, to, ctx, P))
            else:
                timed("decode", record, lambda: pkv.paged_decode_attention(
                    outs[l], t["q"], t["k_cache"], t["v_cache"], table, ctx, scale))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    if args.copy_probe:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b_ = torch.empty_like(a)
        for _ in range(5):
            b_.copy_(a)
        torch.cuda.synchronize()
        del a, b_

    graph = None
    if args.graph:
        # eager steps for the per-kernel times, then one step captured
        for _ in range(args.steps):
            step(("decode",))
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                step()
        torch.cuda.current_stream().wait_stream(side)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
    run_step = (lambda: graph.replay()) if graph is not None else (lambda: step(("decode",)))

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    if flush is None:
        for _ in range(args.steps):
            run_step()
        torch.cuda.synchronize()
        total_s = time.perf_counter() - t_start
    else:
        # single-layer workloads: evict L2/MALL before each step. The
        # evicting read is enqueued first and the step's own events are
        # recorded behind it, so the step's launches are already queued when
        # the GPU reaches them and the step time is device time, free of the
        # host's launch latency
        total_s = 0.0
        for _ in range(args.steps):
            flush.sum()
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record()
            run_step()
            s1.record()
            torch.cuda.synchronize()
            total_s += s0.elapsed_time(s1) / 1e3
    ms_per_step = total_s / args.steps * 1e3
    warm_ms = None
    if flush is not None:
        # secondary figure: the same steps back to back, caches left warm
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        w0.record()
        for _ in range(args.steps):
            run_step()
        w1.record()
        torch.cuda.synchronize()
        warm_ms = w0.elapsed_time(w1) / args.steps
    # the smaller kernels' own durations, from untimed steps (at least 10 calls)
    for _ in range(max(1, -(-10 // L))):
        step(("write", "reduce"))
    torch.cuda.synchronize()

    def avg_ms(name):
        xs = [a.elapsed_time(b) for a, b in ev[name]]
        return (float(np.mean(xs)), float(np.percentile(xs, 10)), float(np.percentile(xs, 90)),
                float(np.median(xs))) if xs else (0.0, 0.0, 0.0, 0.0)

    dec_ms, dec_p10, dec_p90, dec_med = avg_ms("decode")
    red_ms = avg_ms("reduce")[0]
    wr_ms = avg_ms("write")[0]
    logical_bytes = kv_bytes(batch, batch.context_lens)
    layer_bytes = logical_bytes
    if len(batch.sharers) > 1:
        # a shared prefix block is read once per KV head however many
        # sequences map it: algorithmic bytes count it once
        per_pos = logical_bytes / float(np.sum(batch.context_lens, dtype=np.int64))
        layer_bytes -= (len(batch.sharers) - 1) * len(batch.shared_blocks) * \
            batch.block_size * per_pos
    step_bytes = layer_bytes * L
    value = step_bytes / (ms_per_step / 1e3) / 1e9
    achieved = layer_bytes / (dec_ms / 1e3) / 1e9
    positions = float(np.sum(batch.context_lens, dtype=np.int64))
    traffic = traffic_for(args.workload, "paged_varlen_attention", VARLEN_SOURCES) if varlen \
        else traffic_for(args.workload)
    pairs = float(visible_pairs(batch).sum()) if varlen else positions
    flops = 4.0 * batch.num_heads * batch.head_size * pairs   # q.K and P.V, per layer

    probe = None
    if not args.no_probe:
        tph = max(1, batch.block_size * batch.head_size * 2 // 4096)
        probe = read_probe(dev, layer_bytes, batch.num_kv_heads, tph, 1)

    cpu = None
    if cpu_host is not None:
        # every CPU this process may run on, within the thread share the job
        # is given (OMP_NUM_THREADS, when the host sets one)
        topo = host_topology()
        threads = topo["affinity"]
        share = topo["omp_num_threads"]
        if share and share.isdigit() and int(share) > 0:
            threads = min(threads, int(share))
        print(f"[bench] cpu baseline: oracle, {threads} threads (nproc {topo['nproc']}, "
              f"affinity {topo['affinity']}, physical cores {topo['physical_cores']}, sockets "
              f"{topo['sockets']}), ~{args.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        cpu = cpu_baseline(batch, cpu_host, args.cpu_seconds, threads, topo)

    config = {"workload": args.workload, "num_seqs": batch.num_seqs, "layers": L,
              "num_heads": batch.num_heads, "num_kv_heads": batch.num_kv_heads,
              "head_size": batch.head_size, "block_size": batch.block_size,
              "context_lens": f"{int(batch.context_lens.min())}..{int(batch.context_lens.max())}"
                              f" mean {float(batch.context_lens.mean()):.1f}",
              "partition_size": P, "blocks_per_layer": batch.num_blocks,
              "block_utilisation": block_utilisation(batch)}
    if varlen:
        config.update({"num_tokens": batch.num_tokens, "max_partitions": mp,
                       "query_lens": f"{int(batch.query_lens.min())}..{int(batch.query_lens.max())}"
                                     f" total {batch.num_tokens}"})
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": batch.dtype, "data": "synthetic", "config": config,
        "launch": "hip graph replay" if args.graph else "eager",
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_tokens_per_s": round(positions * L / (ms_per_step / 1e3), 1),
        "query_pairs_per_s": round(pairs * L / (ms_per_step / 1e3), 1) if varlen else None,
        "query_tokens_per_s": round(batch.num_tokens * L / (ms_per_step / 1e3), 1)
        if varlen else None,
        "new_tokens_per_s": round(batch.num_seqs / (ms_per_step / 1e3), 1)
        if batch.positions is not None else None,
        "kernels_ms": {"decode_avg": round(dec_ms, 4), "decode_median": round(dec_med, 4),
                       "decode_p10": round(dec_p10, 4),
                       "decode_p90": round(dec_p90, 4), "reduce_avg": round(red_ms, 4),
                       "write_avg": round(wr_ms, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "paged_varlen_attention (split kernel, prefill kernel, merge)"
                     if varlen
                     else "decode_split_kernel" + (
                         "" if args.two_call else
                         " (paged_decode_attention_append: new tokens' K/V stored, pieces merged, "
                         "in the same launch)" if fused_write else
                         " (paged_decode_attention_merged: pieces merged in the same launch)")
                     if P > 0 else "decode_whole_kernel",
                     "bytes_per_launch": layer_bytes,
                     "logical_bytes_per_launch": logical_bytes,
                     "read_probe": None if probe is None else {
                         "gbs": round(probe, 2), "frac": round(achieved / probe, 4),
                         "probe": "bench-only read-stream probe over the kernel's bytes per "
                                  "launch, in its access pattern: whole blocks of Hkv "
                                  "side-by-side KV-head slabs, K and V, distinct blocks in a "
                                  "seeded shuffled order over >= 2 GiB pools, neighbouring "
                                  "waves on one block's slabs, the kernel's launch shape, "
                                  "non-temporal 16-byte loads, two tiles in flight"},
                     "mfma_view": {"flops_per_launch": flops,
                                   "achieved_tflops": round(flops / (dec_ms / 1e3) / 1e12, 2),
                                   "peak_tflops": 2500.0,
                                   "frac": round(flops / (dec_ms / 1e3) / 2.5e15, 4)}},
        "cpu_baseline": cpu,
    }
    if warm_ms is not None:
        line["warm_back_to_back"] = {"ms_per_step": round(warm_ms, 4),
                                     "gbs": round(step_bytes / (warm_ms / 1e3) / 1e9, 2)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
