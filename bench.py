"""Benchmark of the paged-KV decode hot path on one MI355X.

Workload (default): the Llama-3-8B attention shape at decode - 32 query / 8
KV heads, head size 128, bf16 values, 16-token blocks - for the eight-request
batch of the worked example on the clozo.ai page (lengths 128, 700, 1500,
300, 2900, 50, 4100, 900), blocks drawn from a shuffled 4,096-block pool.

One timed step is one decode step of the whole model's attention path:
  * host: the C++ allocator reserves one new token per sequence (lazy block
    allocation, copy-on-write pairs if any) and rebuilds the block tables;
  * the slot mapping / tables / lengths go to the device (pinned, async);
  * for each of the 32 layers (each with its own K/V pool, so the step reads
    1.4 GB and cannot be served from the 256 MB last-level cache):
    pa_copy_blocks (only if the allocator reported pairs), pa_cache_append of
    the new token's K/V, pa_decode.  The layer loop enqueues only kernel
    launches, so it is captured once as a HIP graph and replayed every step
    (--eager launches each call from Python instead).
Lengths grow by one token per step, as in real decoding; the KV bytes of
every step are counted exactly.

Reported: value = KV bytes read by pa_decode per second over the timed steps
(GB/s, whole step, all host work included; 10 warm-up and 100 timed steps by
default, with the median and p10/p90 of the per-step times).  roofline:
pa_decode alone, timed with HIP events around back-to-back launches (100
replays of a graph of the 32 layers' calls) at the batch's exact lengths,
against the 8 TB/s HBM peak; one launch is the whole call, its two kernels
included.  Beside it: the same calls on one pool (labelled MALL-warm: most
of that pool then sits in the last-level cache) and the bandwidth of a plain
1 GiB device copy on the same GPU.  cpu_baseline: the CPU oracle's paged
decode on the same batch (one layer), timed on this host's cores, plus
one-thread passes of this batch and of the tiny reference batch.
"""

from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode attention µs/step + KV-read GB/s (% of HBM peak), Llama-3-8B shape"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--kernel-reps", type=int, default=100,
                   help="graph replays (passes over the layer pools) for the kernel timing")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after the run, copy a MIB-MiB device buffer 4 times (a plain copy kernel "
                        "of known size, to scale the HBM byte counters of a profiler pass)")
    p.add_argument("--workload", default="llama3_8b_decode",
                   help="llama3_8b_decode (the default bench line), or serving_batch, "
                        "block_size_sweep_bs{8,16,32,128}, prefix_sharing_p{2056,2048}, "
                        "worked_batch_xN (the worked batch repeated N times): pa_decode "
                        "alone on that workload's batch (kernel leg only); llama3_8b_prefill, "
                        "llama3_8b_chunked_prefill_cN: pa_prefill alone on the worked batch; "
                        "swap_llama3_8b: pa_swap_blocks out to pinned host memory and back; "
                        "prefix_cache_p2056: prefill with and without the prefix cache; cache_ops: "
                        "slot reservation, pa_copy_blocks, pa_cache_append and the metadata "
                        "upload, each beside the oracle; a _f16 "
                        "suffix (llama3_8b_decode_f16, llama3_8b_prefill_f16, ...) runs a "
                        "decode or prefill leg on fp16 pools")
    p.add_argument("--eager", action="store_true",
                   help="launch every call from Python instead of replaying a captured HIP graph")
    return p.parse_args()


def to_dev(a, dtype, device):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def kv_bytes_per_token(w):
    return 2 * w.num_kv_heads * w.head_dim * (2 if w.dtype == "bf16" else 4)


TRAFFIC_FILES = {
    "llama3_8b_decode": os.path.join(ROOT, "profiles", "pa_decode_llama3_8b_batch8_hbm_traffic.txt"),
    "serving_batch": os.path.join(ROOT, "profiles", "pa_decode_serving_batch_hbm_traffic.txt"),
}
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_cache_338_amd", "csrc", f)
                  for f in ("pa_decode.hip", "pa_attn_tile.h", "pa_device.h")]


def decode_source_hash():
    """sha256 of the decode sources with comments and whitespace removed, so
    that only changes to the code itself invalidate a stored measurement."""
    import hashlib
    import re
    text = "".join(open(f).read() for f in DECODE_SOURCES)
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def measured_traffic(workload="llama3_8b_decode", key="traffic_bytes_per_call"):
    """HBM bytes per call (the `key` line) on a workload from its committed
    counter summary, or None when there is none or the decode code has
    changed since the counters were taken."""
    if workload not in TRAFFIC_FILES:
        return None
    try:
        text = open(TRAFFIC_FILES[workload]).read()
        code_hash = decode_source_hash()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line)
    if fields.get("kernel_source_sha256") != code_hash or key not in fields:
        return None
    return int(fields[key])


def oracle_decode_inputs(w):
    """The oracle's pools, tables and lengths after the workload's script."""
    from oracle import allocator as oa
    from oracle import cache_ops as oc

    alloc = oa.BlockAllocator(w.num_blocks, w.block_size, w.free_order)
    kc, vc = w.empty_pool(), w.empty_pool()
    for op in w.script:
        if op[0] == "create":
            alloc.seq_create(op[1])
        else:
            slots, _ = alloc.seq_reserve(op[1], op[2])
            oc.cache_append(kc, vc, w.k_rows[op[3]], w.v_rows[op[3]], slots, w.block_size)
    maxb = max(len(alloc.seq_block_table(s)) for s in w.seq_ids)
    rows, lens = alloc.block_tables(w.seq_ids, maxb)
    return kc, vc, np.array(rows, np.int32), np.array(lens, np.int32)


def cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, family, model and
    stepping (which identify the part where the name is generic), and the
    logical CPUs the host shows."""
    first, n = {}, 0
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k = k.strip()
            if k == "processor":
                n += 1
            elif k in ("model name", "cpu family", "model", "stepping") and k not in first:
                first[k] = v.strip()
    except OSError:
        return "unknown"
    return (f"{first.get('model name', 'unknown')} (cpu family {first.get('cpu family', '?')}, "
            f"model {first.get('model', '?')}, stepping {first.get('stepping', '?')}; "
            f"{n} logical CPUs on the host)")


def time_oracle_decode(w, inputs, seconds, threads):
    """Repeats the oracle's paged decode of one layer for about `seconds`
    with `threads` BLAS/OpenMP threads: (passes, elapsed seconds)."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as oatt

    kc, vc, tables, lens = inputs
    runs, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=threads):
        while True:
            oatt.paged_decode(w.q, kc, vc, tables, lens, w.block_size, w.scale, w.dtype)
            runs += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return runs, el


def cpu_baseline(w, seconds):
    """The oracle (NumPy fp64) on one layer of the same batch: for 1 thread
    and for every core this process may use, three trials of about
    seconds / 6 each; per thread count the median of the trials' seconds
    per pass, and the better thread count is the value.  Plus a one-thread
    pass of the tiny reference batch."""
    import workloads as W

    cores = len(os.sched_getaffinity(0))
    inputs = oracle_decode_inputs(w)
    ntok = int(inputs[3].sum())
    kv = ntok * kv_bytes_per_token(w)
    counts = sorted({1, cores})
    per_threads = {}
    for t in counts:
        trials = [time_oracle_decode(w, inputs, seconds / (3 * len(counts)), t) for _ in range(3)]
        per_pass = sorted(el / runs for runs, el in trials)
        per_threads[t] = {"median_s_per_pass": per_pass[1],
                          "trials_s_per_pass": [round(x, 5) for x in per_pass],
                          "passes": [runs for runs, _ in trials]}
    best = min(counts, key=lambda t: per_threads[t]["median_s_per_pass"])
    per = per_threads[best]["median_s_per_pass"]
    tw = W.tiny_ref()
    tinp = oracle_decode_inputs(tw)
    r1, e1 = time_oracle_decode(tw, tinp, 1.0, 1)
    tiny = {"us_per_pass": round(e1 / r1 * 1e6, 1), "passes": r1,
            "GB/s": round(int(tinp[3].sum()) * kv_bytes_per_token(tw) / (e1 / r1) / 1e9, 4)}
    return {"value": round(kv / per / 1e9, 4), "unit": "GB/s", "cores": best, "kind": "oracle",
            "us_per_layer": round(per * 1e6, 1), "cpu_model": cpu_model(),
            "threads_tried": {str(t): {"GB/s": round(kv / v["median_s_per_pass"] / 1e9, 4),
                                       "us_per_layer_median": round(v["median_s_per_pass"] * 1e6, 1),
                                       "trials_s_per_pass": v["trials_s_per_pass"],
                                       "passes": v["passes"]}
                              for t, v in per_threads.items()},
            "tiny_ref_one_thread": tiny,
            "sample": f"one layer of the batch ({ntok} tokens, {kv} KV bytes), NumPy fp64 paged "
                      f"decode incl. bf16 widening; 3 trials of about {seconds / (3 * len(counts)):.1f}"
                      f" s per thread count in {counts}; value = median of the 3 at the faster "
                      f"count ({best})"}


def copy_calibration(mib):
    """4 device copies of mib MiB (the runtime's copy kernel): a plain copy of
    known size, to scale the HBM byte counters of a profiler pass."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: 4 copies of {n} bytes")


def copy_bandwidth(dev, nbytes=1 << 30, reps=5):
    """A 1 GiB device-to-device copy (torch copy_), timed with HIP events:
    the bandwidth a plain copy reaches on this GPU, beside the decode's."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del src, dst
    return {"bytes": nbytes, "us": round(us, 1), "read_GBps": round(nbytes / us / 1e3, 1),
            "read_plus_write_GBps": round(2 * nbytes / us / 1e3, 1)}


FLOOR_LIB = os.path.join(ROOT, "paged_kv_cache_338_amd", "libpa_floor.so")


def decode_floor(kpool, vpool, tables_np, lens_np, w, reps, wgs=256):
    """The decode call's cost floor on the same pools: graphs of one launch
    per layer pool, replayed `reps` times between HIP events, of
    * a read of every (block, KV head) tile the call reads, K and V, from a
      precomputed offset list (no table walk, no arithmetic);
    * a contiguous read of the same bytes (the K half from the K pool, the
      V half from the V pool);
    * an empty kernel (the per-launch cost of a back-to-back launch),
    each over `wgs` workgroups of 256 threads, as the decode launches."""
    import ctypes

    import torch

    lib = ctypes.CDLL(FLOOR_LIB)
    lib.pa_floor_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.pa_floor_read_contiguous.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                             ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p,
                                             ctypes.c_void_p]
    lib.pa_floor_empty.argtypes = [ctypes.c_int32, ctypes.c_void_p]
    tile = lib.pa_floor_tile_bytes()
    H_kv, bs, D = w.num_kv_heads, w.block_size, w.head_dim
    if bs * D * 2 != tile or w.dtype != "bf16":
        raise SystemExit("decode_floor: only for bf16 pools with 16 x 128 tiles")
    offs = [(int(tables_np[b, j]) * H_kv + h) * tile
            for h in range(H_kv) for b in range(len(lens_np))
            for j in range(-(-int(lens_np[b]) // bs))]
    pool_bytes = kpool[0].numel() * kpool[0].element_size()
    if max(offs) + tile > pool_bytes or len(offs) * tile > pool_bytes:
        raise SystemExit("decode_floor: tile offsets outside the pools")
    offs_d = torch.tensor(offs, dtype=torch.int64, device=kpool[0].device)
    sink = torch.zeros(wgs * 256, dtype=torch.int32, device=kpool[0].device)
    magic = 0x9E3779B9  # the XOR of the loaded words is never expected to hit it
    n = len(offs)
    per_pool = n * tile  # bytes read from each of K and V
    nl = len(kpool)

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"floor kernel launch failed: hipError {rc}")

    def time_graph(launch):
        stream = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            h = side.cuda_stream
            for l in range(nl):
                launch(l, h)
            side.synchronize()
            with torch.cuda.graph(g, stream=side):
                for l in range(nl):
                    launch(l, h)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * nl)

    tiles_us = time_graph(lambda l, h: check(lib.pa_floor_read_tiles(
        kpool[l].data_ptr(), vpool[l].data_ptr(), offs_d.data_ptr(), n, wgs, magic,
        sink.data_ptr(), h)))
    contig_us = time_graph(lambda l, h: check(lib.pa_floor_read_contiguous(
        kpool[l].data_ptr(), vpool[l].data_ptr(), per_pool, wgs, magic, sink.data_ptr(), h)))
    empty_us = time_graph(lambda l, h: check(lib.pa_floor_empty(wgs, h)))
    return {"tiles": n, "tile_bytes_each_of_k_and_v": tile, "bytes_read": 2 * n * tile,
            "loads": "16-byte non-temporal, as the decode's K/V loads",
            "workgroups": wgs, "read_tiles_us": round(tiles_us, 3),
            "read_contiguous_us": round(contig_us, 3), "empty_launch_us": round(empty_us, 3),
            "timing": f"{reps} replays of a graph of {nl} launches, one per layer pool"}


def replay_timed(make_calls, reps):
    """Captures the prepared calls in one HIP graph (on a side stream, after an
    eager run) and returns the microseconds per replay over reps replays,
    timed with HIP events on the current stream."""
    import torch

    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        calls = make_calls()
        for c in calls:
            c()
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            for c in calls:
                c()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def replay_allocator_script(pa, w):
    """The C++ allocator after the workload's script; its tables and lengths."""
    alloc = pa.Allocator(w.num_blocks, w.block_size, w.free_order)
    for op in w.script:
        if op[0] == "create":
            alloc.seq_create(op[1])
        elif op[0] == "fork":
            alloc.seq_fork(op[1], op[2])
        else:
            alloc.seq_reserve(op[1], op[2], cow_cap=len(op[1]))
    maxb = max(len(alloc.seq_block_table(s)) for s in w.seq_ids)
    tables, lens = alloc.build_block_tables(w.seq_ids, maxb)
    return tables, lens, maxb, alloc


def other_workload(args):
    """pa_decode alone on another workload: the allocator script is replayed
    on the host (tables and lengths exactly as the workload builds them), the
    pools of args.layers layers hold random bf16 values (the values do not
    change the time), and a captured graph of one call per layer is replayed
    args.kernel_reps times between HIP events."""
    import torch

    import paged_kv_cache_338_amd as pa
    import workloads as W

    name = args.workload
    f16 = name.endswith("_f16")  # the same batch on IEEE fp16 pools
    if f16:
        name = name[:-len("_f16")]
    if name == "llama3_8b_decode":
        w = W.llama3_8b_decode(with_values=False)
    elif name.startswith("worked_batch_x"):
        # The worked batch repeated N times (8N sequences, pool 4096N blocks):
        # how the fixed costs of a call fade as the batch grows.
        n = int(name[len("worked_batch_x"):])
        w = W.llama3_8b_decode(lengths=list(W.LLAMA3_8B_BATCH) * n, num_blocks=4096 * n,
                               with_values=False)
    elif name.startswith("block_size_sweep_bs"):
        w = W.block_size_sweep(int(name[len("block_size_sweep_bs"):]), with_values=False)
    elif name.startswith("prefix_sharing_p"):
        w = W.prefix_sharing(prefix_len=int(name[len("prefix_sharing_p"):]), with_values=False)
    elif name == "serving_batch":
        w = W.serving_batch(with_values=False)
    else:
        raise SystemExit(f"unknown workload {name}")
    dev = "cuda:0"
    tables, lens, maxb, alloc = replay_allocator_script(pa, w)
    B, H_q, D = w.batch, w.num_q_heads, w.head_dim
    # Sequences that share blocks (the prefix-sharing batches fork one
    # prompt 128 ways) read them with cached loads; every other batch reads
    # each block once per call, with the library's non-temporal default.
    shared = name.startswith("prefix_sharing")
    pa.pa_set_tuning(pa.PA_TUNE_DECODE_KV_CACHED, 1 if shared else 0)
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, D)
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    dt = torch.float16 if f16 else torch.bfloat16
    kp = [torch.randn(shape, generator=gen, device=dev).to(dt) for _ in range(args.layers)]
    vp = [torch.randn(shape, generator=gen, device=dev).to(dt) for _ in range(args.layers)]
    q = torch.randn((B, H_q, D), generator=gen, device=dev).to(dt)
    outs = [torch.empty_like(q) for _ in range(args.layers)]
    ws = pa.decode_workspace(kp[0], B, H_q, maxb)
    td = torch.from_numpy(tables).to(dev)
    ld = torch.from_numpy(lens).to(dev)
    # A graph of 32 calls cycling over the layer pools (as the default leg's
    # 32 layers), so the gap between graph replays is spread over 32 calls.
    ncalls = 32
    us = replay_timed(lambda: [pa.prepare_decode(q, kp[c % args.layers], vp[c % args.layers], td,
                                                 ld, w.block_size, w.scale,
                                                 outs[c % args.layers], ws)
                               for c in range(ncalls)],
                      args.kernel_reps) / ncalls
    kv = int(lens.sum()) * kv_bytes_per_token(w)
    gbs = kv / (us * 1e-6) / 1e9
    # Tail waste: idle slots at the end of each sequence's last block,
    # ceil(L / bs) bs - L summed over the sequences, as a share of their
    # table slots (blocks shared by several sequences count once per
    # sequence here; blocks_held counts each once).
    held = w.num_blocks - alloc.num_free()
    slots = int(sum(-(-int(L) // w.block_size) * w.block_size for L in lens))
    idle = slots - int(lens.sum())
    idle_pct = 100.0 * idle / slots
    log(f"{args.workload}: B={B} tokens={int(lens.sum())} maxb={maxb}: {us:.2f} us/call, "
        f"{gbs:.0f} GB/s; {held} blocks held, {idle} idle slots ({idle_pct:.3f} %)")
    print(json.dumps({
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.kernel_reps * ncalls, "warmup": 1, "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if f16 else "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: pa_decode alone, graph replay of {ncalls} "
                               f"calls cycling over {args.layers} layer pools",
                   "batch": B, "tokens": int(lens.sum()), "block_size": w.block_size,
                   "kv_loads": "cached (shared blocks)" if shared else "non-temporal (default)",
                   "us_per_call": round(us, 3), "blocks_held": held, "idle_slots": idle,
                   "idle_slots_pct": round(idle_pct, 3)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if f16 else measured_traffic(name),
                     "kernel": "pa_decode (decode_kernel, one launch)",
                     "algorithmic_bytes_per_call": kv}}), flush=True)


CACHE_OPS_METRIC = ("paged KV cache maintenance on the pages' workloads: slot reservation (host), "
                    "pa_copy_blocks, pa_cache_append, metadata upload")


def cache_ops_workload(args):
    """The steps around the decode kernel, each on the workload where the
    pages put it, each timed beside the oracle doing the same on the host:

    * llama3_8b (the worked batch): one decode step's reservation of one
      token per sequence and the append of those 8 tokens;
    * prefix_sharing_p2056: the first call after the forks reserves every
      sequence's suffix plus one token (32,267 tokens), which copies the
      shared, half-filled tail block for 127 of the 128 sequences; then
      pa_copy_blocks of those 127 pairs and the append of the 32,267 tokens;
    * serving_batch: the reservation and append of one token for each of
      256 sequences, and the upload of the tables, lengths and slot mapping
      from pinned host memory.

    Device calls are captured in a graph over args.layers layer pools (32 by
    default, a different pool each call) and replayed args.kernel_reps times; copies
    and appends rewrite the same values, so every replay does the same
    work.  Bytes: a copy reads and writes its whole blocks; an append reads
    the tokens' K/V rows and writes them into the pool."""
    import torch

    import paged_kv_cache_338_amd as pa
    import workloads as W
    from oracle import allocator as oa
    from oracle import cache_ops as oc

    dev = "cuda:0"
    layers = args.layers

    def split_script(w):
        """The script up to its last reservation, and that reservation."""
        last = max(i for i, op in enumerate(w.script) if op[0] == "reserve")
        return w.script[:last], w.script[last]

    def replay(alloc, ops, fork, reserve):
        for op in ops:
            if op[0] == "create":
                alloc.seq_create(op[1])
            elif op[0] == "fork":
                fork(op[1], op[2])
            else:
                reserve(op[1], op[2])

    def host_reserve(w, reps):
        """Microseconds of the last reservation: C++ allocator and oracle,
        each replayed from a fresh allocator before every timed call."""
        head, (_, sids, ns, _) = split_script(w)
        cap = len(sids)
        times = {"cpp": [], "oracle": []}
        slots = pairs = None
        for _ in range(reps):
            a = pa.Allocator(w.num_blocks, w.block_size, w.free_order)
            replay(a, head, a.seq_fork, lambda s, n: a.seq_reserve(s, n, cow_cap=len(s)))
            t0 = time.perf_counter()
            slots, pairs = a.seq_reserve(sids, ns, cow_cap=cap)
            times["cpp"].append(time.perf_counter() - t0)
            a.close()
            o = oa.BlockAllocator(w.num_blocks, w.block_size, w.free_order)
            replay(o, head, o.seq_fork, o.seq_reserve)
            t0 = time.perf_counter()
            oslots, opairs = o.seq_reserve(sids, ns)
            times["oracle"].append(time.perf_counter() - t0)
        assert np.array_equal(np.asarray(slots), np.asarray(oslots, np.int64))
        assert np.array_equal(np.asarray(pairs).reshape(-1, 2), np.asarray(opairs, np.int64).reshape(-1, 2))
        med = {k: float(np.median(v)) * 1e6 for k, v in times.items()}
        return np.asarray(slots, np.int64), np.asarray(pairs, np.int32).reshape(-1, 2), med

    def device_pools(w):
        shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        gen = torch.Generator(device=dev).manual_seed(w.seed)
        kp = [torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16) for _ in range(layers)]
        vp = [torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16) for _ in range(layers)]
        return kp, vp

    def oracle_seconds(fn, min_seconds=1.0):
        runs, t0 = 0, time.perf_counter()
        while True:
            fn()
            runs += 1
            el = time.perf_counter() - t0
            if el >= min_seconds:
                return el / runs

    def append_leg(w, slots, kp, vp):
        T = len(slots)
        gen = torch.Generator(device=dev).manual_seed(w.seed + 100)
        kn = torch.randn((T, w.num_kv_heads, w.head_dim), generator=gen, device=dev).to(torch.bfloat16)
        vn = torch.randn((T, w.num_kv_heads, w.head_dim), generator=gen, device=dev).to(torch.bfloat16)
        sd = torch.from_numpy(slots).to(dev)
        us = replay_timed(lambda: [pa.prepare_cache_append(kn, vn, sd, kp[l], vp[l])
                                   for l in range(layers)], args.kernel_reps) / layers
        row = w.num_kv_heads * w.head_dim * 2
        nbytes = 2 * 2 * T * row  # K and V rows: read from k, v and written to the pools
        kc = np.zeros((w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim), np.uint16)
        vc = np.zeros_like(kc)
        kh = np.zeros((T, w.num_kv_heads, w.head_dim), np.uint16)
        o_us = oracle_seconds(lambda: oc.cache_append(kc, vc, kh, kh, slots, w.block_size)) * 1e6
        return {"tokens": T, "us_per_call": round(us, 3), "bytes": nbytes,
                "GB/s": round(nbytes / us / 1e3, 1), "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                "oracle_us": round(o_us, 1)}

    out = {}
    # ---- the worked batch: one decode step
    w = W.llama3_8b_decode(with_values=False)
    w.script.append(("reserve", list(range(w.batch)), [1] * w.batch,
                     np.arange(w.batch, dtype=np.int64)))
    slots, pairs, med = host_reserve(w, 20)
    kp, vp = device_pools(w)
    out["llama3_8b_step"] = {"a1_reserve_host_us": {k: round(v, 1) for k, v in med.items()},
                             "a3_append": append_leg(w, slots, kp, vp)}
    del kp, vp
    log(f"llama3_8b step: {out['llama3_8b_step']}")

    # ---- prefix sharing: the first step after the forks (copy-on-write)
    w = W.prefix_sharing(with_values=False)
    slots, pairs, med = host_reserve(w, 5)
    kp, vp = device_pools(w)
    P = len(pairs)
    pd = torch.from_numpy(np.ascontiguousarray(pairs)).to(dev)
    us = replay_timed(lambda: [pa.prepare_copy_blocks(pd, P, kp[l], vp[l]) for l in range(layers)],
                      args.kernel_reps) / layers
    blk = w.num_kv_heads * w.block_size * w.head_dim * 2
    cbytes = 2 * 2 * P * blk  # K and V blocks, each read once and written once
    kc = np.zeros((w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim), np.uint16)
    vc = np.zeros_like(kc)
    o_us = oracle_seconds(lambda: oc.copy_blocks(kc, vc, pairs)) * 1e6
    copy = {"pairs": P, "us_per_call": round(us, 3), "bytes": cbytes,
            "GB/s": round(cbytes / us / 1e3, 1), "frac_of_hbm_peak": round(cbytes / us / 1e3 / HBM_PEAK_GBS, 4),
            "oracle_us": round(o_us, 1)}
    out["prefix_sharing_p2056_first_step"] = {
        "a1_reserve_host_us": {k: round(v, 1) for k, v in med.items()},
        "a2_copy_blocks": copy, "a3_append": append_leg(w, slots, kp, vp)}
    del kp, vp
    log(f"prefix sharing: {out['prefix_sharing_p2056_first_step']}")

    # ---- serving batch: one token for each of 256 sequences, and the upload
    w = W.serving_batch(with_values=False)
    slots, pairs, med = host_reserve(w, 5)
    kp, vp = device_pools(w)
    ent = {"a1_reserve_host_us": {k: round(v, 1) for k, v in med.items()},
           "a3_append": append_leg(w, slots, kp, vp)}
    del kp, vp
    a = pa.Allocator(w.num_blocks, w.block_size, w.free_order)
    replay(a, w.script, a.seq_fork, lambda s, n: a.seq_reserve(s, n, cow_cap=len(s)))
    maxb = max(len(a.seq_block_table(s)) for s in w.seq_ids)
    tab = torch.empty((w.batch, maxb), dtype=torch.int32, pin_memory=True)
    lens = torch.empty(w.batch, dtype=torch.int32, pin_memory=True)
    sl = torch.from_numpy(slots).pin_memory()
    t0 = time.perf_counter()
    for _ in range(20):
        a.build_block_tables(w.seq_ids, maxb, tables_out=tab.numpy(), lens_out=lens.numpy())
    build_us = (time.perf_counter() - t0) / 20 * 1e6
    o = oa.BlockAllocator(w.num_blocks, w.block_size, w.free_order)
    replay(o, w.script, o.seq_fork, o.seq_reserve)
    ob_us = oracle_seconds(lambda: o.block_tables(w.seq_ids, maxb)) * 1e6
    td = torch.empty_like(tab, device=dev)
    ld = torch.empty_like(lens, device=dev)
    sd = torch.empty_like(sl, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        td.copy_(tab, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.kernel_reps):
        td.copy_(tab, non_blocking=True)
        ld.copy_(lens, non_blocking=True)
        sd.copy_(sl, non_blocking=True)
    e1.record(stream)
    torch.cuda.synchronize()
    up_us = e0.elapsed_time(e1) * 1e3 / args.kernel_reps
    ubytes = tab.numel() * 4 + lens.numel() * 4 + sl.numel() * 8
    live = int(sum(len(a.seq_block_table(s)) for s in w.seq_ids)) * 4
    a.close()
    ent["a4_metadata"] = {"tables_shape": [w.batch, maxb], "build_tables_host_us": round(build_us, 1),
                          "oracle_build_tables_us": round(ob_us, 1),
                          "upload_us": round(up_us, 2), "upload_bytes": ubytes,
                          "live_table_bytes": live,
                          "upload_GB/s": round(ubytes / up_us / 1e3, 2)}
    out["serving_batch_step"] = ent
    log(f"serving batch: {ent}")

    cp = out["prefix_sharing_p2056_first_step"]["a2_copy_blocks"]
    print(json.dumps({
        "metric": CACHE_OPS_METRIC, "value": cp["GB/s"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.kernel_reps * layers, "warmup": 1, "ms_per_step": round(cp["us_per_call"] / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"cache_ops: {layers} layer pools, graph replay; value = "
                               "pa_copy_blocks of the prefix-sharing batch's 127 copy-on-write "
                               "pairs (bytes read + written)", "rows": out},
        "roofline": {"bound": "hbm", "achieved": cp["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": cp["frac_of_hbm_peak"], "traffic": None,
                     "kernel": "pa_copy_blocks (copy_blocks_kernel), one layer"},
        "cpu_baseline": {"value": round(cbytes / cp["oracle_us"] / 1e3, 4), "unit": "GB/s",
                         "cores": 1, "kind": "oracle",
                         "sample": "the oracle's copy_blocks of the same 127 pairs (NumPy, one "
                                   "thread), repeated for about 1 s"}}), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0
PREFILL_METRIC = ("paged prefill attention TFLOP/s (% of dense bf16 MFMA peak), Llama-3-8B shape, "
                  "worked-example batch")


def prefill_queries(lens, chunk):
    """Query tokens per sequence: the whole prompt (chunk None) or its last
    min(chunk, L_b) tokens (a chunked-prefill step)."""
    lens = np.asarray(lens, np.int64)
    return lens.copy() if chunk is None else np.minimum(lens, chunk)


def prefill_flops(lens, nq, num_q_heads, head_dim):
    """Work of one causal call: every (query row, key) pair the mask keeps
    costs 2*D flops for q.k and 2*D for p.v, per query head."""
    lens, nq = np.asarray(lens, np.int64), np.asarray(nq, np.int64)
    pairs = nq * (lens - nq) + nq * (nq + 1) // 2
    return int(pairs.sum()) * num_q_heads * 4 * head_dim


def prefill_workload(args):
    """pa_prefill alone on the worked batch at the Llama-3-8B shape: the
    whole prompts (llama3_8b_prefill, 10,578 query tokens) or a chunk of the
    last N tokens of each (llama3_8b_chunked_prefill_cN).  Tables come from
    the allocator script; pools of args.layers layers hold random bf16."""
    import torch

    import paged_kv_cache_338_amd as pa
    import workloads as W

    name = args.workload
    f16 = name.endswith("_f16")  # the same batch on IEEE fp16 pools
    if f16:
        name = name[:-len("_f16")]
    if name == "llama3_8b_prefill":
        chunk = None
    elif name.startswith("llama3_8b_chunked_prefill_c"):
        chunk = int(name[len("llama3_8b_chunked_prefill_c"):])
    else:
        raise SystemExit(f"unknown workload {name}")
    dev = "cuda:0"
    w = W.llama3_8b_decode(with_values=False)
    tables, lens, maxb, _ = replay_allocator_script(pa, w)
    nq = prefill_queries(lens, chunk)
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    T, H_q, D = int(qs[-1]), w.num_q_heads, w.head_dim
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, D)
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    dt = torch.float16 if f16 else torch.bfloat16
    kp = [torch.randn(shape, generator=gen, device=dev).to(dt) for _ in range(args.layers)]
    vp = [torch.randn(shape, generator=gen, device=dev).to(dt) for _ in range(args.layers)]
    q = torch.randn((T, H_q, D), generator=gen, device=dev).to(dt)
    outs = [torch.empty_like(q) for _ in range(args.layers)]
    td = torch.from_numpy(tables).to(dev)
    ld = torch.from_numpy(lens).to(dev)
    qsd = torch.from_numpy(qs).to(dev)
    # pa_prefill_split: splits the key range of long query blocks when the
    # call has too few query blocks to fill the GPU (the short chunks), and
    # is pa_prefill otherwise (its workspace is then empty).
    ws = pa.prefill_split_workspace(kp[0], w.batch, H_q, T, tables.shape[1])
    ws_bytes = pa.pa_prefill_split_workspace_size(pa.cache_desc(kp[0]), w.batch, H_q, T,
                                                  tables.shape[1])
    us = replay_timed(lambda: [pa.prepare_prefill(q, kp[l], vp[l], td, ld, qsd, w.block_size,
                                                  w.scale, outs[l], workspace=ws)
                               for l in range(args.layers)],
                      args.kernel_reps) / args.layers
    flops = prefill_flops(lens, nq, H_q, D)
    tfs = flops / (us * 1e-6) / 1e12
    log(f"{args.workload}: B={w.batch} query tokens={T} cache tokens={int(lens.sum())}: "
        f"{us:.2f} us/call, {tfs:.1f} TFLOP/s")
    result = {
        "metric": PREFILL_METRIC, "value": round(tfs, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.kernel_reps * args.layers, "warmup": 1, "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if f16 else "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: pa_prefill alone, {args.layers} layer pools, "
                               "graph replay; "
                               "32 Q / 8 KV heads, head 128, bs 16, bf16",
                   "batch": w.batch, "query_tokens": T, "cache_tokens": int(lens.sum()),
                   "query_tokens_per_seq": nq.tolist(), "us_per_call": round(us, 3),
                   "entry_point": "pa_prefill_split" + (" (key range split, workspace "
                                                        f"{ws_bytes} B)" if ws_bytes else
                                                        " (not split: runs as pa_prefill)")},
        "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "pa_prefill_split (attention kernel, plus the merge kernel when split), one layer",
                     "us_per_launch": round(us, 3), "algorithmic_flops_per_call": flops},
    }
    if not args.no_cpu_baseline and not f16:
        log("cpu baseline (oracle)...")
        result["cpu_baseline"] = cpu_baseline_prefill(w.seed, chunk, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline_prefill(seed, chunk, seconds):
    """The oracle's paged prefill on the same batch, one sequence per call in
    batch order until the time budget is spent (the sample)."""
    from threadpoolctl import threadpool_limits

    from oracle import allocator as oa
    from oracle import cache_ops as oc
    from oracle import prefill as op
    import workloads as W

    w = W.llama3_8b_decode(seed=seed)
    cores = len(os.sched_getaffinity(0))
    alloc = oa.BlockAllocator(w.num_blocks, w.block_size, w.free_order)
    kc, vc = w.empty_pool(), w.empty_pool()
    for o in w.script:
        if o[0] == "create":
            alloc.seq_create(o[1])
        else:
            slots, _ = alloc.seq_reserve(o[1], o[2])
            oc.cache_append(kc, vc, w.k_rows[o[3]], w.v_rows[o[3]], slots, w.block_size)
    maxb = max(len(alloc.seq_block_table(s)) for s in w.seq_ids)
    rows, lens = alloc.block_tables(w.seq_ids, maxb)
    tables, lens = np.array(rows, np.int32), np.array(lens, np.int64)
    nq = prefill_queries(lens, chunk)
    rng = np.random.default_rng(seed)
    flops, done, t0 = 0, [], time.perf_counter()
    with threadpool_limits(limits=cores):
        for b in range(len(lens)):
            n = int(nq[b])
            qb = W.round_to_bf16_bits(rng.standard_normal((n, w.num_q_heads, w.head_dim),
                                                          dtype=np.float32))
            op.paged_prefill(qb, kc, vc, tables[b:b + 1], lens[b:b + 1], [0, n], w.block_size,
                             w.scale, w.dtype)
            flops += op.prefill_flops(lens[b:b + 1], [0, n], w.num_q_heads, w.head_dim)
            done.append(n)
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"sequences 0..{len(done) - 1} of the batch (query tokens {done}) in "
                      f"{el:.1f} s, NumPy fp64 paged prefill incl. bf16 widening"}


HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, per direction


def swap_workload(args):
    """pa_swap_blocks alone: every block of the worked Llama-3-8B batch (665
    blocks of 64 KiB, all eight sequences preempted) from the device pool to
    a pinned host pool, and back into other device blocks, as the C
    allocator's swap-out and swap-in emit the pairs.  One launch per
    direction, captured in a graph and replayed args.kernel_reps times."""
    import torch

    import paged_kv_cache_338_amd as pa
    import workloads as W

    dev = "cuda:0"
    w = W.llama3_8b_decode(with_values=False)
    alloc = pa.Allocator(w.num_blocks, w.block_size, w.free_order)
    for op in w.script:
        if op[0] == "create":
            alloc.seq_create(op[1])
        else:
            alloc.seq_reserve(op[1], op[2], cow_cap=len(op[1]))
    nblk = sum(len(alloc.seq_block_table(s)) for s in w.seq_ids)
    alloc.add_host_pool(nblk, np.random.default_rng(w.seed).permutation(nblk))
    out_pairs = np.concatenate([alloc.seq_swap_out(s) for s in w.seq_ids])
    in_pairs = np.concatenate([alloc.seq_swap_in(s) for s in w.seq_ids])
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    hshape = (nblk,) + shape[1:]
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    kp = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
    vp = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
    hk = torch.empty(hshape, dtype=torch.bfloat16).pin_memory()
    hv = torch.empty(hshape, dtype=torch.bfloat16).pin_memory()
    po = torch.from_numpy(out_pairs).to(dev)
    pi = torch.from_numpy(in_pairs).to(dev)
    block_bytes = 2 * w.num_kv_heads * w.block_size * w.head_dim * 2  # K and V, bf16
    moved = nblk * block_bytes
    us_out = replay_timed(lambda: [pa.prepare_swap_blocks(po, nblk, kp, vp, hk, hv)],
                          args.kernel_reps)
    us_in = replay_timed(lambda: [pa.prepare_swap_blocks(pi, nblk, hk, hv, kp, vp)],
                         args.kernel_reps)
    gbs_out, gbs_in = moved / (us_out * 1e-6) / 1e9, moved / (us_in * 1e-6) / 1e9
    both = 2 * moved / ((us_out + us_in) * 1e-6) / 1e9
    log(f"swap: {nblk} blocks, {moved} B each way: out {us_out:.1f} us ({gbs_out:.1f} GB/s), "
        f"in {us_in:.1f} us ({gbs_in:.1f} GB/s)")
    print(json.dumps({
        "metric": "preemption swap GB/s (device pool <-> pinned host pool), Llama-3-8B batch",
        "value": round(both, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.kernel_reps,
        "warmup": 1, "ms_per_step": round((us_out + us_in) / 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "swap_llama3_8b: all 8 sequences of the worked batch swapped out "
                               "to pinned host blocks and back in to other device blocks, one "
                               "pa_swap_blocks launch per direction, graph replay",
                   "blocks": int(nblk), "bytes_each_way": int(moved),
                   "us_swap_out": round(us_out, 2), "us_swap_in": round(us_in, 2),
                   "gbs_swap_out": round(gbs_out, 2), "gbs_swap_in": round(gbs_in, 2)},
        "roofline": {"bound": "host-link", "achieved": round(both, 2), "peak": HOST_LINK_PEAK_GBS,
                     "unit": "GB/s", "frac": round(both / HOST_LINK_PEAK_GBS, 4),
                     "traffic": None, "kernel": "pa_swap_blocks (move_blocks_kernel), one "
                                                "launch per direction"}}), flush=True)


def prefix_cache_workload(args):
    """Prefix caching on the prefix-sharing requests: 128 prompts of a shared
    2,056-token system prompt plus each request's own suffix (uniform 0-512
    tokens plus one), at the Llama-3-8B head layout.  Without the cache every
    prompt is prefilled whole; with it, a first request fills the prompt's
    blocks, and each request then takes its 128 cached blocks
    (pa_seq_match_prefix) and prefills only the rest, as one chunked-prefill
    call against the shared blocks.  Reports both pa_prefill times (graph
    replay) and the host cost of the lookups."""
    import torch

    import paged_kv_cache_338_amd as pa
    import workloads as W

    dev = "cuda:0"
    w = W.prefix_sharing(with_values=False)
    P, bs, H_q, H_kv, D = w.notes["prefix_len"], w.block_size, w.num_q_heads, w.num_kv_heads, w.head_dim
    suffix = [x + 1 for x in w.notes["suffix"]]
    rng = np.random.default_rng(w.seed)
    prompt = rng.integers(0, 32000, P).astype(np.int32)
    prompts = [np.concatenate([prompt, rng.integers(0, 32000, n).astype(np.int32)])
               for n in suffix]
    lens = np.array([len(t) for t in prompts], np.int32)
    B = len(prompts)
    nb = int(sum(-(-L // bs) for L in lens) * 1.1) + 64
    shape = (nb, H_kv, bs, D)
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    kp = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
    vp = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)

    def prefill_us(alloc, ids, nq):
        maxb = max(len(alloc.seq_block_table(s)) for s in ids)
        tables, ln = alloc.build_block_tables(ids, maxb)
        qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
        T = int(qs[-1])
        q = torch.randn((T, H_q, D), generator=gen, device=dev).to(torch.bfloat16)
        out = torch.empty_like(q)
        td, ld, qsd = (torch.from_numpy(x).to(dev) for x in (tables, ln, qs))
        us = replay_timed(lambda: [pa.prepare_prefill(q, kp, vp, td, ld, qsd, bs, w.scale, out)],
                          args.kernel_reps)
        return us, prefill_flops(ln, nq, H_q, D), T

    # Without the cache: every prompt prefilled whole.
    order = rng.permutation(nb)
    a0 = pa.Allocator(nb, bs, order)
    for i in range(B):
        a0.seq_create(i)
        a0.seq_reserve([i], [int(lens[i])])
    us_full, fl_full, T_full = prefill_us(a0, list(range(B)), lens)
    del a0
    # With the cache: one request fills the prompt, then each request reuses it.
    a1 = pa.Allocator(nb, bs, order)
    a1.enable_prefix_cache()
    a1.seq_create(-1)
    a1.match_prefix(-1, prompt)
    a1.seq_reserve([-1], [P])
    a1.seq_free(-1)
    t0 = time.perf_counter()
    hits = []
    for i, toks in enumerate(prompts):
        a1.seq_create(i)
        h = a1.match_prefix(i, toks)
        a1.seq_reserve([i], [len(toks) - h])
        hits.append(h)
    host_us = (time.perf_counter() - t0) * 1e6 / B
    nq = lens - np.array(hits, np.int32)
    us_cached, fl_cached, T_cached = prefill_us(a1, list(range(B)), nq)
    log(f"prefix cache: {B} requests, prompt {P} + suffixes: whole prompts {T_full} queries "
        f"{us_full:.1f} us; cached prefix (hits {min(hits)}-{max(hits)} tokens) {T_cached} queries "
        f"{us_cached:.1f} us ({us_full / us_cached:.2f}x); lookup + reserve {host_us:.1f} us/request")
    tfs = fl_cached / (us_cached * 1e-6) / 1e12
    print(json.dumps({
        "metric": "prefix-cached prefill time per call (us), 128 requests sharing a 2,056-token "
                  "prompt, Llama-3-8B heads", "value": round(us_cached, 2), "unit": "us",
        "n_gpus": 1, "steps": args.kernel_reps, "warmup": 1,
        "ms_per_step": round(us_cached / 1e3, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefix_cache_p2056: pa_seq_match_prefix + suffix-only pa_prefill "
                               "vs whole-prompt pa_prefill, graph replay",
                   "requests": B, "prompt_tokens": P, "query_tokens_whole": T_full,
                   "query_tokens_cached": T_cached, "us_whole_prompts": round(us_full, 2),
                   "us_cached_prefix": round(us_cached, 2),
                   "speedup": round(us_full / us_cached, 3),
                   "host_us_per_request": round(host_us, 2),
                   "cached_tokens_per_request": int(min(hits))},
        "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "pa_prefill over the cached prefix",
                     "algorithmic_flops_per_call": fl_cached}}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode path "
              "shards by sequence or KV head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if args.workload != "llama3_8b_decode":  # kernel legs on other workloads
        if args.layers == 32 and args.workload != "cache_ops":
            args.layers = 2  # each of these batches is larger than the last-level cache
        if "prefill" in args.workload:
            prefill_workload(args)
        elif args.workload == "swap_llama3_8b":
            swap_workload(args)
        elif args.workload == "prefix_cache_p2056":
            prefix_cache_workload(args)
        elif args.workload == "cache_ops":
            cache_ops_workload(args)
        else:
            other_workload(args)
        if args.copy_calibration > 0:
            copy_calibration(args.copy_calibration)
        return
    import torch

    import paged_kv_cache_338_amd as pa
    import workloads as W

    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = W.llama3_8b_decode()
    B, L0 = w.batch, w.context_lens.copy()
    H_q, H_kv, D, bs = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    nl = args.layers
    if args.warmup < 1:
        args.warmup = 1  # the first step captures the layer loop
        log("--warmup raised to 1: the first step captures the layer loop")
    total_steps = args.warmup + args.steps
    maxb = int(math.ceil((L0.max() + total_steps + 1) / bs))
    log(f"workload {w.name}: B={B} tokens={int(L0.sum())} layers={nl} pool={w.num_blocks} "
        f"blocks/layer, maxb={maxb}")

    # ---- set-up (untimed): allocator + prefill of every layer's pools
    alloc = pa.Allocator(w.num_blocks, bs, w.free_order)
    kpool = [to_dev(w.empty_pool(), w.dtype, dev) for _ in range(nl)]
    vpool = [to_dev(w.empty_pool(), w.dtype, dev) for _ in range(nl)]
    krows = to_dev(w.k_rows, w.dtype, dev)
    vrows = to_dev(w.v_rows, w.dtype, dev)
    for op in w.script:
        if op[0] == "create":
            alloc.seq_create(op[1])
            continue
        slots, pairs = alloc.seq_reserve(op[1], op[2])
        assert len(pairs) == 0
        idx = torch.from_numpy(op[3]).to(dev)
        kr, vr = krows.index_select(0, idx), vrows.index_select(0, idx)
        sd = torch.from_numpy(slots.copy()).to(dev)
        for l in range(nl):
            pa.pa_cache_append(kr, vr, sd, kpool[l], vpool[l])
    del krows, vrows
    q = to_dev(w.q, w.dtype, dev)
    outs = [torch.empty_like(q) for _ in range(nl)]
    ws = pa.decode_workspace(kpool[0], B, H_q, maxb)
    tables_np, lens_np = alloc.build_block_tables(w.seq_ids, maxb)
    # The tables and the lengths side by side in one device buffer, so that
    # each step uploads its metadata with one copy.
    meta_d = torch.empty(B * maxb + B, dtype=torch.int32, device=dev)
    tables_d = meta_d[:B * maxb].view(B, maxb)
    lens_d = meta_d[B * maxb:]
    tables_d.copy_(torch.from_numpy(tables_np))
    lens_d.copy_(torch.from_numpy(lens_np))
    torch.cuda.synchronize()
    log("prefill done")

    # ---- decode-only leg: pa_decode alone, back-to-back over the layer
    # pools, on the prefilled cache.  The calls only enqueue kernels (no
    # allocation, no memset), so they are captured once in a HIP graph and
    # replayed: the timing is then the GPU's, not Python's launch rate.
    stream = torch.cuda.current_stream()

    def captured(make_calls):
        """Calls made on the capture stream, and a replay function."""
        if args.eager:
            calls = make_calls()
            return lambda: [c() for c in calls]
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            calls = make_calls()  # prepared on the capture stream
            for c in calls:  # eager run first: library loaded, attributes set
                c()
            side.synchronize()
            with torch.cuda.graph(g, stream=side):
                for c in calls:
                    c()
        torch.cuda.synchronize()
        return g.replay

    run_dec = captured(lambda: [pa.prepare_decode(q, kpool[l], vpool[l], tables_d, lens_d, bs,
                                                  w.scale, outs[l], ws) for l in range(nl)])
    def timed_replays(run):
        """Microseconds per call: the mean over all replays, and the
        per-replay means (one HIP event between consecutive replays)."""
        run()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.kernel_reps + 1)]
        evs[0].record(stream)
        for i in range(args.kernel_reps):
            run()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.kernel_reps)])
        return evs[0].elapsed_time(evs[-1]) * 1e3 / (args.kernel_reps * nl), per * 1e3 / nl

    us_dec, per_rep = timed_replays(run_dec)
    d10, d50, d90 = (float(x) for x in np.percentile(per_rep, [10, 50, 90]))
    launches = args.kernel_reps * nl
    kv_dec = int(lens_np.sum()) * kv_bytes_per_token(w)
    achieved_dec = kv_dec / (us_dec * 1e-6) / 1e9
    log(f"pa_decode alone: {us_dec:.2f} us/launch (median {d50:.2f}, p10 {d10:.2f}, p90 {d90:.2f}), "
        f"{achieved_dec:.0f} GB/s over {launches} launches")
    # The same calls all on layer 0's pools: the 268 MB pair then stays in
    # the 256 MB last-level cache in large part (labelled MALL-warm).
    us_warm, _ = timed_replays(captured(
        lambda: [pa.prepare_decode(q, kpool[0], vpool[0], tables_d, lens_d, bs, w.scale,
                                   outs[l], ws) for l in range(nl)]))
    log(f"pa_decode, one pool (MALL-warm): {us_warm:.2f} us/launch")
    floor = decode_floor(kpool, vpool, tables_np, lens_np, w, args.kernel_reps)
    log(f"floor: tile read {floor['read_tiles_us']:.2f} us, contiguous read "
        f"{floor['read_contiguous_us']:.2f} us, empty launch {floor['empty_launch_us']:.2f} us "
        f"({floor['tiles']} tiles)")

    # ---- whole decode steps.  Per layer one pa_decode_append call: the
    # new token's K and V are written at position L - 1 (its slot from the
    # table) and the layer's attention runs, in one kernel.
    new_k = to_dev(w.notes["new_k"], w.dtype, dev)
    new_v = to_dev(w.notes["new_v"], w.dtype, dev)
    pin = [dict(slots=torch.empty(B, dtype=torch.int64, pin_memory=True),
                meta=torch.empty(B * maxb + B, dtype=torch.int32, pin_memory=True),
                pairs=torch.empty((B, 2), dtype=torch.int32, pin_memory=True),
                ev=torch.cuda.Event()) for _ in range(2)]
    for buf in pin:  # the layout of meta_d
        buf["tables"] = buf["meta"][:B * maxb].view(B, maxb)
        buf["lens"] = buf["meta"][B * maxb:]
    pairs_d = torch.empty((B, 2), dtype=torch.int32, device=dev)

    def layer_calls():
        return [pa.prepare_decode_append(q, new_k, new_v, kpool[l], vpool[l], tables_d, lens_d, bs,
                                         w.scale, outs[l], ws) for l in range(nl)]

    seq_ids = np.array(w.seq_ids, np.int64)
    ones = np.ones(B, np.int32)
    kv_read = []
    last_lens = np.zeros(B, np.int32)

    def step(i):
        buf = pin[i % 2]
        buf["ev"].synchronize()  # its previous upload has finished
        slots_np = buf["slots"].numpy()
        s, p = alloc.seq_reserve(seq_ids, ones, cow_cap=B, out=slots_np)
        npairs = len(p)
        if npairs:
            buf["pairs"].numpy()[:npairs] = p
        alloc.build_block_tables(seq_ids, maxb, tables_out=buf["tables"].numpy(),
                                 lens_out=buf["lens"].numpy())
        meta_d.copy_(buf["meta"], non_blocking=True)
        if npairs:
            pairs_d[:npairs].copy_(buf["pairs"][:npairs], non_blocking=True)
        buf["ev"].record(stream)
        kv_read.append(int(buf["lens"].numpy().sum()) * kv_bytes_per_token(w) * nl)
        last_lens[:] = buf["lens"].numpy()
        if npairs:  # copy-on-write before the step's appends (none in this batch)
            for l in range(nl):
                pa.prepare_copy_blocks(pairs_d, npairs, kpool[l], vpool[l])()
        nonlocal run_layers
        if run_layers is None:
            run_layers = captured(layer_calls)
        else:
            run_layers()

    # The first (warm-up) step captures the layer loop: the capture's eager
    # run is that step's work, after its uploads; later steps replay.
    run_layers = None
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    kv_read.clear()
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    gc.collect()
    gc.disable()  # no collector pauses inside the timed steps
    t_start = time.perf_counter()
    sev[0].record(stream)
    for i in range(args.warmup, total_steps):
        step(i)
        sev[i - args.warmup + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gc.enable()
    gpu_ms = sev[0].elapsed_time(sev[-1])
    ms_step = max(gpu_ms, wall * 1e3) / args.steps
    step_ms = np.array([sev[i].elapsed_time(sev[i + 1]) for i in range(args.steps)])
    sp10, sp50, sp90 = (float(x) for x in np.percentile(step_ms, [10, 50, 90]))
    value = sum(kv_read) / (ms_step * args.steps * 1e-3) / 1e9
    log(f"steps: {ms_step:.3f} ms/step ({ms_step * 1e3 / nl:.2f} us/layer; median {sp50:.3f}, "
        f"p10 {sp10:.3f}, p90 {sp90:.3f}, max {step_ms.max():.3f} ms; wall {wall * 1e3:.1f} ms, "
        f"GPU {gpu_ms:.1f} ms), {value:.0f} GB/s")

    # ---- roofline leg: the step's kernel, pa_decode_append, on the last
    # step's tables and lengths, back-to-back over the layer pools (each
    # replay writes the same new rows again and decodes).
    run_app = captured(lambda: [pa.prepare_decode_append(q, new_k, new_v, kpool[l], vpool[l],
                                                         tables_d, lens_d, bs, w.scale, outs[l],
                                                         ws) for l in range(nl)])
    us_launch, per_rep = timed_replays(run_app)
    p10, p50, p90 = (float(x) for x in np.percentile(per_rep, [10, 50, 90]))
    kv_launch = int(last_lens.sum()) * kv_bytes_per_token(w)
    alg_launch = kv_launch + B * kv_bytes_per_token(w)  # + the new rows written
    achieved = alg_launch / (us_launch * 1e-6) / 1e9
    log(f"pa_decode_append: {us_launch:.2f} us/launch (median {p50:.2f}, p10 {p10:.2f}, "
        f"p90 {p90:.2f}), {achieved:.0f} GB/s over {launches} launches")

    mode = "eager launches" if args.eager else "HIP graph replay of the layer loop"
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_decode: per step, host slot reservation + table upload, "
                               f"then {nl} layers x pa_decode_append (the new token's K/V "
                               f"written at its slot and the layer's decode, one kernel) by "
                               f"{mode}; 32 Q / 8 KV heads, head 128, bs 16, bf16, pool 4096 "
                               "blocks per layer",
                   "batch": B, "context_lens_at_first_step": (L0 + args.warmup + 1).tolist(),
                   "tokens_added_per_step": B, "layers": nl,
                   "us_per_layer": round(ms_step * 1e3 / nl, 3),
                   "step_ms_median": round(sp50, 4), "step_ms_p10": round(sp10, 4),
                   "step_ms_p90": round(sp90, 4), "step_ms_max": round(float(step_ms.max()), 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "traffic_note": "HBM bytes per call from FETCH_SIZE/WRITE_SIZE counter "
                                     "passes scaled by a copy of known size; null when the "
                                     "decode sources changed since",
                     "kernel": "pa_decode_append (decode_kernel with the newest token's "
                               "append, one launch), one layer: "
                               f"{int(last_lens.sum())} tokens x 4096 B read + {B} x 4096 B "
                               "written",
                     "us_per_launch": round(us_launch, 3),
                     "us_per_launch_median": round(p50, 3), "us_per_launch_p10": round(p10, 3),
                     "us_per_launch_p90": round(p90, 3),
                     "timing": f"{args.kernel_reps} replays of a graph of {nl} pa_decode_append "
                               f"calls, one per layer pool; mean over all {launches} calls, "
                               "median and p10/p90 of the per-replay means",
                     "algorithmic_bytes_per_call": alg_launch,
                     "decode_only": {
                         "kernel": "pa_decode alone on the prefilled cache, one layer, "
                                   f"{int(lens_np.sum())} tokens x 4096 B",
                         "us_per_launch": round(us_dec, 3),
                         "us_per_launch_median": round(d50, 3),
                         "us_per_launch_p10": round(d10, 3), "us_per_launch_p90": round(d90, 3),
                         "achieved": round(achieved_dec, 1),
                         "frac": round(achieved_dec / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(key="decode_only_traffic_bytes_per_call"),
                         "algorithmic_bytes_per_call": kv_dec,
                         "mall_warm_us_per_launch": round(us_warm, 3),
                         "floor_us": floor["read_tiles_us"],
                         "floor": floor}},
    }
    cb = copy_bandwidth(dev)
    result["roofline"]["copy_1gib"] = cb
    log(f"1 GiB device copy: {cb['read_plus_write_GBps']:.0f} GB/s read + write")
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)...")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
