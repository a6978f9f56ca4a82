#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV cache hot path on one MI355X.

A step is one pass of the whole path for one batch of sequences: every
sequence appends one token (host block allocator: slot, new block every 16th
token, copy-on-write pairs), the copy-on-write block copies run, the new
token's K/V are written into its slot, and paged decode attention runs over
each sequence's whole cached context (plus the log-sum-exp merge when the
sequence is split into partitions).  By default the device part of a step is
one paged_decode_step call (copy, write and decode fused in one launch);
--unfused runs paged_copy_blocks + paged_kv_write + paged_attention_decode.

The host allocator's results for all steps are computed before the timed
region and uploaded, so the timed steps read resident inputs; the allocator's
own cost is reported separately (host_alloc_us_per_step).  The timed steps are
captured in one HIP graph, replayed once untimed and then five times, each
replay timed on its own; the median is reported.  Several disjoint batches from
one block pool are used in rotation so that the working set exceeds the 256 MB
Infinity Cache and the KV reads come from HBM (stand-in for the per-layer
caches of a real model).

value = KV bytes read per step / step time (GB/s).  roofline: the decode
call's algorithmic bytes per launch (each physical block once) / its average
duration (HIP events around graph replays of back-to-back decode launches on
the launch stream, median of five).  The default run reports the
Qwen3-32B-shaped layer and, in "configs", the 8 x 32K split-K decode, the
quantized decode over int8 and E4M3 caches and the shared-prefix step, each
measured the same way in the same process.
cpu_baseline: the fp64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
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
METRIC = "paged-attn decode KV-read GB/s (% of MI355X HBM peak) + decoded seqs/s"
EB = {"f32": 4, "f16": 2, "i8": 1, "e4m3": 1}


def _workloads():
    from synth import workloads as W
    return {
        # name: (factory(replica) -> Workload, replicas, pool blocks or None)
        "c2": (lambda r: W.c2_qwen3_32b_layer(seed_offset=r), 8, 12480),
        "c3": (lambda r: W.c3_long_context(), 1, None),
        # the same long uniform sequences over an int8 / E4M3 cache
        "c3_i8": (lambda r: _quantized(W.c3_long_context(), "i8"), 1, None),
        "c3_e4m3": (lambda r: _quantized(W.c3_long_context(), "e4m3"), 1, None),
        "c4_i8": (lambda r: W.c4_quantized("i8"), 2, None),
        "c4_e4m3": (lambda r: W.c4_quantized("e4m3"), 2, None),
        "c5": (lambda r: W.c5_shared_prefix(), 2, 8192),
        "c5_cow": (lambda r: W.c5_shared_prefix(cow_pairs=True), 2, 8192),
        "c1": (lambda r: W.c1_tiny(), 1, None),
        # multi-token queries: 8 x (1536 cached + 512 new tokens), bench_prefill
        "prefill": (lambda r: W.chunked_prefill(), 1, None),
        # block swap to pinned host memory and back, bench_swap
        "swap": (lambda r: W.c2_qwen3_32b_layer(), 1, None),
    }


def _quantized(w, cache_dtype: str):
    """Workload `w` with its fp16 K/V stored in an int8 or E4M3 cache (the
    cache write quantizes them)."""
    w.cache_dtype = cache_dtype
    w.name += "_" + cache_dtype
    return w


def kv_bytes(lens, w) -> int:
    """Algorithmic bytes one decode launch must move (KV, scales, q, out, tables, lens)."""
    lens = np.asarray(lens, np.int64)
    tok = int(lens.sum())
    b = tok * w.num_kv_heads * 2 * w.head_dim * EB[w.cache_dtype]
    if w.cache_dtype in ("i8", "e4m3"):
        b += tok * w.num_kv_heads * 2 * 2
    b += len(lens) * w.num_heads * w.head_dim * (EB[w.q_dtype] + EB[w.out_dtype])
    b += 4 * int(np.sum((lens + w.block_size - 1) // w.block_size)) + 4 * len(lens)
    return b


def kv_bytes_shared(sh, w) -> int:
    """Algorithmic bytes of one shared-prefix decode call: each group's prefix
    once, every suffix, q and out of every sequence, both tables."""
    pieces = np.concatenate([np.asarray(sh["suffix_lens"], np.int64),
                             np.asarray(sh["group_prefix_lens"], np.int64)])
    b = kv_read_bytes(pieces, w)
    b += len(sh["suffix_lens"]) * w.num_heads * w.head_dim * (EB[w.q_dtype] + EB[w.out_dtype])
    b += 4 * int(np.sum((pieces + w.block_size - 1) // w.block_size)) + 4 * len(pieces)
    return b


def kv_read_bytes(lens, w) -> int:
    tok = int(np.asarray(lens, np.int64).sum())
    b = tok * w.num_kv_heads * 2 * w.head_dim * EB[w.cache_dtype]
    if w.cache_dtype in ("i8", "e4m3"):
        b += tok * w.num_kv_heads * 2 * 2
    return b


def cpu_baseline(w, budget_s: float = 10.0):
    """Time the oracle (as it stands) on a bounded sample of one batch: the
    first k sequences (k grown until one pass takes at least 0.5 s, or the
    whole batch), passed over repeatedly until budget_s seconds have gone (at
    least three passes); the rate is that of the median pass."""
    import oracle
    from oracle.replay import replay as oracle_replay
    ro = oracle_replay(w)
    n = len(w.decode_seqs)
    lens = ro.seq_lens
    k = min(n, 4)
    while True:
        t0 = time.perf_counter()
        _, used = oracle.decode(ro.pools, ro.q[:k], ro.block_tables[:k], lens[:k],
                                np.float32(w.scale))
        dt = time.perf_counter() - t0
        if dt >= 0.5 or k >= n:
            break
        k = min(n, k * 4)
    passes = [dt]
    while sum(passes) < budget_s or len(passes) < 3:
        t0 = time.perf_counter()
        oracle.decode(ro.pools, ro.q[:k], ro.block_tables[:k], lens[:k], np.float32(w.scale))
        passes.append(time.perf_counter() - t0)
    reps, elapsed = len(passes), sum(passes)
    per = float(np.median(passes))
    b = kv_read_bytes(lens[:k], w)
    # the same oracle on one thread (after the timing above: the thread count
    # set here stays for the rest of the process), first sequence only
    passes1 = []
    while sum(passes1) < min(3.0, budget_s) or len(passes1) < 3:
        t0 = time.perf_counter()
        oracle.decode(ro.pools, ro.q[:1], ro.block_tables[:1], lens[:1], np.float32(w.scale),
                      num_threads=1)
        passes1.append(time.perf_counter() - t0)
    reps1, el1 = len(passes1), sum(passes1)
    per1 = float(np.median(passes1))
    return {"value": round(b / per / 1e9, 4), "unit": "GB/s", "cores": int(used),
            "kind": "oracle",
            "sample": f"{k} of {n} sequences of one batch ({int(lens[:k].sum())} tokens), "
                      f"fp64, {reps} pass(es) in {elapsed:.1f} s, median {per:.3f} s per pass",
            "seqs_per_s": round(k / per, 3),
            "one_core": {"value": round(kv_read_bytes(lens[:1], w) / per1 / 1e9, 4),
                         "unit": "GB/s", "cores": 1,
                         "sample": f"sequence 0 ({int(lens[0])} tokens), {reps1} pass(es) "
                                   f"in {el1:.1f} s"}}


BENCH_KERNELS_SRC = os.path.join(ROOT, "bench_kernels.hip")
BENCH_KERNELS_LIB = os.path.join(ROOT, "libpkv_bench.so")
_bench_lib = None


def build_bench_kernels() -> str:
    """Compile the benchmark's bandwidth-diagnostic kernels (bench_kernels.hip,
    not part of libpkv) into libpkv_bench.so beside this file."""
    import subprocess
    from paged_kv_cache_387_amd import build as B
    tmp = BENCH_KERNELS_LIB + f".tmp{os.getpid()}"
    subprocess.run([B.HIPCC, *B.HIP_FLAGS, "-shared", BENCH_KERNELS_SRC, "-o", tmp], check=True,
                   capture_output=True)
    os.replace(tmp, BENCH_KERNELS_LIB)
    return BENCH_KERNELS_LIB


def bench_lib():
    global _bench_lib
    if _bench_lib is None:
        if not os.path.exists(BENCH_KERNELS_LIB):
            raise ImportError(f"{BENCH_KERNELS_LIB} is not built (bench.build_bench_kernels)")
        L = ctypes.CDLL(BENCH_KERNELS_LIB)
        P, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        L.bench_stream_read.argtypes = [P, sz, P, i32, P]
        L.bench_stream_copy.argtypes = [P, P, sz, i32, i32, P]
        L.bench_stream_read.restype = L.bench_stream_copy.restype = ctypes.c_int
        _bench_lib = L
    return _bench_lib


def _stream(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def read_ceiling(torch, nbytes: int = 2 << 30, reps: int = 10):
    """Achievable streaming-read bandwidth (GB/s) of this device: a plain
    non-temporal read over nbytes, the best of a sweep of grid sizes."""
    L = bench_lib()
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    best = 0.0
    for wgs in (256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536):
        sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
        args = (ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), wgs,
                _stream(torch))
        assert L.bench_stream_read(*args) == 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            L.bench_stream_read(*args)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    return round(best, 1)


def pmc_copy(nbytes: int = 1 << 30, reps: int = 5, nontemporal: bool = True) -> int:
    """Run a plain copy of nbytes a few times: the known-size reference for
    scaling hardware byte counters (FETCH_SIZE / WRITE_SIZE).  Non-temporal
    loads and stores by default, as the decode kernel reads K/V."""
    import torch
    L = bench_lib()
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    dst = torch.empty_like(src)
    for _ in range(reps):
        assert L.bench_stream_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                   nbytes, 4096, int(nontemporal), _stream(torch)) == 0
    torch.cuda.synchronize()
    print(json.dumps({"pmc_copy_bytes": nbytes, "launches": reps,
                      "nontemporal": bool(nontemporal)}), flush=True)
    return 0


# Sources that determine what one paged_attention_decode call moves: the
# counter-based traffic figure is used only while these are unchanged.
DECODE_SOURCES = ("decode_kernel.h", "decode.hip", "decode_runs.hip", "decode_stream.hip",
                  "api.hip", "pkv_internal.h", "attn_common.h", "kv_write.h")


# Sources of the multi-query passes (shared prefixes, multi-token queries).
PASS_SOURCES = ("prefix.hip", "prefix_pipe.hip", "lds_ring.h", "api.hip", "pkv_internal.h",
                "attn_common.h")


def decode_source_hash(files=DECODE_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "paged_kv_cache_387_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def source_line() -> str:
    return (f"# source={decode_source_hash()}  (hash of the decode sources); "
            f"pass_source={decode_source_hash(PASS_SOURCES)}  (of the multi-query passes)")


def read_traffic(workload: str):
    """HBM bytes per paged_attention_decode call from the committed counter
    summary of this workload, or None if absent or taken on other sources."""
    tpath = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(tpath):
        return None
    sha = decode_source_hash()
    for line in open(tpath):
        if line.startswith("traffic_bytes_per_launch") and f"source={sha}" in line:
            return int(line.split()[1])
    return None


def summarize_traffic(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv,
                      commands):
    """Write profiles/traffic_<workload>.txt from rocprofv3 --pmc FETCH_SIZE /
    WRITE_SIZE counter CSVs of the decode run and of the copy calibration run
    (bench.py --pmc-copy, 1 GiB).  Counters are KiB per dispatch; each is scaled
    by (true bytes of the copy) / (what the counter read for the copy)."""
    import csv
    import collections

    def per_kernel(path):
        agg = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return agg

    def copy_value(path):
        vals = [v for k, vs in per_kernel(path).items() if "stream_copy_kernel" in k for v in vs]
        return sum(vals) / len(vals)

    nbytes = 1 << 30
    f_scale = nbytes / 1024.0 / copy_value(copy_fetch_csv)
    w_scale = nbytes / 1024.0 / copy_value(copy_write_csv)
    fetch, write = per_kernel(fetch_csv), per_kernel(write_csv)
    def is_plain_decode(name):
        # decode_kernel<KV, D, OUT, SRC, BS>: SRC = -1 is paged_attention_decode, any
        # other value the fused step (which also writes the new token)
        args = name.split("decode_kernel<", 1)[1].split(">", 1)[0].split(",")
        return int(args[3]) == -1

    lines, total = [], 0.0
    for name in sorted(fetch):
        if "decode_kernel" not in name and "merge_kernel" not in name:
            continue
        fk = sum(fetch[name]) / len(fetch[name])
        wk = sum(write.get(name, [0.0])) / max(1, len(write.get(name, [])))
        b = (fk * f_scale + wk * w_scale) * 1024.0
        counted = "merge_kernel" in name or is_plain_decode(name)
        if counted:
            total += b
        lines.append(f"  {name}\n    dispatches {len(fetch[name])}  FETCH_SIZE {fk:.1f} KiB  "
                     f"WRITE_SIZE {wk:.1f} KiB  -> {b / 1e6:.3f} MB per dispatch (scaled)"
                     + ("" if counted else "  [fused step: not part of the decode call]"))
    out = [f"# HBM traffic per paged_attention_decode call, workload {workload}",
           "# commands (run from the repository root on the GPU host):"]
    out += [f"#   {c}" for c in commands]
    out += [f"copy calibration: 1 GiB copy reads FETCH_SIZE {copy_value(copy_fetch_csv):.1f} KiB, "
            f"WRITE_SIZE {copy_value(copy_write_csv):.1f} KiB -> scale fetch x{f_scale:.4f}, "
            f"write x{w_scale:.4f}", "kernels:"] + lines
    out.append(f"traffic_bytes_per_launch {int(round(total))} source={decode_source_hash()}")
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    open(path, "w").write("\n".join(out) + "\n")
    print("\n".join(out))
    return 0


def summarize_trace(workload, trace_csv, stats_csv, commands):
    """Write profiles/decode_<workload>_kernel_trace.txt from the rocprofv3
    --kernel-trace --stats CSVs of a bench run: the kernel statistics and the
    library's kernels per launch shape (rows with at least 5 launches)."""
    import csv
    import collections
    import re

    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        name = r["Kernel_Name"]
        if "pkv::" not in name:
            continue
        short = re.sub(r"^void ", "", name).replace("pkv::(anonymous namespace)::", "")
        short = short.split("(pkv::")[0]
        agg[(short, r["Grid_Size_X"], r["Grid_Size_Y"])].append(
            int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = [f"# rocprofv3 kernel trace summary, workload {workload}: kernels of the library "
           f"(decode_kernel<KV, D, OUT, SRC, BS, WALK>: SRC >= 0 is the fused step, -1 the plain "
           f"decode; prefix32_kernel<KV, D, BS, MODE, OUT> and pipe32_kernel<D, BS, MODE, OUT, "
           f"TG>: MODE 0 shared prefix, 1 prefill)",
           "# commands (run from the repository root on the GPU host):"]
    out += [f"#   {c}" for c in commands]
    out.append(source_line())
    out.append("# run_kernel_stats.csv (durations in ns; the bench setup's bulk cache writes and "
               "host copies are included):")
    out += [line.rstrip("\n") for line in open(stats_csv)]
    out.append("# per (kernel, grid) from run_kernel_trace.csv, rows with >= 5 launches (grid in "
               "threads):")
    out.append(f"{'kernel':44s} {'grid_x':>9s} {'grid_y':>6s} {'calls':>6s} {'avg_us':>9s} "
               f"{'min_us':>9s} {'max_us':>9s}")
    for k, v in sorted(agg.items(), key=lambda kv: -len(kv[1])):
        if len(v) >= 5:
            out.append(f"{k[0]:44s} {k[1]:>9s} {k[2]:>6s} {len(v):6d} {sum(v) / len(v) / 1e3:9.2f} "
                       f"{min(v) / 1e3:9.2f} {max(v) / 1e3:9.2f}")
    name = f"{workload}_kernel_trace.txt" if workload == "prefill" else \
        f"decode_{workload}_kernel_trace.txt"
    path = os.path.join(ROOT, "profiles", name)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    open(path, "w").write("\n".join(out) + "\n")
    print("\n".join(out))
    return 0


def summarize_counters(name, csv_path, commands, kernels=("decode_kernel", "prefix32_kernel",
                                                         "pipe32_kernel", "merge_kernel")):
    """Write profiles/<name>_sq_counters.txt from rocprofv3 --pmc counter CSVs
    (one per pass, comma-separated): each library kernel's counters averaged
    over its dispatches."""
    import csv
    import collections
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    rows = [r for path in csv_path.split(",") for r in csv.DictReader(open(path))]
    for r in rows:
        k = r["Kernel_Name"]
        if any(x in k for x in kernels):
            short = k.replace("void ", "").replace("pkv::(anonymous namespace)::", "")
            short = short.split("(pkv::")[0]
            agg[short][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = [f"# rocprofv3 counters per dispatch (averages), {name}",
           "# commands (run from the repository root on the GPU host):"]
    out += [f"#   {c}" for c in commands]
    out.append(source_line())
    for k, v in sorted(agg.items()):
        n = max(len(x) for x in v.values())
        out.append(f"{k}  ({n} dispatches)")
        for c, vals in sorted(v.items()):
            out.append(f"  {c:28s} {sum(vals) / len(vals):18.1f}")
    path = os.path.join(ROOT, "profiles", f"{name}_sq_counters.txt")
    open(path, "w").write("\n".join(out) + "\n")
    print("\n".join(out))
    return 0


MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 MFMA


def prefill_flops(w) -> float:
    """q.K and P.V flops of one multi-token-query call: query i of a chunk of
    n at the end of L tokens sees L - n + i + 1 of them."""
    tot = 0
    lens = [op[2] for op in w.ops if op[0] == "allocate"]
    for L, n in zip(lens, w.q_lens):
        tot += sum(L - n + i + 1 for i in range(n))
    return 4.0 * w.head_dim * w.num_heads * tot


def bench_prefill(args, torch, pkv, driver) -> int:
    """A chunked-prefill step: the chunk's K/V written into its slots
    (paged_kv_write) and its queries' causal attention over the cache
    (paged_attention_prefill), captured in a graph."""
    from synth import workloads as W
    w = W.chunked_prefill(cache_dtype=args.kv_dtype)
    if args.block_size != 16:
        w = W.with_block_size(w, args.block_size)
    K, Wm = args.steps, args.warmup
    part = 0 if args.partition < 0 else args.partition
    r = driver.replay(w)
    T = sum(w.q_lens)
    offs = w.q_offsets()
    # the chunk tokens' slots and values (rewritten by every step)
    slots, ks, vs = [], [], []
    for sidx, seq in enumerate(w.decode_seqs):
        L = int(r.lens_host[sidx])
        n = w.q_lens[sidx]
        slots.append(r.alloc.slots(seq, L - n, n))
        ks.append(w.kv_rows("k", seq, L - n, n))
        vs.append(w.kv_rows("v", seq, L - n, n))
    slot_t = torch.from_numpy(np.concatenate(slots)).cuda()
    k_t = torch.from_numpy(np.concatenate(ks)).cuda()
    v_t = torch.from_numpy(np.concatenate(vs)).cuda()
    out = torch.empty((T, w.num_heads, w.head_dim), dtype=torch.float16, device="cuda")
    off_t = torch.from_numpy(offs).cuda()
    scale = float(np.float32(w.scale))
    maxq = max(w.q_lens)
    need = pkv.prefill_workspace_bytes(w.num_seqs, T, maxq, w.num_heads, w.num_kv_heads,
                                       w.head_dim, w.max_blocks_per_seq, part, w.block_size)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")

    def attn():
        pkv.paged_attention_prefill(r.query, r.cache, r.block_tables, r.seq_lens, off_t, scale,
                                    maxq, out=out, partition_size=part, workspace=ws)

    def step():
        pkv.paged_kv_write(k_t, v_t, slot_t, r.cache)
        attn()

    def timed(fn, n):
        for _ in range(Wm):
            fn()
        torch.cuda.synchronize()
        return float(np.median(graph_ms(torch, [fn] * n))) / n

    step_ms = timed(step, K)
    attn_ms = timed(attn, K)
    fl = prefill_flops(w)
    achieved = fl / (attn_ms * 1e-3) / 1e12
    result = {
        "metric": "paged prefill attention TFLOP/s (chunked prefill over the paged cache)",
        "value": round(fl / (step_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": Wm, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.cache_dtype, "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "query_tokens": T,
                   "context_plus_chunk": int(r.lens_host.max()), "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "kv_dtype": w.cache_dtype,
                   "partition_size": part, "graph": True},
        "tokens_per_s": round(T / (step_ms * 1e-3), 1),
        "attention_ms": round(attn_ms, 5),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                     "traffic": None, "flops_per_launch": fl},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        from oracle.replay import replay as oracle_replay
        ro = oracle_replay(w)
        # sample: the last query rows of the first sequence (the longest views)
        n = 8
        L = int(ro.seq_lens[0])
        rows = np.arange(offs[1] - n, offs[1])
        lens = np.array([L - w.q_lens[0] + (rw - offs[0]) + 1 for rw in rows], np.int32)
        tables = np.repeat(ro.block_tables[:1], n, axis=0)
        t0, reps, used = time.perf_counter(), 0, 1
        while time.perf_counter() - t0 < args.cpu_budget:
            _, used = oracle.decode(ro.pools, ro.q[rows], tables, lens, np.float32(w.scale))
            reps += 1
        dt = time.perf_counter() - t0
        fl_s = 4.0 * w.head_dim * w.num_heads * float(lens.sum()) * reps
        result["cpu_baseline"] = {"value": round(fl_s / dt / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": int(used), "kind": "oracle",
                                  "sample": f"{n} query rows of sequence 0 (views of {lens.min()}-"
                                            f"{lens.max()} tokens), {reps} passes in {dt:.1f} s"}
    print(json.dumps(result), flush=True)
    return 0


HOST_LINK_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction


def bench_swap(args, torch, pkv) -> int:
    """Whole-block copies between the device pools and a pinned host pool
    (paged_swap_blocks) for 4096 blocks of the C2 layer's shape (16 tokens x
    8 kv heads x 128 x fp16: 64 KiB of K+V per block, 256 MiB), each
    direction timed over a graph of repeated copies."""
    nb = 4096
    cache = pkv.PagedKVCache(nb, 8, 128, "f16", fill_byte=0x3C)
    host = pkv.HostKVPool(nb, cache)
    rng = np.random.default_rng(0)
    dev_ids = rng.permutation(nb).astype(np.int32)
    host_ids = np.arange(nb, dtype=np.int32)
    out_pairs = torch.from_numpy(np.stack([dev_ids, host_ids], 1).copy()).cuda()
    in_pairs = torch.from_numpy(np.stack([host_ids, dev_ids], 1).copy()).cuda()
    nbytes = 2 * cache.k.numel()

    def timed(fn, reps=5):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        return float(np.median(graph_ms(torch, [fn] * reps))) / reps

    out_ms = timed(lambda: pkv.paged_swap_blocks(cache, host, out_pairs, to_host=True))
    in_ms = timed(lambda: pkv.paged_swap_blocks(cache, host, in_pairs, to_host=False))
    gbs_out = nbytes / (out_ms * 1e-3) / 1e9
    gbs_in = nbytes / (in_ms * 1e-3) / 1e9
    best = max(gbs_out, gbs_in)
    result = {
        "metric": "paged block swap GB/s (device <-> pinned host, whole blocks)",
        "value": round((gbs_out + gbs_in) / 2, 2), "unit": "GB/s", "n_gpus": 1, "steps": 5,
        "warmup": 2, "ms_per_step": round(out_ms + in_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "swap", "blocks": nb, "block_bytes_kv": nbytes // nb,
                   "num_kv_heads": 8, "head_dim": 128, "block_size": 16},
        "swap_out_gbs": round(gbs_out, 2), "swap_in_gbs": round(gbs_in, 2),
        "roofline": {"bound": "host-link", "achieved": round(best, 2),
                     "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                     "frac": round(best / HOST_LINK_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_len_sweep(args, torch, pkv) -> int:
    """Cost of one paged_attention_decode call at the Qwen3-32B layer shape
    (32 sequences, 64 query / 8 kv heads, head_dim 128, fp16, 12480-block
    pool) against the sequence length: every sequence gets the same length,
    then the configuration's U[512, 768] mix.  Eight disjoint sets of block
    tables (a seeded permutation of the pool) rotate, as in the main bench.
    A straight-line fit over lengths >= 256 gives the fixed cost per call (the
    intercept) and the streaming rate of the KV bytes beyond it (the slope)."""
    S, H, HKV, D, NBLK, MAXB, R = 32, 64, 8, 128, 12480, 48, 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(387)
    cache = pkv.PagedKVCache(NBLK, HKV, D, "f16")
    cache.k.view(torch.float16).normal_(generator=gen)
    cache.v.view(torch.float16).normal_(generator=gen)
    rng = np.random.default_rng(387)
    perm = rng.permutation(NBLK)[: R * S * MAXB].reshape(R, S, MAXB).astype(np.int32)
    tables = [torch.from_numpy(perm[r].copy()).cuda() for r in range(R)]
    q = torch.randn(S, H, D, device="cuda", generator=gen).half()
    out = torch.empty(S, H, D, device="cuda", dtype=torch.float16)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    n = max(R, args.steps)

    def per_call_us(lens_np):
        lens = torch.from_numpy(lens_np.astype(np.int32)).cuda()
        for r in range(R):
            pkv.paged_attention_decode(q, cache, tables[r], lens, scale, out=out)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                pkv.paged_attention_decode(q, cache, tables[i % R], lens, scale, out=out)
        g.replay()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / n)
        return best

    rows, fit_x, fit_y = [], [], []
    for L in (0, 1, 16, 128, 256, 384, 512, 640, 768):
        us = per_call_us(np.full(S, L))
        kv = S * L * HKV * 2 * D * 2
        rows.append({"len": L, "us": round(us, 3), "kv_gbs": round(kv / us / 1e3, 1)})
        print(f"# len {L:4d}: {us:7.2f} us per call", file=sys.stderr, flush=True)
        if L >= 256:
            fit_x.append(kv)
            fit_y.append(us)
    mix = rng.integers(512, 769, S)
    us = per_call_us(mix)
    kv = int(mix.sum()) * HKV * 2 * D * 2
    rows.append({"len": "U[512,768]", "us": round(us, 3), "kv_gbs": round(kv / us / 1e3, 1)})
    slope, icept = np.polyfit(np.asarray(fit_x, np.float64), np.asarray(fit_y, np.float64), 1)
    print(json.dumps({
        "metric": "paged_attention_decode cost per call vs sequence length (Qwen3-32B layer shape)",
        "config": {"workload": "qwen3_32b_layer_len_sweep", "num_seqs": S, "num_heads": H,
                   "num_kv_heads": HKV, "head_dim": D, "kv_dtype": "f16", "pool_blocks": NBLK,
                   "rotating_batches": R, "calls_per_graph": n},
        "points": rows,
        "fit_len_ge_256": {"fixed_us": round(float(icept), 3),
                           "marginal_gbs": round(1e-3 / float(slope), 1)},
    }), flush=True)
    return 0


def unique_kv_bytes(tables, lens, w) -> int:
    """Algorithmic bytes of one decode call counting each physical block once:
    a block that several sequences share (a forked prefix) is read for all of
    them from the same place, so it counts once, with its filled tokens.  Plus
    q, out, the table entries and the lengths, as kv_bytes."""
    bs = w.block_size
    filled = {}
    ntab = 0
    for row, L in zip(tables, lens):
        nb = -(-int(L) // bs)
        ntab += nb
        for i in range(nb):
            b = int(row[i])
            filled[b] = max(filled.get(b, 0), min(bs, int(L) - i * bs))
    b = kv_read_bytes([sum(filled.values())], w)
    b += len(lens) * w.num_heads * w.head_dim * (EB[w.q_dtype] + EB[w.out_dtype])
    return b + 4 * ntab + 4 * len(lens)


TIMED_REPLAYS = 5


def graph_ms(torch, calls, reps: int = TIMED_REPLAYS):
    """Capture `calls` (a list of no-argument launches) in one HIP graph,
    replay it once untimed, then `reps` times, each timed with HIP events on
    the launch stream and synchronized on both sides.  Returns the
    milliseconds of each timed replay."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    del g
    return out


def measure(args, name: str, torch, pkv, driver, shared: bool = False, partition: int = -1,
            steps: int = 200, warmup: int = 20, block_size: int = 16, replicas: int = 0,
            unfused: bool = False, no_graph: bool = False, memo=None):
    """One workload's decode steps, timed: returns the result fields (value,
    ms_per_step, roofline, ...) of its bench line."""
    factory, replicas_default, pool = _workloads()[name]
    R = replicas or replicas_default
    bs = block_size
    ws = [factory(r) for r in range(R)]
    if bs != 16:
        from synth.workloads import with_block_size
        ws = [with_block_size(w, bs) for w in ws]
        pool = pool and -(-pool * 16 // bs)   # the same token capacity
    w0 = ws[0]
    K, Wm = steps, warmup
    total_steps = Wm + K
    growth = -(-total_steps // R) + 1
    max_len = max(max(int(op[2]) for op in w.ops if op[0] == "allocate") for w in ws)
    maxb = -(-(max_len + growth) // bs)
    need_blocks = sum(sum(-(-int(op[2]) // bs) for op in w.ops if op[0] == "allocate")
                      for w in ws)
    num_blocks = pool or int(math.ceil((need_blocks + R * len(w0.decode_seqs) * (growth // bs + 2))
                                       * 1.1))
    if pool and num_blocks == w0.num_blocks:
        order = w0.free_order
    else:
        from synth import permutation, stream_key
        order = permutation(stream_key(w0.seed, "bench_pool"), num_blocks)
    part = w0.partition_size if partition < 0 else partition
    print(f"# setup {name}: {R} batch(es) of {w0.num_seqs} seqs, pool {num_blocks} "
          f"blocks, table width {maxb}, partition {part}", file=sys.stderr, flush=True)

    alloc = pkv.BlockAllocator(num_blocks, bs, order)
    cache = pkv.PagedKVCache(num_blocks, w0.num_kv_heads, w0.head_dim, w0.cache_dtype,
                             block_size=bs)
    OFF = 1 << 24
    batches = []
    for r, w in enumerate(ws):
        if memo is not None:      # K/V rows shared with another run of the same script
            w.memo = memo.setdefault(r, {})
        driver.replay(w, alloc=alloc, cache=cache, seq_offset=r * OFF, stop_at_step=True)
        w.memo = None
        seqs = [s + r * OFF for s in w.decode_seqs]
        q = torch.from_numpy(w.query()).cuda()
        rng = np.random.default_rng(r)
        newk = torch.from_numpy(rng.standard_normal(
            (len(seqs), w.num_kv_heads, w.head_dim)).astype(np.float16)).cuda()
        newv = torch.from_numpy(rng.standard_normal(
            (len(seqs), w.num_kv_heads, w.head_dim)).astype(np.float16)).cuda()
        if w.src_dtype == "f32":
            newk, newv = newk.float(), newv.float()
        odt = torch.float16 if w.out_dtype == "f16" else torch.float32
        out = torch.empty((len(seqs), w.num_heads, w.head_dim), dtype=odt, device="cuda")
        batches.append(dict(seqs=seqs, ids=np.ascontiguousarray(seqs, dtype=np.int64), q=q,
                            k=newk, v=newv, out=out))
    torch.cuda.synchronize()

    # host allocator for every step, ahead of time: one pkv_seq_step call per
    # step (appends, copy sources, tables, lengths), timed around the C call
    # itself; the same call with an empty batch (argument passing only) is
    # timed too and subtracted, which leaves the allocator's own work
    steps_l = []
    t_host, t_empty = 0.0, 0.0
    L_ = pkv.lib()
    n_ = len(batches[0]["seqs"])
    buf = {"tables": np.empty((n_, maxb), np.int32), "lens": np.empty(n_, np.int32),
           "cow_src": np.empty(n_, np.int32), "slots": np.empty(n_, np.int64)}
    ptrs = [b_.ctypes.data_as(ctypes.c_void_p) for b_ in
            (buf["slots"], buf["cow_src"], buf["tables"], buf["lens"])]
    for i in range(total_steps):
        b = batches[i % R]
        ids = b["ids"]
        idp = ids.ctypes.data_as(ctypes.c_void_p)
        t0 = time.perf_counter()
        st_ = L_.pkv_seq_step(alloc._h, idp, n_, maxb, *ptrs)
        t1 = time.perf_counter()
        L_.pkv_seq_step(alloc._h, idp, 0, maxb, *ptrs)
        t2 = time.perf_counter()
        if st_ != 0:
            raise pkv.PkvError(st_, "pkv_seq_step")
        t_host += t1 - t0
        t_empty += t2 - t1
        tables, lens = buf["tables"].copy(), buf["lens"].copy()
        src, slots = buf["cow_src"].copy(), buf["slots"].copy()
        sh = alloc.export_shared(b["seqs"], maxb, maxb) if shared else None
        pairs = np.stack([src, tables[np.arange(n_), (lens - 1) // bs]], 1)[src >= 0]
        steps_l.append(dict(b=i % R, slots=torch.from_numpy(slots).cuda(),
                            cow_src=torch.from_numpy(src).cuda(),
                            pairs=torch.from_numpy(np.ascontiguousarray(pairs)).cuda()
                            if len(pairs) else None, npairs=len(pairs),
                            tables=torch.from_numpy(tables).cuda(), tables_host=tables,
                            lens=torch.from_numpy(lens).cuda(), lens_host=lens, sh=sh))
    host_alloc_us = max(0.0, t_host - t_empty) / total_steps * 1e6
    host_call_us = t_host / total_steps * 1e6
    S, H, D, Hkv = w0.num_seqs, w0.num_heads, w0.head_dim, w0.num_kv_heads
    workspace = pkv.alloc_workspace(S, H, Hkv, D, maxb, part, block_size=bs)
    if shared:
        # suffix tables cut to the widest suffix of any step; device group arrays
        msb = max(1, max(-(-int(st["sh"]["suffix_lens"].max()) // bs) for st in steps_l))
        ws_need = 0
        for st in steps_l:
            sh = st["sh"]
            st["grp"] = pkv.PrefixGroups(sh)
            st["stables"] = torch.from_numpy(
                np.ascontiguousarray(sh["suffix_tables"][:, :msb])).cuda()
            st["slens"] = torch.from_numpy(sh["suffix_lens"]).cuda()
            ws_need = max(ws_need, pkv.shared_workspace_bytes(S, H, Hkv, D, msb, st["grp"],
                                                              part, bs))
        workspace = torch.empty(max(ws_need, 256), dtype=torch.uint8, device="cuda")
        print(f"# shared: {steps_l[0]['sh']['num_groups']} group(s), prefix "
              f"{steps_l[0]['sh']['group_prefix_lens'].tolist()}, suffix width {msb} blocks",
              file=sys.stderr, flush=True)
    scale = float(np.float32(w0.scale))
    torch.cuda.synchronize()

    def run_step(st):
        b = batches[st["b"]]
        if shared:
            pkv.paged_attention_decode_shared(b["q"], cache, st["stables"], st["slens"], scale,
                                              st["grp"], key=b["k"], value=b["v"],
                                              cow_src=st["cow_src"], out=b["out"],
                                              partition_size=part, workspace=workspace)
        elif unfused:
            if st["pairs"] is not None:
                pkv.paged_copy_blocks(cache, st["pairs"])
            pkv.paged_kv_write(b["k"], b["v"], st["slots"], cache)
            pkv.paged_attention_decode(b["q"], cache, st["tables"], st["lens"], scale,
                                       out=b["out"], partition_size=part, workspace=workspace)
        else:
            pkv.paged_decode_step(b["q"], b["k"], b["v"], cache, st["tables"], st["lens"], scale,
                                  cow_src=st["cow_src"], out=b["out"], partition_size=part,
                                  workspace=workspace)

    for st in steps_l[:Wm]:
        run_step(st)
    torch.cuda.synchronize()

    timed = steps_l[Wm:]
    if no_graph:
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for st in timed:
            run_step(st)
        ev1.record()
        torch.cuda.synchronize()
        step_reps = [ev0.elapsed_time(ev1)]
    else:
        step_reps = graph_ms(torch, [lambda st=st: run_step(st) for st in timed])
    step_ms = float(np.median(step_reps)) / K
    bytes_step = np.mean([kv_read_bytes(st["lens_host"], w0) for st in timed])
    value = bytes_step / (step_ms * 1e-3) / 1e9

    # the decode call alone: back-to-back launches in a graph, HIP events
    # around each replay, median of the replays
    last = {}
    for st in timed:
        last[st["b"]] = st
    dec_steps = [last[i % R] for i in range(K)] if len(last) == R else timed
    single_pass = pkv.workspace_bytes(S, H, Hkv, D, maxb, part, bs) == 0

    def run_decode(st):
        b = batches[st["b"]]
        if shared:
            pkv.paged_attention_decode_shared(b["q"], cache, st["stables"], st["slens"], scale,
                                              st["grp"], out=b["out"], partition_size=part,
                                              workspace=workspace)
            return
        pkv.paged_attention_decode(b["q"], cache, st["tables"], st["lens"], scale, out=b["out"],
                                   partition_size=part, workspace=workspace)

    dec_reps = graph_ms(torch, [lambda st=st: run_decode(st) for st in dec_steps])
    dec_ms = float(np.median(dec_reps)) / len(dec_steps)
    logical = np.mean([kv_bytes(st["lens_host"], w0) for st in dec_steps])
    if shared:
        dec_alg = np.mean([kv_bytes_shared(st["sh"], w0) for st in dec_steps])
    else:
        dec_alg = np.mean([unique_kv_bytes(st["tables_host"], st["lens_host"], w0)
                           for st in dec_steps])
    achieved = dec_alg / (dec_ms * 1e-3) / 1e9
    traffic = read_traffic(name) if not shared else None

    mean_len = float(np.mean([st["lens_host"].mean() for st in timed]))
    res = {
        "value": round(value, 2), "unit": "GB/s", "ms_per_step": round(step_ms, 5),
        "dtype": w0.cache_dtype,
        "config": {"workload": w0.name, "num_seqs": S, "num_heads": H, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": bs, "kv_dtype": w0.cache_dtype,
                   "mean_seq_len": round(mean_len, 1), "pool_blocks": num_blocks,
                   "rotating_batches": R, "partition_size": part,
                   "split_k": not single_pass, "graph": not no_graph,
                   "fused_step": not unfused, "shared_prefix": bool(shared)},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "seqs_per_s": round(S / (step_ms * 1e-3), 1),
        "tokens_per_s": round(S / (step_ms * 1e-3), 1),
        "host_alloc_us_per_step": round(host_alloc_us, 2),
        "host_alloc_call_us_per_step": round(host_call_us, 2),
        "decode_kernel_ms": round(dec_ms, 5),
        "timing": f"median of {len(step_reps)} graph replays of {K} steps (decode call: of "
                  f"{len(dec_reps)} replays of {len(dec_steps)} calls)",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": int(dec_alg)},
    }
    if abs(logical - dec_alg) > 0.01 * dec_alg:
        res["roofline"]["logical_bytes_per_launch"] = int(logical)
    del cache, workspace, batches, steps_l
    torch.cuda.empty_cache()
    return res, factory


# The default run's further configurations: the 8 x 32K split-K decode (its
# 512-token partitions), the quantized decode over int8 and E4M3 caches, and
# the shared-prefix step through the shared-prefix path.
DEFAULT_CONFIGS = [("c3", dict()), ("c4_i8", dict(memo="c4")), ("c4_e4m3", dict(memo="c4")),
                   ("c5", dict(shared=True))]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, choices=sorted(_workloads()),
                    help="one workload only (default: c2, plus the configurations of "
                         "DEFAULT_CONFIGS in the same line)")
    ap.add_argument("--partition", type=int, default=-1,
                    help="partition size in tokens (-1: the workload's, 0: library choice)")
    ap.add_argument("--replicas", type=int, default=0, help="rotating batches (0: default)")
    ap.add_argument("--block-size", type=int, default=16, choices=(8, 16, 32),
                    help="tokens per physical block (the pool keeps its token capacity)")
    ap.add_argument("--kv-dtype", default="f16", choices=("f16", "i8", "e4m3"),
                    help="cache dtype of the prefill workload")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--shared", action="store_true",
                    help="decode through paged_attention_decode_shared: sequences that "
                         "share prefix blocks read them once per group")
    ap.add_argument("--unfused", action="store_true",
                    help="run the step as copy + write + decode launches instead of the fused "
                         "paged_decode_step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read ceiling measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="default run: leave out the further configurations")
    ap.add_argument("--len-sweep", action="store_true",
                    help="decode cost per call against sequence length at the Qwen3-32B layer shape")
    ap.add_argument("--pmc-copy", action="store_true",
                    help="only run the plain copy kernel (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic_<workload>.txt from rocprofv3 counter CSVs "
                         "(no GPU needed)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "STATS_CSV"),
                    help="write profiles/decode_<workload>_kernel_trace.txt from rocprofv3 "
                         "kernel-trace CSVs (no GPU needed)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("NAME", "COUNTER_CSV"),
                    help="write profiles/<NAME>_sq_counters.txt from a rocprofv3 --pmc CSV "
                         "(no GPU needed)")
    ap.add_argument("--command", action="append", default=[],
                    help="with --summarize-*: command line that produced a CSV")
    args = ap.parse_args()
    default_run = args.workload is None
    workload = args.workload or "c2"
    if args.summarize_traffic:
        return summarize_traffic(workload, *args.summarize_traffic, args.command)
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters, args.command)
    if args.summarize_trace:
        wl = workload + ("_shared" if args.shared else "")
        return summarize_trace(wl, *args.summarize_trace, args.command)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this library has no "
              f"multi-GPU path.", file=sys.stderr)
        return 2

    import torch
    import paged_kv_cache_387_amd as pkv
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import hip_replay as driver   # the test side's replay of workload scripts

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    pkv.lib()
    torch.cuda.set_device(0)
    if args.pmc_copy:
        return pmc_copy()
    if args.len_sweep:
        return bench_len_sweep(args, torch, pkv)
    if workload == "prefill":
        return bench_prefill(args, torch, pkv, driver)
    if workload == "swap":
        return bench_swap(args, torch, pkv)

    K, Wm = args.steps, args.warmup
    res, factory = measure(args, workload, torch, pkv, driver, shared=args.shared,
                           partition=args.partition, steps=K, warmup=Wm,
                           block_size=args.block_size, replicas=args.replicas,
                           unfused=args.unfused, no_graph=args.no_graph)
    result = {"metric": METRIC, "value": res.pop("value"), "unit": res.pop("unit"),
              "n_gpus": 1, "steps": K, "warmup": Wm, "ms_per_step": res.pop("ms_per_step"),
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": res.pop("dtype"), "data": "synthetic", "config": res.pop("config")}
    result.update(res)
    result["cpu_baseline"] = None
    result["hbm_read_ceiling_gbs"] = None if args.no_ceiling else read_ceiling(torch)
    if default_run and not args.no_configs:
        configs, memos = {}, {}
        for name, kw in DEFAULT_CONFIGS:
            memo = memos.setdefault(kw["memo"], {}) if "memo" in kw else None
            r2, _ = measure(args, name, torch, pkv, driver, shared=kw.get("shared", False),
                            steps=K, warmup=Wm, memo=memo)
            configs[name + ("_shared" if kw.get("shared") else "")] = r2
            print(f"# {name}: {r2['decode_kernel_ms'] * 1e3:.2f} us per decode call, "
                  f"roofline frac {r2['roofline']['frac']}", file=sys.stderr, flush=True)
        memos.clear()
        result["configs"] = configs
    if not args.no_cpu_baseline:
        wb = factory(0)
        if workload == "c3":
            from synth import workloads as W
            wb = W.c3_long_context(num_seqs=1)
        result["cpu_baseline"] = cpu_baseline(wb, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
