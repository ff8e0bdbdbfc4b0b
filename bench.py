"""Paged decode attention throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--path auto|mfma|valu]
                    [--partition-tokens N] [--no-cpu-baseline] [--copy-probe] [--read-probe]

A step is one pa_attention call (pa_attention_tree for a tree of drafted
tokens) over the whole batch of the workload (every sequence, every query
head), inputs resident in HBM. Default workload: the
Llama-3-70B-shaped layer, 64 sequences x 8192 tokens, bf16, block size 32.
Prints one JSON line on stdout; progress goes to stderr.

Algorithmic bytes of a step: every sequence's K and V once
(sum_b L_b * 2 * H_kv * d * elem; for an FP8 cache d + 4 bytes per token, head
and K/V: the codes and the fp32 scale), q in and out once (2 * B * q_len *
H_q * d * elem), the block-table entries read (sum_b ceil(L_b/bs) * 4) and the
context lengths (4 * B).
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
METRIC = "KV GB/s & % of HBM peak; decode tokens/s, 70B-shape layer, 64×8192 ctx"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, lens) -> int:
    esz = cfg.elem_bytes
    if cfg.kv_dtype == "fp8":   # one byte per element plus one fp32 scale per token, head, K and V
        kv = int(lens.astype(np.int64).sum()) * 2 * cfg.num_kv_heads * (cfg.head_dim + 4)
    else:
        kv = int(lens.astype(np.int64).sum()) * 2 * cfg.num_kv_heads * cfg.head_dim * esz
    qo = 2 * cfg.batch * cfg.q_len * cfg.num_q_heads * cfg.head_dim * esz
    tables = int((-(-lens.astype(np.int64) // cfg.block_size)).sum()) * 4 + 4 * cfg.batch
    return kv + qo + tables


def cpu_baseline(w, budget_s: float = 15.0):
    """The fp64 oracle (gather through the block table, then the definition)
    on as many whole sequences as fit in about budget_s seconds."""
    from oracle import attention as oatt
    from oracle import tree as otree
    from oracle.build import build_pool
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    cfg = w.cfg
    log("cpu baseline: building the oracle's host pool")
    pool, _, tables, _ = build_pool(w, fill_nan=False)
    done, t_used = 0, 0.0
    for b in range(cfg.batch):
        t0 = time.perf_counter()
        if w.tree_parents is None:
            oatt.attention_paged_seq(w.seqs[b].q, pool, tables[b], int(w.lens[b]), cfg.q_len,
                                     cfg.num_q_heads, cfg.scale)
        else:
            otree.attention_tree_seq(w.seqs[b].q, pool, tables[b], int(w.lens[b]), cfg.q_len,
                                     otree.ancestor_masks(w.tree_parents[b]), cfg.num_q_heads, cfg.scale)
        t_used += time.perf_counter() - t0
        done += 1
        if t_used >= budget_s:
            break
    sub = w.lens[:done]
    bytes_done = algorithmic_bytes(_sub_cfg(cfg, done), sub)
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {
        "value": round(bytes_done / t_used / 1e9, 4),
        "unit": "GB/s",
        "cores": blas_threads if blas_threads else affinity,
        "kind": "oracle",
        "sample": f"{done} of {cfg.batch} sequences (all {cfg.num_q_heads} query heads, full contexts), "
                  f"{t_used:.1f} s; numpy fp64 with {blas_threads} BLAS threads on {affinity} visible cores",
        "seconds": round(t_used, 3),
        "tokens_per_s": round(done * cfg.q_len / t_used, 3),
        "affinity_cores": affinity, "cpu_count": os.cpu_count(), "blas_threads": blas_threads,
    }


def kernel_name(cfg, plan, desc) -> str:
    """Name of the main kernel pa_attention launches for this plan (as rocprofv3 shows it)."""
    if plan.path == 1:
        t = "float" if cfg.dtype == "f32" else "unsigned short"
        return f"valu_attn<{t}, {cfg.head_dim}, {cfg.block_size}>"
    base = {0: "mfma_attn", 1: "mfma_attn_balanced", 2: "mfma_attn_wave"}[plan.schedule]
    nt = plan.tiles_per_wave
    stream = "false" if desc.kv_shared else "true"
    kv8 = "true" if desc.kv_format else "false"
    tree = "true" if cfg.tree else "false"
    if plan.schedule == 2:  # one wavefront per partition, or per run of partitions
        runs = "true" if plan.partitions_per_wave > 1 else "false"
        return f"{base}<{cfg.head_dim}, {cfg.block_size}, {nt}, {stream}, {kv8}, {tree}, {runs}>"
    return f"{base}<{cfg.head_dim}, {cfg.block_size}, {nt}, {stream}, {kv8}, {tree}>"


def _code_only(text: str) -> str:
    """C++ source without its comments and with whitespace collapsed (string
    and character literals kept as they are)."""
    import re
    token = re.compile(r"//[^\n]*|/\*.*?\*/|\"(?:\\.|[^\"\\])*\"|'(?:\\.|[^'\\])*'", re.S)
    text = token.sub(lambda m: " " if m.group(0).startswith("/") else m.group(0), text)
    return " ".join(text.split())


def source_digest() -> str:
    """sha256 of the library's sources without comments or layout: counters
    taken on other code are stale, an edit of comments alone keeps them."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_218_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            h.update(_code_only(open(os.path.join(csrc, f), encoding="utf-8").read()).encode())
    return h.hexdigest()


def committed_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the main kernel from committed rocprofv3 counter
    runs (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a
    copy of known size), if they were taken on the current sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_digest() or rec.get("kernel") != kernel:
        return None
    return rec["traffic_bytes_per_launch"]


def _pmc_rows(run_dir):
    import csv
    path = os.path.join(run_dir, "run_counter_collection.csv")
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(open(path))]


def pmc_summary(workload: str, fetch_dir: str, write_dir: str, copy_bytes: int = 2**30,
                bench_json: str = None):
    """Turn two rocprofv3 --pmc runs of `bench.py --copy-probe` (FETCH_SIZE,
    then WRITE_SIZE; KiB per dispatch) into HBM bytes per launch of the main
    kernel. Each counter is scaled by copy_bytes over what it reads for the
    copy probe's dispatches (a device-to-device copy of copy_bytes)."""
    import statistics
    import workloads
    import paged_kv_cache_218_amd as pa
    if workload in workloads.SPEC_CONFIGS:
        # data-dependent bytes: taken from the bench line of the same workload
        rec = json.loads(open(bench_json).read().strip().splitlines()[-1])
        out = {"workload": workload, "kernel": rec["roofline"]["kernel"], "source_sha256": source_digest(),
               "algorithmic_bytes": rec["algorithmic_bytes"]}
        return _pmc_finish(out, fetch_dir, write_dir, copy_bytes, out["kernel"], workload)
    cfg = workloads.CONFIGS[workload]
    lens = workloads.context_lengths(cfg)
    nb = workloads.pool_blocks(cfg, lens)
    max_blocks = int(-(-int(lens.max()) // cfg.block_size))
    desc = pa.make_desc(cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size,
                        max_blocks, nb, pa.PA_DTYPE_F32 if cfg.dtype == "f32" else pa.PA_DTYPE_BF16,
                        int(lens.max()), 0, max(cfg.partition_tokens, 0), 0, int(cfg.prefix_len > 0),
                        pa.PA_KV_FP8_E4M3 if cfg.kv_dtype == "fp8" else pa.PA_KV_SAME)
    plan = pa.pa_attention_plan(desc, cfg.q_len)
    kernel = kernel_name(cfg, plan, desc)
    out = {"workload": workload, "kernel": kernel, "source_sha256": source_digest(),
           "algorithmic_bytes": algorithmic_bytes(cfg, lens)}
    return _pmc_finish(out, fetch_dir, write_dir, copy_bytes, kernel, workload)


def _pmc_finish(out, fetch_dir, write_dir, copy_bytes, kernel, workload):
    import statistics
    for name, d in (("fetch", fetch_dir), ("write", write_dir)):
        rows = _pmc_rows(d)
        copy = [v for k, v in rows if "copyBuffer" in k and v * 1024 > 0.25 * copy_bytes]
        main = [v for k, v in rows if kernel in k]
        if not copy or not main:
            raise SystemExit(f"{d}: no copy-probe or {kernel} dispatches")
        factor = copy_bytes / (statistics.median(copy) * 1024)
        out[f"{name}_kib_per_launch"] = statistics.mean(main)
        out[f"{name}_dispatches"] = len(main)
        out[f"{name}_copy_kib"] = statistics.median(copy)
        out[f"{name}_scale"] = factor
    tb = (out["fetch_kib_per_launch"] * 1024 * out["fetch_scale"]
          + out["write_kib_per_launch"] * 1024 * out["write_scale"])
    out["traffic_bytes_per_launch"] = int(round(tb))
    out["traffic_over_algorithmic"] = tb / out["algorithmic_bytes"]
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def trace_summary(run_dir: str, kernel: str, skip: int, take: int = 0):
    """Per-dispatch durations of `kernel` from a rocprofv3 --kernel-trace run
    (run_kernel_trace.csv in run_dir), in dispatch order, with the first
    `skip` dispatches (the warm-up calls) dropped and at most `take` kept
    (0: all the rest): the steady-state figures of the timed region."""
    import csv
    import statistics
    rows = [r for r in csv.DictReader(open(os.path.join(run_dir, "run_kernel_trace.csv")))
            if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    keep = rows[skip:skip + take] if take else rows[skip:]
    if not keep:
        raise SystemExit(f"{run_dir}: no {kernel} dispatches after the first {skip}")
    us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in keep]
    span = (int(keep[-1]["End_Timestamp"]) - int(keep[0]["Start_Timestamp"])) / 1e3
    out = {"kernel": kernel, "dispatches_total": len(rows), "skipped": skip, "kept": len(us),
           "mean_us": round(statistics.mean(us), 2), "median_us": round(statistics.median(us), 2),
           "min_us": round(min(us), 2), "max_us": round(max(us), 2),
           "span_per_dispatch_us": round(span / len(us), 2)}
    print(json.dumps(out))
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published (no sparsity)
SIMD_CLOCK_GHZ = 2.4             # MI355X peak engine clock


def counter_summary(workload: str, run_dirs, bench_json: str, out_dir: str = None):
    """Per-launch means of the main kernel's rocprofv3 --pmc counters (one or
    more runs of bench.py, derived metrics such as MfmaUtil, MfmaFlopsBF16,
    VALUBusy, OccupancyPercent allowed) written to
    profiles/counters_<workload>.json, stamped with the source digest.
    bench_json: a bench line of the same workload, whose launch time turns the
    MFMA flops per launch into a rate; its kernel name selects the dispatches."""
    import csv
    import statistics
    rec = json.loads(open(bench_json).read().strip().splitlines()[-1])
    kernel = rec["roofline"]["kernel"]
    launch_us = rec["roofline"]["launch_us"]
    values = {}
    for d in run_dirs:
        rows = [r for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv")))
                if kernel in r["Kernel_Name"]]
        if not rows:
            raise SystemExit(f"{d}: no {kernel} dispatches")
        for r in rows:
            values.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = {"workload": workload, "kernel": kernel, "source_sha256": source_digest(),
           "launch_us": launch_us, "dispatches": {k: len(v) for k, v in values.items()},
           "per_launch": {k: statistics.mean(v) for k, v in values.items()}}
    flops = out["per_launch"].get("MfmaFlopsBF16")
    if flops is not None:
        tflops = flops / (launch_us * 1e-6) / 1e12
        out["mfma_bf16_tflops"] = tflops
        out["mfma_bf16_frac_of_peak"] = tflops / MFMA_BF16_PEAK_TFLOPS
        if "flops" in rec:
            out["algorithmic_flops"] = rec["flops"]
            out["mfma_flops_over_algorithmic"] = flops / rec["flops"]
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"counters_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))
    return out


def committed_counters(workload: str, kernel: str, profiles_dir: str = None):
    """MFMA and VALU utilisation of the main kernel from committed rocprofv3
    counter runs, if they were taken on the current sources; else None."""
    path = os.path.join(profiles_dir or os.path.join(ROOT, "profiles"), f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_digest() or rec.get("kernel") != kernel:
        return None
    pl = rec["per_launch"]
    keep = {"mfma_util_pct": pl.get("MfmaUtil"), "mfma_bf16_tflops": rec.get("mfma_bf16_tflops"),
            "mfma_bf16_frac_of_peak": rec.get("mfma_bf16_frac_of_peak"), "valu_busy_pct": pl.get("VALUBusy"),
            "occupancy_pct": pl.get("OccupancyPercent"), "source": f"profiles/counters_{workload}.json"}
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in keep.items() if v is not None}


def attention_flops(cfg, lens, tree_parents=None) -> int:
    """Useful flops of a call: a multiply and an add for QK and again for P.V
    over every visible (query head, row, token) triple, 4 * d each. A chain of
    drafted tokens sees the context and the drafts up to itself; a tree node
    sees the context and its own ancestors (parent index -1: the context)."""
    total = 0
    for b, L in enumerate(lens.astype(np.int64)):
        for i in range(cfg.q_len):
            if tree_parents is None:
                seen = i + 1
            else:
                seen, p = 1, int(tree_parents[b][i])
                while p >= 0:
                    seen, p = seen + 1, int(tree_parents[b][p])
            total += 4 * cfg.num_q_heads * cfg.head_dim * int(L - cfg.q_len + seen)
    return total


def read_probe(gib: int = 4, reps: int = 10):
    """Practical HBM read ceilings: the library's read probe over a `gib` GiB
    buffer read once per call, over a few launch shapes, in four orders: a
    seeded random permutation of 8 KiB blocks (the attention kernels' access
    pattern at block size 32: each (block, KV head) slice is one 8 KiB block
    somewhere in the pool), the same of 4 KiB blocks (block size 16), random
    64 KiB runs (eight adjacent 8 KiB blocks) and ascending 8 KiB blocks (a
    contiguous streaming read). The best random-order rate at the slice size
    of a workload is the ceiling its attention kernel is compared with; the
    streaming rate says what the random order of slices costs."""
    import torch
    import paged_kv_cache_218_amd as pa
    nbytes = gib * 2**30
    n_blocks = nbytes // 8192
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    gen = torch.Generator().manual_seed(218)
    runs = torch.randperm(n_blocks // 8, generator=gen).to(torch.int32)
    orders = {"random": (8192, torch.randperm(n_blocks, generator=gen).to(torch.int32).cuda()),
              "random_4k": (4096, torch.randperm(2 * n_blocks, generator=gen).to(torch.int32).cuda()),
              # 64 KiB runs (eight adjacent 8 KiB blocks, e.g. every KV head of one pool block) in random order
              "random_64k_runs": (8192, (runs[:, None] * 8 + torch.arange(8, dtype=torch.int32)).reshape(-1).cuda()),
              "sequential": (8192, torch.arange(n_blocks, dtype=torch.int32, device="cuda"))}
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rows = []
    for name, (block_bytes, order) in orders.items():
        for depth in (1, 2, 4):
            for waves_per_cu in (8, 16, 32):
                wgs = 256 * waves_per_cu // 4
                for _ in range(2):
                    pa.pa_read_probe(buf, order, depth, wgs, sink, block_bytes=block_bytes)
                torch.cuda.synchronize()
                e0.record()
                for _ in range(reps):
                    pa.pa_read_probe(buf, order, depth, wgs, sink, block_bytes=block_bytes)
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / reps * 1e3
                rows.append({"order": name, "block_bytes": block_bytes, "blocks_in_flight": depth,
                             "workgroups": wgs, "us": round(us, 1), "gbs": round(nbytes / us / 1e3, 1)})
                log(f"read probe ({name}, {block_bytes} B blocks): {depth} blocks in flight per wave, "
                    f"{wgs} workgroups: {us:.1f} us, {rows[-1]['gbs']} GB/s")
    best = {name: max((r for r in rows if r["order"] == name), key=lambda r: r["gbs"])["gbs"] for name in orders}
    return {"bytes": nbytes, "order": "seeded random permutation of 8 KiB blocks",
            "best_gbs": best["random"], "best_frac_of_8tbs": round(best["random"] / 8000, 4),
            "random_4k_best_gbs": best["random_4k"], "random_4k_best_frac_of_8tbs": round(best["random_4k"] / 8000, 4),
            "random_64k_runs_best_gbs": best["random_64k_runs"],
            "sequential_best_gbs": best["sequential"], "sequential_best_frac_of_8tbs": round(best["sequential"] / 8000, 4),
            "runs": rows}


def host_timing(call, plan_call, calls: int = 1000):
    """CPU time per call of the library, measured with perf_counter_ns around
    each of `calls` back-to-back asynchronous calls (no synchronisation inside
    the loop; the kernels queue up behind each other on the stream), through
    ctypes with the arguments converted once beforehand. plan_call is a
    host-only entry point taking the same descriptor (it plans, launches
    nothing), timed the same way: the difference is what a launch adds."""
    import statistics
    import torch

    def run(fn):
        ts = []
        for _ in range(calls):
            t0 = time.perf_counter_ns()
            st = fn()
            ts.append(time.perf_counter_ns() - t0)
            if st:
                raise SystemExit(f"host timing: status {st}")
        return ts

    torch.cuda.synchronize()
    launch = run(call)
    torch.cuda.synchronize()
    plan = run(plan_call)
    q = lambda ts, f: sorted(ts)[int(f * (len(ts) - 1))] / 1e3
    return {"calls": calls,
            "us_per_call_median": round(statistics.median(launch) / 1e3, 2),
            "us_per_call_mean": round(statistics.mean(launch) / 1e3, 2),
            "us_per_call_p99": round(q(launch, 0.99), 2),
            "plan_only_us_median": round(statistics.median(plan) / 1e3, 2),
            "how": "perf_counter_ns around each raw ctypes call of the entry point, arguments pre-converted; "
                   "asynchronous calls back to back; plan_only = pa_attention_workspace_size on the same "
                   "descriptor (host planning, no launch)"}


def _sub_cfg(cfg, batch):
    from dataclasses import replace
    return replace(cfg, batch=batch)


def copy_probe(gib: float = 1.0, reps: int = 20):
    """Bandwidth of a plain device-to-device copy (torch's copy kernel)."""
    import torch
    n = int(gib * 2**30)
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"bytes_read": n, "bytes_written": n, "ms": round(ms, 4),
            "gbs_read_plus_write": round(2 * n / ms / 1e6, 1)}


def spec_bytes(cfg, n_accepted) -> int:
    """Algorithmic bytes of one accept / resample call: per sequence the
    acceptance reads (p, q, draft token, uniform) of the drafts tested, the
    row(s) the draw reads once (p and q at a rejection, p alone for the extra
    token), the draw's uniform and the outputs."""
    V, K = cfg.vocab, cfg.k
    total = 0
    for n in n_accepted:
        n = int(n)
        tested = min(n + 1, K)
        rows = 2 if n < K else 1
        total += tested * 16 + rows * V * 4 + 4 + 4 + (K + 1) * 4
    return total


def bench_spec(args):
    import torch
    import workloads
    import paged_kv_cache_218_amd as pa
    cfg = workloads.SPEC_CONFIGS[args.workload]
    log(f"generating {cfg.name}")
    w = workloads.generate_spec(cfg)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    p, q, draft, ua, ud = d(w.p), d(w.q), d(w.draft), d(w.u_accept), d(w.u_draw.view(np.int32))
    n = torch.empty(cfg.batch, dtype=torch.int32, device="cuda")
    toks = torch.empty(cfg.batch, cfg.k + 1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(pa.pa_spec_accept_workspace_size(cfg.batch, cfg.vocab), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    step = lambda: pa.pa_spec_accept(p, q, draft, ua, ud, n, toks, ws, stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps
    n_acc = n.cpu().numpy()
    nbytes = spec_bytes(cfg, n_acc)
    gbs = nbytes / (ms * 1e-3) / 1e9
    result = {
        "metric": "accept/resample GB/s & % of HBM peak; sequences/s",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded N(0, 36) logits; draft = target + N(0, 0.25) noise)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "drafts": cfg.k, "vocab": cfg.vocab,
                   "mean_accepted": float(n_acc.mean()), "all_accepted": int((n_acc == cfg.k).sum())},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "sequences_per_s": round(cfg.batch / (ms * 1e-3), 1),
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "hbm", "kernel": "spec_accept_kernel<true>", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "launch_us": round(ms * 1e3, 2), "traffic": committed_traffic(cfg.name, "spec_accept_kernel<true>"),
                     "note": "one kernel per step: launch time from HIP events over the timed region"},
        "wall_s_timed_region": round(t_wall, 4),
    }
    if args.copy_probe:
        result["copy_probe"] = copy_probe()
    if not args.no_cpu_baseline:
        from oracle import spec as ospec
        t0 = time.perf_counter()
        done = 0
        while done < cfg.batch and time.perf_counter() - t0 < 15.0:
            ospec.accept_sequence(w.p[done], w.q[done], w.draft[done], w.u_accept[done], int(w.u_draw[done]))
            done += 1
        t_used = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(spec_bytes(cfg, n_acc[:done]) / t_used / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "sample": f"{done} of {cfg.batch} sequences, {t_used:.1f} s (Python integer draw)",
            "seconds": round(t_used, 3)}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_70b_decode")
    ap.add_argument("--path", default="auto", choices=["auto", "mfma", "valu"])
    ap.add_argument("--partition-tokens", type=int, default=-1,
                    help="-1: the workload's own setting; 0: library's choice")
    ap.add_argument("--waves", type=int, default=0, help="wavefronts per workgroup (0: library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--host-calls", type=int, default=1000,
                    help="after the timed region, time this many calls on the CPU side (0: skip)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--read-probe", action="store_true",
                    help="measure the device's read ceilings (4 and 8 KiB blocks in random order, streaming) and exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--bench-json", help="with --pmc-summary: a bench line of the workload (data-dependent bytes); "
                                         "with --counter-summary: the launch time and kernel name")
    ap.add_argument("--counter-summary", nargs="+", metavar="RUN_DIR",
                    help="write profiles/counters_<workload>.json from rocprofv3 --pmc runs (utilisation "
                         "counters) and a --bench-json line, and exit")
    ap.add_argument("--trace-summary", metavar="RUN_DIR",
                    help="steady-state durations of --kernel from a rocprofv3 --kernel-trace run and exit")
    ap.add_argument("--kernel", help="with --trace-summary: kernel name (substring)")
    ap.add_argument("--skip", type=int, default=0, help="with --trace-summary: leading dispatches to drop")
    ap.add_argument("--take", type=int, default=0, help="with --trace-summary: dispatches to keep (0: all)")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary, args.kernel, args.skip, args.take)
        return
    if args.pmc_summary:
        pmc_summary(args.workload, *args.pmc_summary, bench_json=args.bench_json)
        return
    if args.counter_summary:
        counter_summary(args.workload, args.counter_summary, args.bench_json)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the sharding design is written up, not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import paged_kv_cache_218_amd as pa
    from paged_kv_cache_218_amd.cache import PagedKVCache, lens_to_device, queries_to_device

    if args.read_probe:
        print(json.dumps({"read_probe": read_probe()}), flush=True)
        return
    if args.workload in workloads.SPEC_CONFIGS:
        bench_spec(args)
        return
    cfg = workloads.CONFIGS[args.workload]
    log(f"generating {cfg.name}")
    t0 = time.time()
    w = workloads.generate(cfg, threads=16)
    log(f"  {time.time() - t0:.1f} s; building the paged cache through pa_write_kv")
    cache = PagedKVCache.from_workload(w)
    q = queries_to_device(w)
    lens_d = lens_to_device(w)
    tables_d = cache.tables_device()
    path = {"auto": pa.PA_PATH_AUTO, "mfma": pa.PA_PATH_MFMA, "valu": pa.PA_PATH_VALU}[args.path]
    pt = cfg.partition_tokens if args.partition_tokens < 0 else args.partition_tokens
    max_ctx = int(w.lens.max())
    desc = cache.desc(cfg.num_q_heads, max_ctx, path, pt, args.waves)
    plan = pa.pa_attention_plan(desc, cfg.q_len)
    out = torch.empty_like(q)
    # zero-filled: the balanced schedule's arrival counters start at zero
    ws = torch.zeros(max(plan.workspace_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    masks = None
    if w.tree_parents is not None:   # tree verification: ancestor masks from the library's helper
        from paged_kv_cache_218_amd.cache import tree_masks_to_device
        masks = tree_masks_to_device(w.tree_parents)
    torch.cuda.synchronize()

    def step():
        if masks is None:
            pa.pa_attention(desc, q, cache.k_pool, cache.v_pool, tables_d, lens_d, cfg.q_len, cfg.scale,
                            out, ws if plan.workspace_bytes else None, stream)
        else:
            pa.pa_attention_tree(desc, q, cache.k_pool, cache.v_pool, tables_d, lens_d, cfg.q_len, masks,
                                 cfg.q_len, cfg.scale, out, ws if plan.workspace_bytes else None, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # HIP events on the stream the kernels are launched on
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps
    # per-launch time of the main kernel alone (one kernel per step unless a
    # separate merge kernel runs after it)
    main_ms = ms if plan.merge_grid == 0 else None

    nbytes = algorithmic_bytes(cfg, w.lens)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tokens = cfg.batch * cfg.q_len / (ms * 1e-3)
    path_name = {1: "valu", 2: "mfma"}[plan.path]
    kernel = kernel_name(cfg, plan, desc)
    traffic = committed_traffic(cfg.name, kernel)
    roof_ms = main_ms if main_ms is not None else ms
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1), bf16-rounded; no public dataset)",
        "config": {
            "workload": cfg.name, "batch": cfg.batch, "q_len": cfg.q_len,
            "context_tokens": {"min": int(w.lens.min()), "max": max_ctx, "mean": float(w.lens.mean())},
            "q_heads": cfg.num_q_heads, "kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim,
            "block_size": cfg.block_size, "num_blocks": w.num_blocks, "prefix_len": cfg.prefix_len,
            "kv_storage": "fp8_e4m3+scales" if cfg.kv_dtype == "fp8" else cfg.dtype,
            "drafted_tokens": f"tree ({cfg.tree})" if cfg.tree else ("chain" if cfg.q_len > 1 else "none"),
            "path": path_name, "partition_tokens": plan.partition_tokens,
            "schedule": {0: "partitions", 1: "balanced", 2: "partitions_wave"}[plan.schedule], "kv_shared": int(desc.kv_shared),
            "partitions": plan.num_partitions, "waves_per_group": plan.waves_per_group,
            "grid": plan.grid, "merge_grid": plan.merge_grid, "tiles_per_wave": plan.tiles_per_wave,
            "partitions_per_wave": plan.partitions_per_wave,
        },
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(tokens, 1),
        "tokens_per_s_80_layers": round(tokens / 80, 2),
        "algorithmic_bytes": nbytes,
        "flops": attention_flops(cfg, w.lens, w.tree_parents),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(nbytes / (roof_ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(nbytes / (roof_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "launch_us": round(roof_ms * 1e3, 2),
            "traffic": traffic,
            "note": ("one kernel per step: launch time from HIP events over the timed region"
                     if main_ms is not None else
                     "partition kernel + merge kernel per step: time is the pair's"),
        },
        "wall_s_timed_region": round(t_wall, 4),
    }
    counters = committed_counters(cfg.name, kernel)
    if counters is not None:
        result["roofline"]["counters"] = counters
    if args.host_calls > 0:
        import ctypes as C
        lib = pa._lib.lib
        ws_arg = ws.data_ptr() if plan.workspace_bytes else None
        ws_n = plan.workspace_bytes
        ptrs = [t.data_ptr() for t in (q, cache.k_pool, cache.v_pool, tables_d, lens_d)]
        desc_ref, sid, out_p = C.byref(desc), stream.cuda_stream, out.data_ptr()
        if masks is None:
            call = lambda: lib.pa_attention(desc_ref, *ptrs, cfg.q_len, cfg.scale, out_p, ws_arg, ws_n, sid)
        else:
            mp = masks.data_ptr()
            call = lambda: lib.pa_attention_tree(desc_ref, *ptrs, cfg.q_len, mp, cfg.q_len, cfg.scale, out_p,
                                                 ws_arg, ws_n, sid)
        ql = cfg.q_len
        plan_call = lambda: 0 if lib.pa_attention_workspace_size(desc_ref, ql) == plan.workspace_bytes else 1
        log(f"host timing: {args.host_calls} calls")
        result["host_timing"] = host_timing(call, plan_call, args.host_calls)
    if args.copy_probe:
        result["copy_probe"] = copy_probe()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
