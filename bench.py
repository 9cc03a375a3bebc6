#!/usr/bin/env python3
"""Throughput of the unmerged multi-LoRA projection on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload decode|prefill|many|tiny|stack13b|prefetch|adapters] [--fuse-slots]

A step is one pass of the whole projection (token grouping, shrink, base GEMM + expand) over one
batch of the workload, with every input already resident in HBM.  The default workload is the
Llama-7B-shaped q_proj decode batch: H = 4096, bf16, 32 adapters of ranks {8, 16, 32, 64},
64 tokens (one per request), pages scattered through a pool that is 60 % KV pages.

HBM honesty: the 256 MiB Infinity Cache would hold one replica of the decode working set, so the
timed loop rotates through enough independent replicas (pool, page table, W, x, y) to touch
>= 1 GiB between reuses.

Prints one JSON line: the throughput, the dominant kernel's roofline fraction (its algorithmic
bytes or flops over its average device time, from HIP events recorded on its launch stream) with
the whole call's fraction beside it (roofline.call), and the fp64 CPU oracle timed on this host as a
baseline.  The default run also times the prefill batch (MFMA-bound), the 2000-adapter batch
(HBM-bound, its q/k/v/o in one call) and the 40-layer 13B-shaped stack (one call per layer) and adds
their lines' figures under "more_workloads".  The
roofline's "traffic" (HBM bytes per launch from committed rocprofv3 counters) is given when the
counters were taken on the current kernel source, the same workload and the same slots per launch;
null otherwise.  With --fuse-slots a layer's q, k, v
and o (each with its own x) are projected by one lora_project_slots_x call; the per-launch figures then
cover every slot of the launch.  (The workloads give o its own input; in a model's forward pass o
follows attention and would be a call of its own.)  --workload stack13b runs the whole 40-layer stack
(160 slots, a 115 GiB pool, one replica: a step moves 42 GiB, far beyond the Infinity Cache).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "multi-LoRA proj tokens/s + %HBM/%MFMA roofline, H=4096, 32 adapters, 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w, T_ids, slots):
    """Bytes and flops the method itself must move/compute per step, and each kernel's share.

    Per projection call: W once (H^2 e), x in and y out (2 T H e), each A and B page of every
    distinct adapter the batch uses once (2 r H e), the ids (4 T).  Flops: 2 T H^2 + 4 H r per
    token with an adapter.  Per kernel (decode path): the first launch reads W, x, the ids and the
    A pages (base partials and the shrink); the second reads the B pages and writes y.  Prefill
    path: the shrink reads x and the A pages; the tiled GEMM reads x, W, the B pages, writes y.
    Partial sums the kernels exchange through the workspace are not algorithmic bytes.
    """
    H, e = w.hidden, w.elem
    ids = T_ids
    distinct = sorted({int(a) for a in ids if a >= 0 and w.ranks[a] > 0})
    r_sum_distinct = sum(int(w.ranks[a]) for a in distinct)
    r_sum_tokens = sum(int(w.ranks[a]) for a in ids if a >= 0)
    T = len(ids)
    pages = r_sum_distinct * H * e           # all A pages (or all B pages) of the batch
    per_call_bytes = H * H * e + 2 * T * H * e + 2 * pages + 4 * T
    per_call_flops = 2 * T * H * H + 4 * H * r_sum_tokens
    return {
        "bytes": per_call_bytes * slots, "flops": per_call_flops * slots,
        "decode_first_bytes": H * H * e + T * H * e + pages + 4 * T,
        "decode_second_bytes": pages + T * H * e,
        "prefill_second_flops": 2 * T * H * H + 2 * H * r_sum_tokens,
        "prefill_first_flops": 2 * H * r_sum_tokens,
        "distinct_adapters": len(distinct), "r_sum_distinct": r_sum_distinct,
    }


def source_hash(paths):
    """First 16 hex digits of the SHA-256 of the files' contents, in the given order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key, src_file, workload):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they were taken on the
    current kernel source and launch planning (project.hip picks the grid and the K splits) and on
    this workload; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    planner = os.path.join(os.path.dirname(src_file), "project.hip")
    if d.get("source_sha256_16") != source_hash([src_file, planner]) or d.get("workload") != workload:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, seconds, slots):
    """The fp64 oracle, as it stands, on this host's cores: full batch of one projection, repeated.

    BLAS threads: the cores this process may run on (sched_getaffinity), capped by OMP_NUM_THREADS
    when the host sets it (the GPU hosts give each GPU a share of their cores and set it to that share);
    `cores` is the thread count the BLAS pool then reports."""
    import numpy as np
    import oracle
    from workloads import storage_to_f64
    affinity = len(os.sched_getaffinity(0))
    want = min(affinity, int(os.environ.get("OMP_NUM_THREADS", affinity) or affinity))
    limiter = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=want, user_api="blas")
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [want])
    except Exception:
        cores = want
    slot = 0
    x64 = storage_to_f64(w.x_for_slot(slot))
    W64 = storage_to_f64(w.W(slot)).T
    A, B = {}, {}
    for a in sorted({int(a) for a in w.ids if a >= 0 and w.ranks[a] > 0}):
        at, b = w.adapter(a)
        A[a], B[a] = storage_to_f64(at[slot]).T, storage_to_f64(b[slot])
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.project(x64, W64, A, B, w.ids, w.scales)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    tokens_per_s = n * w.T / el / slots      # a step pushes T tokens through `slots` projections
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": int(cores), "affinity_cores": affinity,
            "kind": "oracle",
            "sample": f"full {w.T}-token batch of one projection (slot 0), {n} repeats in {el:.1f} s, "
                      f"scaled to {slots} projection(s) per step"}


def prefetch_bench(args, rg, torch):
    """Adapter prefetch ("S-LoRA, in depth", section "Scheduling: prefetch, clustering and early
    abort": the next batch's adapters are copied from pinned host memory on a separate stream while
    the current batch computes).  Eight 32 MiB adapters (rank 16 over q/k/v/o of 32 layers at
    H = 4096, the pages' example) are loaded into a 128-slot pool on a copy stream: alone, and while
    the 64-token decode projection steps run on the compute stream.  Loads are issued from a second
    host thread (the library releases the interpreter lock inside each call), so a load that waits
    for a free load buffer does not hold up the decode issue loop."""
    import threading
    from workloads import build
    dev = torch.device("cuda:0")
    H, SLOTS, RANK, NAD = 4096, 128, 16, 8
    ad_bytes = 2 * RANK * SLOTS * H * 2
    cp = rg.Pool(NAD * 2 * RANK * SLOTS + 64, H, rg.LORA_BF16, n_slots=SLOTS, max_adapters=NAD, max_rank=RANK)
    g = torch.Generator().manual_seed(20251)
    host = []
    for a in range(NAD):
        pair = []
        for _ in range(2):
            t = torch.empty((SLOTS, RANK, H), dtype=torch.bfloat16, pin_memory=True)
            t.copy_((torch.randn((SLOTS, RANK, H), generator=g) * 0.02).to(torch.bfloat16))
            pair.append(t)
        host.append(pair)
    copy = torch.cuda.Stream()   # default priority, like every stream here
    comp = torch.cuda.current_stream()

    def load_all():
        for a in range(NAD):
            rg.lora_pool_load_adapter(cp.handle, a, RANK, host[a][0], host[a][1], stream=copy)

    def evict_all():
        for a in range(NAD):
            rg.lora_pool_release_adapter(cp.handle, a)
            rg.lora_pool_evict_adapter(cp.handle, a, stream=copy)
        torch.cuda.synchronize()

    # the compute side: the default decode workload, rotated over a few replicas
    w = build("decode", device="cuda")
    d_ids, d_ranks, d_scale = (torch.as_tensor(v, device=dev) for v in (w.ids, w.ranks, w.scales))
    reps = []
    for _ in range(8):
        pool = rg.Pool(w.num_pages, w.hidden, rg.LORA_BF16, n_slots=1, max_adapters=w.max_adapters,
                       free_order=w.free_order)
        assert all(st == 0 for st in pool.run_ops(w.ops, w.ranks, w.adapter))
        reps.append((pool, w.W(0).clone(), w.x().clone(), torch.empty_like(w.x())))
    ws = torch.empty(rg.lora_project_workspace_size(reps[0][0].handle, w.T), dtype=torch.uint8, device=dev)

    def decode(n):
        for i in range(n):
            pool, W, x, y = reps[i % len(reps)]
            rg._lib.lora_project(pool.handle, x.data_ptr(), W.data_ptr(), pool.table[0].data_ptr(), d_ids.data_ptr(),
                                 d_ranks.data_ptr(), d_scale.data_ptr(), w.T, y.data_ptr(), ws.data_ptr(), ws.numel(),
                                 comp.cuda_stream)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    N = 500
    # warm-up of both sides
    load_all(); torch.cuda.synchronize(); evict_all()
    decode(50); torch.cuda.synchronize()
    # 1. loads alone
    a0, a1 = ev(), ev()
    a0.record(copy); load_all(); a1.record(copy); torch.cuda.synchronize()
    t_load = a0.elapsed_time(a1) / 1e3
    evict_all()
    # 2. decode alone
    d0, d1 = ev(), ev()
    d0.record(comp); decode(N); d1.record(comp); torch.cuda.synchronize()
    t_dec = d0.elapsed_time(d1) / 1e3
    # 3. both: the loads start with the decode steps
    c0, c1, e0, e1 = ev(), ev(), ev(), ev()
    e0.record(comp); c0.record(copy)
    th = threading.Thread(target=lambda: (load_all(), c1.record(copy)))
    th.start()
    decode(N)
    e1.record(comp)
    th.join()
    torch.cuda.synchronize()
    t_dec_ov = e0.elapsed_time(e1) / 1e3
    t_load_ov = c0.elapsed_time(c1) / 1e3
    t_both = max(t_dec_ov, e0.elapsed_time(c1) / 1e3)
    hidden = (t_dec + t_load - t_both) / t_load
    out = {
        "metric": "adapter prefetch: host-to-pool copy rate, alone and beside the decode projection",
        "value": NAD * ad_bytes / t_load_ov / 1e9, "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
        "data": "synthetic (seeded; pinned host memory)",
        "config": {"workload": "8 adapters of 32 MiB (rank 16, q/k/v/o of 32 layers, H=4096 bf16) into a 128-slot "
                               "pool on a copy stream, beside 64-token decode steps (H=4096, 32 adapters)",
                   "adapter_bytes": ad_bytes, "adapters": NAD, "decode_steps": N},
        "load_alone_GBps": NAD * ad_bytes / t_load / 1e9, "load_alone_ms_per_adapter": t_load / NAD * 1e3,
        "load_beside_decode_GBps": NAD * ad_bytes / t_load_ov / 1e9,
        "load_beside_decode_ms_per_adapter": t_load_ov / NAD * 1e3,
        "decode_alone_us_per_step": t_dec / N * 1e6, "decode_beside_loads_us_per_step": t_dec_ov / N * 1e6,
        "loads_hidden_fraction": hidden,
    }
    cp.close()
    for r in reps:
        r[0].close()
    print(json.dumps(out), flush=True)


def adapter_sweep_bench(args, rg, torch):
    """The load test of "S-LoRA, in depth" (section "What to do next"): the projection with 1, 10,
    100 and 1,000 adapters in play at the configs' rank mix (uniform over {8, 16, 32, 64}), for a
    64-token and a 256-token decode batch at H = 4096 (ids uniform over the adapters): mean time per
    call, tokens/s and the 99th percentile of single calls (HIP events around each call, minus the
    events' own cost measured by an event-free loop)."""
    import numpy as np
    from workloads import custom
    dev = torch.device("cuda:0")
    rows = []
    for T in (64, 256):
        for K in (1, 10, 100, 1000):
            rng = np.random.default_rng(1000 * T + K)
            ranks = rng.choice([8, 16, 32, 64], K).astype(np.int32)
            ids = rng.integers(0, K, T).astype(np.int32)
            w = custom(4096, ranks, ids, device="cuda", seed=77 + K + T)
            d_ids, d_ranks, d_scale = (torch.as_tensor(v, device=dev) for v in (w.ids, w.ranks, w.scales))
            reps = []
            for _ in range(4):
                pool = rg.Pool(w.num_pages, w.hidden, rg.LORA_BF16, n_slots=1, max_adapters=K, free_order=w.free_order)
                assert all(st == 0 for st in pool.run_ops(w.ops, w.ranks, w.adapter))
                reps.append((pool, w.W(0).clone(), w.x().clone(), torch.empty_like(w.x())))
            w.drop_cache("AB")
            ws = torch.empty(rg.lora_project_workspace_size(reps[0][0].handle, T), dtype=torch.uint8, device=dev)
            sh = torch.cuda.current_stream().cuda_stream

            def call(i):
                pool, W, x, y = reps[i % len(reps)]
                rg._lib.lora_project(pool.handle, x.data_ptr(), W.data_ptr(), pool.table[0].data_ptr(),
                                     d_ids.data_ptr(), d_ranks.data_ptr(), d_scale.data_ptr(), T, y.data_ptr(),
                                     ws.data_ptr(), ws.numel(), sh)
            N = 600
            for i in range(50):
                call(i)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for i in range(N):
                call(i)
            b.record()
            torch.cuda.synchronize()
            mean_us = a.elapsed_time(b) / N * 1e3
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(N + 1)]
            evs[0].record()
            for i in range(N):
                call(i)
                evs[i + 1].record()
            torch.cuda.synchronize()
            per = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(N)])
            gap = max(0.0, per.mean() - mean_us)     # each interval also holds its closing event
            distinct = len({int(v) for v in ids})
            rows.append({"tokens": T, "adapters": K, "distinct_in_batch": distinct, "us_per_call": mean_us,
                         "tokens_per_s": T / (mean_us / 1e6), "p99_us": float(np.percentile(per, 99)) - gap,
                         "p50_us": float(np.percentile(per, 50)) - gap})
            log(f"T={T} adapters={K} distinct={distinct}: {mean_us:.2f} us/call, p99 {rows[-1]['p99_us']:.2f} us")
            for r in reps:
                r[0].close()
    out = {"metric": "multi-LoRA projection with 1, 10, 100, 1000 adapters: tokens/s and p99 per call",
           "value": rows[-1]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True,
           "data": "synthetic (seeded; inputs resident in HBM)",
           "config": {"workload": "H=4096 bf16 decode batches of 64 and 256 tokens, ids uniform over 1/10/100/1000 "
                                  "adapters of ranks U{8,16,32,64}; value = 256 tokens, 1000 adapters"},
           "sweep": rows}
    print(json.dumps(out), flush=True)


DESCRIPTIONS = {
    "decode": "Llama-7B-shaped q_proj decode: H=4096 bf16, 32 adapters ranks U{8,16,32,64}, 64 tokens "
              "(1 per request), pool 60% KV pages",
    "prefill": "prefill grouped GEMM: H=4096 bf16, 8 requests x 512 tokens, ranks {8,8,16,16,32,32,64,64}",
    "many": "2000 adapters, q/k/v/o of one layer, H=4096 bf16, 256 decode tokens Zipf(1.0), 10% identity",
    "tiny": "tiny: H=256 fp32, 4 adapters, 16 tokens",
    "stack13b": "Llama-13B-shaped stack: H=5120 bf16, 40 layers x q/k/v/o (160 slots), 1000 adapters, "
                "4x2048 prefill + 256 decode rows Zipf(1.2), churned pool of 115 GiB",
}


def load_pool(rg, torch, w):
    """A device pool holding the workload's adapters and KV pages (ops run in chunks; adapters drawn
    without keeping them, so the largest pool does not hold its weights twice)."""
    pool = rg.Pool(w.num_pages, w.hidden, rg.LORA_F32 if w.dtype == "f32" else rg.LORA_BF16, n_slots=w.n_slots,
                   max_adapters=w.max_adapters, free_order=w.free_order)
    for i in range(0, len(w.ops), 20000):
        st = pool.run_ops(w.ops[i:i + 20000], w.ranks, w.adapter_uncached)
        assert all(s == 0 for s in st), rg.lora_last_error()
        torch.cuda.synchronize()
        if len(w.ops) > 20000:
            log(f"  pool ops {min(i + 20000, len(w.ops))}/{len(w.ops)}")
    return pool


def measure(rg, torch, name, steps, warmup, fuse_slots, profile_calls, replicas=0):
    """Time `steps` steps of one workload (after `warmup`), then the per-kernel device times from HIP
    events on the launch stream.  Returns the JSON fields of the workload's line."""
    from workloads import build
    dev = torch.device("cuda:0")
    w = build(name, device="cuda")
    slots = list(range(w.n_slots))
    info = algorithmic(w, w.ids, len(slots))
    log(f"workload {w.name}: H={w.hidden} T={w.T} slots={len(slots)} adapters={w.max_adapters} "
        f"distinct={info['distinct_adapters']} step bytes={info['bytes'] / 2**20:.1f} MiB "
        f"flops={info['flops'] / 1e9:.2f} G")
    # cold HBM: rotate replicas so that >= 1 GiB is touched between reuses (one replica when a step
    # alone moves more than that)
    R = replicas or max(1, math.ceil(2 ** 30 / max(info["bytes"], 1)))
    R = 1 if info["bytes"] >= 2 ** 30 else max(2, min(R, 64))
    d_ids = torch.as_tensor(w.ids, device=dev)
    d_ranks = torch.as_tensor(w.ranks, device=dev)
    d_scale = torch.as_tensor(w.scales, device=dev)
    reps = []
    for i in range(R):
        pool = load_pool(rg, torch, w)
        Ws = [w.W(s) if R == 1 else w.W(s).clone() for s in slots]
        xs = [w.x(i2) if R == 1 else w.x(i2).clone() for i2 in range(w.n_x)]
        ys = [torch.empty_like(xs[0]) for _ in slots]
        reps.append((pool, Ws, xs, ys))
    # the calls of one step: one per slot, or (fuse_slots) one per run of up to LORA_MAX_CALL_SLOTS
    # consecutive slots (a layer's q, k, v and o: lora_project_slots_x, each slot with its own x)
    groups = []
    for s in slots:
        if fuse_slots and groups and len(groups[-1]) < rg.LORA_MAX_CALL_SLOTS:
            groups[-1].append(s)
        else:
            groups.append([s])
    # one workspace shared by every replica, as a caller issuing the calls on one stream would
    ws = torch.empty(max(rg.lora_project_slots_workspace_size(p.handle, len(g), w.T) for p, *_ in reps
                         for g in groups), dtype=torch.uint8, device=dev)
    wsb = ws.numel()
    log(f"replicas: {R}; calls per step: {len(groups)}")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    fused = []
    if fuse_slots:   # argument arrays built once per replica, outside the timed loop
        for pool, Ws, xs, ys in reps:
            calls = []
            for g in groups:
                n = len(g)
                calls.append((n, (ctypes.c_int32 * n)(*g), (ctypes.c_void_p * n)(*[xs[w.slot_x[s]].data_ptr() for s in g]),
                              (ctypes.c_void_p * n)(*[Ws[s].data_ptr() for s in g]),
                              (ctypes.c_void_p * n)(*[ys[s].data_ptr() for s in g])))
            fused.append(calls)

    def step(i):
        pool, Ws, xs, ys = reps[i % R]
        if fuse_slots:
            for n, sl, xp, wp, yp in fused[i % R]:
                rg._lib.lora_project_slots_x(pool.handle, n, sl, xp, wp, d_ids.data_ptr(), d_ranks.data_ptr(),
                                             d_scale.data_ptr(), w.T, yp, ws.data_ptr(), wsb, sh)
            return
        for s in slots:
            rg._lib.lora_project(pool.handle, xs[w.slot_x[s]].data_ptr(), Ws[s].data_ptr(), pool.table[s].data_ptr(),
                                 d_ids.data_ptr(), d_ranks.data_ptr(), d_scale.data_ptr(), w.T, ys[s].data_ptr(),
                                 ws.data_ptr(), wsb, sh)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(reps[0][0].handle, check=False) == 0, rg.lora_last_error()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / steps
    tokens_per_s = w.T / (ms_per_step / 1e3)
    log(f"timed {steps} steps: {ms_per_step * 1e3:.2f} us/step, {tokens_per_s / 1e6:.3f} M tokens/s, "
        f"step algorithmic {info['bytes'] / (ms_per_step / 1e3) / 1e9:.0f} GB/s, "
        f"{info['flops'] / (ms_per_step / 1e3) / 1e12:.0f} TFLOP/s")

    # per-kernel device time from HIP events on the launch stream (separate loop: events add gaps)
    calls_per_rep = max(1, profile_calls // (R * len(groups)))
    for pool, *_ in reps:
        rg.lora_profile_start(pool.handle, calls_per_rep * len(groups))
    for i in range(calls_per_rep * R):
        step(i)
    torch.cuda.synchronize()
    prof = {"calls": 0, "ms_group": 0.0, "ms_first": 0.0, "ms_second": 0.0}
    for pool, *_ in reps:
        pr = rg.lora_profile_stop(pool.handle)
        for k in prof:
            prof[k] += pr[k]
    n = max(prof["calls"], 1)
    avg = {k.replace("ms_", "") + "_us": prof[k] / n * 1e3 for k in ("ms_group", "ms_first", "ms_second")}
    # Each interval between two event records on the stream also holds the closing record's own
    # cost.  The timed loop above ran the same launches with no events in between, so the
    # per-interval cost is (sum of the kernel intervals - event-free time per call) / intervals.
    decode_like = w.dtype == "bf16" and w.T <= 256
    keys = ["first_us", "second_us"] if decode_like else ["group_us", "first_us", "second_us"]
    call_us = ms_per_step * 1e3 / len(groups)
    per_call = len(slots) / len(groups)   # slots one launch projects, on average
    event_gap_us = max(0.0, (sum(avg[k] for k in keys) - call_us) / len(keys))
    log(f"kernel event intervals (us): {avg} over {prof['calls']} calls; per-interval event cost {event_gap_us:.2f} us")

    src = os.path.join(ROOT, "rank_gemm_unified_amd", "csrc")
    first_us = avg["first_us"] - event_gap_us
    second_us = avg["second_us"] - event_gap_us
    timing = ("HIP events around each launch on its stream, minus the per-interval event cost "
              f"({event_gap_us:.2f} us, from the event-free timed loop)")
    if decode_like:
        stream_kernel = w.T <= 64 and w.hidden <= 8192
        achieved = info["decode_first_bytes"] * per_call / (first_us / 1e6) / 1e9
        call_gbs = info["bytes"] / (ms_per_step / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "kernel": ("k_decode_stream (W stream + MFMA partials, gathered-A shrink)" if stream_kernel else
                           "k_decode_wide (x and W through LDS + MFMA partials, shrink work units)")
                          + (f" ({per_call:g} slots per launch)" if per_call != 1 else ""),
                "algorithmic_bytes_per_launch": info["decode_first_bytes"] * per_call, "avg_launch_us": first_us,
                "traffic": traffic_from_profiles(
                    ("decode_stream" if stream_kernel else "decode_wide") + ("" if per_call == 1 else f"_slots{per_call:g}"),
                    os.path.join(src, "k_decode.hip" if stream_kernel else "k_decode_wide.hip"), w.name),
                "timing": timing,
                "second_kernel": {"kernel": "k_decode_finish (partials + gathered-B expand + rounding)",
                                  "avg_launch_us": second_us,
                                  "achieved_GBps": info["decode_second_bytes"] * per_call / (second_us / 1e6) / 1e9},
                "call": {"what": "the whole step (every launch of every call), event-free loop",
                         "algorithmic_bytes": info["bytes"], "us": ms_per_step * 1e3, "achieved": call_gbs,
                         "frac": call_gbs / HBM_PEAK_GBS}}
    else:
        achieved = info["prefill_second_flops"] * per_call / (second_us / 1e6) / 1e12
        call_tf = info["flops"] / (ms_per_step / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                "kernel": "k_prefill_main (tiled MFMA GEMM + fused expand)" + (f" ({per_call:g} slots per launch)" if per_call != 1 else ""),
                "algorithmic_flops_per_launch": info["prefill_second_flops"] * per_call, "avg_launch_us": second_us,
                "traffic": traffic_from_profiles("prefill_main" + ("" if per_call == 1 else f"_slots{per_call:g}"),
                                                 os.path.join(src, "k_prefill.hip"), w.name),
                "timing": timing,
                "call": {"what": "the whole step (every launch of every call), event-free loop",
                         "algorithmic_flops": info["flops"], "us": ms_per_step * 1e3, "achieved": call_tf,
                         "frac": call_tf / MFMA_BF16_PEAK_TFLOPS,
                         "hbm_GBps": info["bytes"] / (ms_per_step / 1e3) / 1e9}}
    out = {
        "value": tokens_per_s, "unit": "tokens/s", "steps": steps, "warmup": warmup, "ms_per_step": ms_per_step,
        "dtype": w.dtype,
        "config": {"workload": DESCRIPTIONS[w.name], "hidden": w.hidden, "tokens": w.T,
                   "projections_per_step": len(slots), "adapters": w.max_adapters,
                   "distinct_adapters_in_batch": info["distinct_adapters"], "replicas_rotated": R,
                   "parallelism": "single GPU", "calls_per_step": len(groups),
                   "slots_per_call": [len(g) for g in groups][:8]},
        "step_algorithmic_bytes": info["bytes"], "step_algorithmic_flops": info["flops"],
        "step_hbm_GBps": info["bytes"] / (ms_per_step / 1e3) / 1e9,
        "step_hbm_frac": info["bytes"] / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS,
        "kernel_event_intervals_us": avg, "event_cost_per_interval_us": event_gap_us,
        "roofline": roof,
    }
    for pool, *_ in reps:
        pool.close()
    return w, out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 2000; 20 for stack13b)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps first (default 200; 3 for stack13b)")
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "many", "tiny", "stack13b", "prefetch", "adapters"],
                    help="stack13b runs the whole 40-layer stack (160 slots); prefetch measures adapter loads from "
                         "pinned host memory beside the decode projection; adapters runs the 1/10/100/1000-adapter "
                         "load test")
    ap.add_argument("--fuse-slots", action="store_true",
                    help="project up to 4 consecutive slots (a layer's q, k, v and o, each with its own x) in one "
                         "lora_project_slots_x call instead of one lora_project call per slot")
    ap.add_argument("--no-more", action="store_true",
                    help="default workload only: skip the extra prefill, many-adapter and stack blocks")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough to touch >= 1 GiB between reuses")
    ap.add_argument("--profile-calls", type=int, default=400)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB 20 times (HBM counter calibration) and exit")
    args = ap.parse_args()

    rank = int(os.environ.get("RANK", "0"))
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        if rank == 0:
            print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); the projection is "
                  "data-parallel over tokens and its multi-GPU sharding is a design note, not a run", flush=True)
        sys.exit(2)

    import torch
    import rank_gemm_unified_amd as rg

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        n = args.calibrate_copy * 2**20
        src_t = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst_t = torch.empty_like(src_t)
        for _ in range(20):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n, "launches": 20}), flush=True)
        return
    if args.workload == "prefetch":
        prefetch_bench(args, rg, torch)
        return
    if args.workload == "adapters":
        adapter_sweep_bench(args, rg, torch)
        return
    big = args.workload == "stack13b"
    steps = args.steps if args.steps is not None else (20 if big else 2000)
    warmup = args.warmup if args.warmup is not None else (3 if big else 200)
    w, res = measure(rg, torch, args.workload, steps, warmup, args.fuse_slots, args.profile_calls, args.replicas)

    cpu = None
    if not args.no_cpu_baseline and rank == 0:
        log("timing the fp64 oracle on the host ...")
        cpu = cpu_baseline(w, args.cpu_seconds, w.n_slots)
    out = {"metric": METRIC, "value": res["value"], "unit": "tokens/s", "n_gpus": 1, "steps": steps,
           "warmup": warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": res["dtype"], "data": "synthetic (seeded; inputs resident in HBM)"}
    out.update({k: v for k, v in res.items() if k not in out})
    out["cpu_baseline"] = cpu
    w.drop_cache()
    del w
    torch.cuda.empty_cache()
    if args.workload == "decode" and not args.no_more:
        # the prefill (MFMA-bound) and many-adapter (HBM-bound) workloads, timed in the same run,
        more = {}
        # (the many-adapter layer as a user projects it: q, k, v and o in one lora_project_slots_x call)
        # and the whole 40-layer 13B-shaped stack, one lora_project_slots_x call per layer
        for name, n_steps, n_warm, fuse in (("prefill", 300, 30, False), ("many", 300, 30, True), ("stack13b", 10, 2, True)):
            w2, r2 = measure(rg, torch, name, n_steps, n_warm, fuse, args.profile_calls)
            more[name] = {k: r2[k] for k in ("value", "unit", "ms_per_step", "steps", "config", "step_hbm_frac",
                                             "roofline")}
            w2.drop_cache()
            del w2
            torch.cuda.empty_cache()
        out["more_workloads"] = more
    if rank == 0:
        print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
