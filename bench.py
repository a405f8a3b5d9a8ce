#!/usr/bin/env python3
"""Benchmark of the multi-adapter LoRA-linear hot path on one MI355X.

A step is one pass of the whole path over one batch: build the batch index
(plan: group rows by adapter slot, tile segments, upload), then one
LoRA-linear call (base GEMM over all rows, shrink and expand for the rows
with adapters).  Inputs are resident in HBM before the timed region.

Cold-cache measurement: each step uses the next of R copies of the layer
(its own base weight, input/output buffers and adapter pages, identical
values) and the next of NB pre-drawn batches, so consecutive steps do not
hit the 256 MB Infinity Cache with the previous step's data.

Prints one JSON line (rank 0).  Default workload: the Llama-7B stack step
(32 layers x 7 projections q, k, v, o, gate, up, down at their Llama-7B
shapes, bf16, 8 prefill segments + 192 decode rows, 16 cold adapters paged in
from pinned host memory during every step).  --config c2 / c3 / c4 select
the single-projection workloads (decode 4096 x 4096, mixed-rank decode
4096 -> 11008, prefill SGMV).  --sweep-distinct times the C2 shape over 1..64
distinct adapters per batch instead (its own JSON line); --copy-calibration
runs only the copy the HBM byte counters are scaled by.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LoRA-linear tokens/s at Llama-7B shapes; BGMV/SGMV HBM GB/s as % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
# Kernel durations: HIP events around the kernels of every TIMING_PERIOD-th LoRA-linear call
# of the timed region (25 is coprime with the batch and layer-copy cycles and with the 7
# projections of a layer, so the sample covers all of them; a timed call's events cost the
# GPU about 15 us, which stays out of the other calls).
TIMING_PERIOD = 25
# timed steps by default: a timed region of a few tenths of a second (short regions read
# the clocks before they settle)
DEFAULT_STEPS = {"c2": 5000, "c3": 2000, "c4": 500, "c5": 20}
KERNEL_TIMING = (f"HIP events on the launch stream around the kernels of every {TIMING_PERIOD}th LoRA-linear "
                 "call inside the timed region (avg_us = event-measured launch duration)")
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
STACK_STAGE_BYTES = 512 << 20  # the stack step's page-in staging area (a layer of the 16 cold adapters is ~56 MB)

WORKLOADS = {
    "c2": "decode BGMV, Llama-7B attention projection 4096x4096, bf16, 1000 resident rank-16 adapters "
          "(alpha 32) in 8 KB pages scattered over the pool, 64 single-token rows, adapter ids Zipf(1.0)",
    "c3": "decode BGMV with mixed ranks, Llama-7B MLP up projection 4096->11008, bf16, 2000 resident adapters "
          "of ranks {8,16,32,64} (alpha 2r), pool fragmented by dummy KV blocks, 256 rows (26 null), Zipf(0.8)",
    "c4": "prefill SGMV, 4096x4096, bf16, 16 requests of U[64,1024] tokens, one segment each, adapters from "
          "500 of ranks {8,16,32,64}, two null segments",
    "c5": "Llama-7B stack step, 32 layers x 7 projections (q,k,v,o 4096x4096; gate,up 4096->11008; down "
          "11008->4096), bf16, 8 prefill segments of U[128,512] tokens + 192 decode rows, adapters Zipf(1.0) over "
          "2000 (ranks {8,16,32,64}), 16 cold adapters paged in from pinned host memory during every step, KV "
          "blocks of 2 pages per token per layer taken from the same pool",
}


# HBM-side bytes per call of the dominant kernel from rocprofv3 --pmc runs of this bench
# (FETCH_SIZE / 0.500 + WRITE_SIZE / 1.000, the factors a plain 1 GiB copy gives; see profiles/),
# valid only for the kernel sources they were taken on (sha256 of each file).
_GEMM_SRC = {n: d for n, d in (
    ("gemm_kernels.hip", "79d9767fc880377e499d74f987f54cc8d2d94611145d3b152fa26c211ad4f6e2"),
    ("common.h", "2c2dc731e4bbbc397f7de27a14ed55e3f1f1a1fa449485ae11dfc60113113fef"),
    ("bgmv_device.h", "2697fedf22141b5292182872ef017b26bf86dcb1e6c60448eeb4be9738871fcb"),
    ("internal.h", "d4b661c72f9890c6f5989e8cbfa09d1fd56086eabf36962d289907edd69eaa37"))}
TRAFFIC = {
    "c2": {"kernel": "gemm_bgmv_shrink", "bytes": 45.06e6, "sources": _GEMM_SRC},
    "c3": {"kernel": "gemm", "bytes": 119.91e6, "sources": _GEMM_SRC},
    # both launches of the call: 256 x 256 tiles, then the last round as 256 x 128 halves
    "c4": {"kernel": "gemm", "bytes": 701.09e6, "sources": _GEMM_SRC},
    # per projection's GEMM in the step (224: 160 of 192 x 256 tiles; 64 of 256 x 256 tiles plus the
    # last round's 4 tiles as 16 pieces each), mean over the projections
    "c5": {"kernel": "gemm", "bytes": 334.10e6, "sources": _GEMM_SRC},
}


def measured_traffic(cfg, kernel):
    """Counter-measured bytes per call, or None once a source of the kernel changed."""
    import hashlib
    t = TRAFFIC.get(cfg)
    if not t or t["kernel"] != kernel:
        return None
    for name, digest in t["sources"].items():
        path = os.path.join(ROOT, "heterogeneous_adapter_gemm_amd", "csrc", name)
        try:
            with open(path, "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest:
                    return None
        except OSError:
            return None
    return t["bytes"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def rotated_pool(wl, R, max_tokens, max_segments):
    """A pool whose R layers each hold every adapter (same values per layer)."""
    import torch

    from heterogeneous_adapter_gemm_amd import LORA_BF16, DevicePool
    P = wl.page_elems
    per_layer = sum(s.rank * (-(-wl.d_in[0] // P) + -(-wl.d_out[0] // P)) for s in wl.adapters.values())
    kv_pages = sum(op[1] for op in wl.setup_ops if op[0] == "alloc_kv") * R
    num_pages = int(np.ceil(1.25 * (per_layer * R + kv_pages) / 1024)) * 1024
    free = np.random.default_rng([wl.seed, 77]).permutation(num_pages).astype(np.int32)
    pool = DevicePool(LORA_BF16, P, num_pages, free, R, [wl.d_in[0]], [wl.d_out[0]], wl.max_slots, wl.max_rank,
                      max_tokens, max_segments)
    n = 0
    for op in wl.setup_ops:
        if op[0] == "page_in":
            a = wl.adapters[op[1]]
            A, B = wl.adapter_AB(a.adapter_id)
            pool.page_in(a.adapter_id, a.rank, a.alpha, np.tile(A.reshape(-1), R), np.tile(B.reshape(-1), R))
            wl.drop_cache()
            n += 1
            if n % 128 == 0:
                torch.cuda.synchronize()
                pool.drop_host_copies()
        elif op[0] == "alloc_kv":
            pool.alloc_kv(op[1] * R)
    torch.cuda.synchronize()
    pool.drop_host_copies()
    return pool


def delta_bytes(wl, rows_adapter):
    """Algorithmic bytes of the shrink and of the expand for one batch: the
    distinct adapters' A (resp. B) rows once, the adapter rows' x (resp. the
    bf16 read-modify-write of their y) and v (fp32)."""
    e = wl.elem_bytes
    ids = [int(a) for a in rows_adapter if a >= 0]
    distinct = set(ids)
    r_sum_distinct = sum(wl.adapters[a].rank for a in distinct)
    r_sum_rows = sum(wl.adapters[a].rank for a in ids)
    di, do = wl.d_in[0], wl.d_out[0]
    shrink = r_sum_distinct * di * e + len(ids) * di * e + 4 * r_sum_rows
    expand = r_sum_distinct * do * e + 2 * len(ids) * do * e + 4 * r_sum_rows
    return shrink, expand, len(distinct)


def cpu_baseline(wl, budget_s=12.0):
    """The oracle on the host cores: the first batch (all rows), repeated
    until ~budget_s of work."""
    import oracle
    from workloads.device import oracle_adapters
    x, w0, ra, ad = wl.x(), wl.w0(), wl.row_adapter(), oracle_adapters(wl)
    if wl.T > 512:   # prefill: a seeded row sample of the batch
        rows = np.sort(np.random.default_rng(5).choice(wl.T, 64, replace=False))
    else:
        rows = np.arange(wl.T)
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.lora_linear(x, w0, ra, ad, rows=rows)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    return {"value": rows.size * reps / el, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{rows.size} rows of the batch x {reps} repetitions ({el:.1f} s), fp64 loops, OpenMP over rows"}


def run_oracle_timing(budget_s=10.0):
    """The oracle alone on the host cores: all rows of the first batch of the three small
    configurations (fp64 loops), repeated for about budget_s each; one JSON line."""
    import oracle
    from workloads import make_workload
    from workloads.device import oracle_adapters
    out = {"metric": "oracle tokens/s on the host", "cores": oracle.num_threads(), "kind": "oracle", "configs": {}}
    for cfg in ("c1", "c2", "c3"):
        wl = make_workload(cfg, cache=True)
        x, w0, ra, ad = wl.x(), wl.w0(), wl.row_adapter(), oracle_adapters(wl)
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.lora_linear(x, w0, ra, ad)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 1000:
                break
        out["configs"][cfg] = {"rows": int(wl.T), "repetitions": reps, "seconds": round(el, 2),
                               "tokens_per_s": wl.T * reps / el}
        log(cfg, out["configs"][cfg])
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default per workload: c2 5000, c3 2000, c4 500, c5 20)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps first (default: a tenth of --steps)")
    ap.add_argument("--config", default="c5", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate", type=int, default=None, help="layer copies cycled to keep caches cold")
    ap.add_argument("--batches", type=int, default=8, help="pre-drawn batches cycled over the steps")
    ap.add_argument("--fp8-base", action="store_true",
                    help="c2 / c3 / c4: the base weight as E4M3 codes with a scale per output channel "
                         "(lora_linear_fp8); the adapters stay bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single-calls", action="store_true",
                    help="stack: one lora_linear call per projection (no shared shrink launches for q, k, v and "
                         "gate, up)")
    ap.add_argument("--no-prefetch", action="store_true",
                    help="stack step: issue each step's cold page-in when the previous step's work ends, not while "
                         "it runs (no look-ahead)")
    ap.add_argument("--json-out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--sweep-distinct", action="store_true",
                    help="only time the C2 shape with 64-row batches over 1..64 distinct adapters (one JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB 5 times (reference for the HBM byte counters)")
    ap.add_argument("--gemm-vs-library", action="store_true",
                    help="only time the library's base_gemm against hipBLASLt (torch.matmul) on the Llama-7B "
                         "projection shapes of the stack step and the prefill batch (its own JSON line)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure the chip's sustained rates: a 1 GiB device copy (HBM) and the matrix-core "
                         "probe of the library (bf16 16x16x32 chains on register data), one JSON line")
    ap.add_argument("--oracle-timing", action="store_true",
                    help="only time the oracle on the host (no GPU): every row of the first batch of c1, c2 and c3, "
                         "about 10 s each, with the threads OpenMP gives it (OMP_NUM_THREADS=1: one core)")
    ap.add_argument("--engine-trace", action="store_true",
                    help="only run Zipf(1.0) arrivals over the 2000-adapter Llama-7B universe through the engine "
                         "layer, every step's 224 LoRA-linear projections on the GPU (its own JSON line)")
    ap.add_argument("--trace-slots", type=int, default=256, help="engine trace: adapter slots of the pool")
    ap.add_argument("--trace-pool-gb", type=float, default=96.0, help="engine trace: pool size (adapters + KV)")
    ap.add_argument("--trace-host-gb", type=float, default=64.0, help="engine trace: pinned host cache")
    ap.add_argument("--trace-distinct", type=int, default=192, help="engine trace: max distinct adapters per step")
    args = ap.parse_args()
    if args.engine_trace and args.steps is None:
        args.steps, args.warmup = 300, 200 if args.warmup is None else args.warmup
    if args.sweep_distinct and args.steps is None:   # per point, at the C2 shape
        args.steps = DEFAULT_STEPS["c2"]
    if args.steps is None:
        args.steps = DEFAULT_STEPS[args.config]
    if args.warmup is None:
        args.warmup = max(1, args.steps // 10)
    if args.oracle_timing:
        return run_oracle_timing()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import heterogeneous_adapter_gemm_amd as hg
    from workloads import make_workload
    from workloads.device import batch_index

    torch.cuda.set_device(0)
    if args.copy_calibration:
        # the counters' reading for a copy of known size: 1 GiB read and 1 GiB written per launch
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 2 * src.numel(), "launches": 5}), flush=True)
        return
    hg.library()
    cfg = args.config
    if args.sweep_distinct:
        return run_sweep_distinct(args)
    if args.engine_trace:
        return run_engine_trace(args)
    if args.gemm_vs_library:
        return run_gemm_vs_library(args)
    if args.peaks:
        return run_peaks(args)
    if cfg == "c5":
        return run_stack(args)
    R = args.rotate or {"c2": 16, "c3": 4, "c4": 4}[cfg]
    wl = make_workload(cfg, cache=True)
    NB = max(1, args.batches)
    batches = [make_workload(cfg, seed=wl.seed + 1000 + b, cache=False) for b in range(NB)]
    if cfg == "c4":  # prefill: keep this workload's segment lengths, vary the adapters
        for bw in batches:
            bw.requests = [type(r)(r.n_tokens, int(b.adapter_id), r.kind)
                           for r, b in zip(wl.requests, bw.requests)]
    T = wl.T
    log(f"config {cfg}: T={T}, rotate={R}, batches={NB}")
    t_setup = time.perf_counter()
    pool = rotated_pool(wl, R, max_tokens=T, max_segments=32)
    idx = [batch_index(b, pool) for b in batches]
    x1 = hg.device_tensor(wl.x())
    xs = x1.unsqueeze(0).repeat(R, 1, 1).contiguous()
    if args.fp8_base:
        codes, scale = wl.w0_fp8()
        ws = torch.from_numpy(codes).to("cuda").unsqueeze(0).repeat(R, 1, 1).contiguous()
        ss = torch.from_numpy(scale).to("cuda").unsqueeze(0).repeat(R, 1).contiguous()
    else:
        ws = hg.device_tensor(wl.w0()).unsqueeze(0).repeat(R, 1, 1).contiguous()
    ys = torch.empty((R, T, wl.d_out[0]), dtype=torch.bfloat16, device="cuda")
    del x1
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s; pool {pool.num_pages} pages")

    # the step's calls go straight to the C ABI with the stream handle and buffer addresses
    # resolved once (what a native caller passes), so the Python marshalling per call is small
    st = torch.cuda.current_stream().cuda_stream
    xp = [xs[l].data_ptr() for l in range(R)]
    wp = [ws[l].data_ptr() for l in range(R)]
    sp = [ss[l].data_ptr() for l in range(R)] if args.fp8_base else None
    yp = [ys[l].data_ptr() for l in range(R)]
    idx_c = [(ix.get("seg_start"), ix.get("seg_slot"), ix.get("token_slot")) for ix in idx]

    def step(i):
        b, l = i % NB, i % R
        plan = pool.plan(*idx_c[b], stream=st)
        if sp is not None:
            pool.linear_fp8(plan, l, 0, xp[l], wp[l], sp[l], yp[l], stream=st)
        else:
            pool.linear(plan, l, 0, xp[l], wp[l], yp[l], stream=st)
        hg.lora_plan_destroy(plan)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    pool.set_timing(TIMING_PERIOD)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    tim = pool.timing()
    pool.set_timing(False)
    ms_step = el * 1e3 / args.steps
    tok_s = T * args.steps / el

    # per-kernel averages (HIP events on the launch stream, inside the timed region)
    M, N, K = T, wl.d_out[0], wl.d_in[0]
    kern = {}
    for name, (ms, n) in tim.items():
        if n:
            kern[name] = {"avg_us": 1e3 * ms / n, "launches": n}
    sb = eb = 0.0
    dist = 0
    for b in range(NB):
        s, e, d = delta_bytes(batches[b], batches[b].row_adapter())
        sb += s / NB
        eb += e / NB
        dist += d / NB
    # (FP8 base: one byte per weight and a 4-byte scale per output channel)
    gemm_bytes = (N * K + 4 * N if args.fp8_base else N * K * 2) + (M * K + M * N) * 2
    gemm_flops = 2.0 * M * N * K
    alg = {"gemm": gemm_bytes, "bgmv_shrink": sb, "bgmv_expand": eb, "sgmv_shrink": sb, "sgmv_expand": eb,
           "gemm_bgmv_shrink": gemm_bytes + sb}
    for name, k in kern.items():
        if name in alg:
            k["alg_bytes"] = alg[name]
            k["GBps"] = alg[name] / (k["avg_us"] * 1e-6) / 1e9
            k["frac_hbm_peak"] = k["GBps"] / HBM_PEAK_GBS
    for gk in ("gemm", "gemm_bgmv_shrink"):
        if gk in kern:
            kern[gk]["TFLOPs"] = gemm_flops / (kern[gk]["avg_us"] * 1e-6) / 1e12
            kern[gk]["frac_mfma_peak"] = kern[gk]["TFLOPs"] / BF16_PEAK_TFLOPS
    dk = [k for k in ("bgmv_shrink", "bgmv_expand", "sgmv_shrink", "sgmv_expand") if k in kern]
    delta = None
    if dk:
        us = sum(kern[k]["avg_us"] for k in dk)
        byt = sum(kern[k]["alg_bytes"] for k in dk)
        delta = {"kernels": dk, "us": us, "alg_bytes": byt, "GBps": byt / (us * 1e-6) / 1e9,
                 "frac_hbm_peak": byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "distinct_adapters": dist}
    dom = max(kern, key=lambda k: kern[k]["avg_us"])
    traffic = None if args.fp8_base else measured_traffic(cfg, dom)
    if dom == "gemm" and cfg == "c4":
        roof = {"bound": "mfma", "achieved": kern[dom]["TFLOPs"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": kern[dom]["TFLOPs"] / BF16_PEAK_TFLOPS, "traffic": traffic, "kernel": dom}
    else:
        roof = {"bound": "hbm", "achieved": kern[dom]["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": kern[dom]["GBps"] / HBM_PEAK_GBS, "traffic": traffic, "kernel": dom}
    if traffic is not None:
        roof["traffic_unit"] = "bytes per call (HBM side, counters)"
        roof["alg_bytes"] = kern[dom]["alg_bytes"]
    out = {"metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": WORKLOADS[cfg] + (", base weight as E4M3 codes with a scale per output channel"
                                                     if args.fp8_base else ""),
                      "name": cfg + ("_fp8base" if args.fp8_base else ""), "tokens_per_step": T, "layer_copies": R,
                      "batches": NB, "parallelism": "none (1 GPU)"},
           "roofline": roof, "kernels": kern, "delta": delta, "kernel_timing": KERNEL_TIMING}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(wl)
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(line + "\n")



def run_sweep_distinct(args):
    """Step time at the C2 shape (4096 x 4096, bf16, 64 decode rows, rank 16,
    1,000 resident adapters) as the number of distinct adapters in the batch
    goes from 1 to 64, rows spread evenly over them: the pages observe that
    batching many adapters costs little more than one."""
    import torch

    import heterogeneous_adapter_gemm_amd as hg
    from workloads import make_workload
    wl = make_workload("c2", cache=True)
    R, NB, T = 16, 8, wl.T
    pool = rotated_pool(wl, R, max_tokens=T, max_segments=4)
    x1, w1 = hg.device_tensor(wl.x()), hg.device_tensor(wl.w0())
    xs = x1.unsqueeze(0).repeat(R, 1, 1).contiguous()
    ws = w1.unsqueeze(0).repeat(R, 1, 1).contiguous()
    ys = torch.empty((R, T, wl.d_out[0]), dtype=torch.bfloat16, device="cuda")
    del x1, w1
    torch.cuda.synchronize()
    st = torch.cuda.current_stream().cuda_stream
    xp, wp, yp = ([t[l].data_ptr() for l in range(R)] for t in (xs, ws, ys))
    ids = np.array(sorted(wl.adapters), np.int64)
    points = []
    for k in (1, 2, 4, 8, 16, 32, 64):
        g = np.random.default_rng([wl.seed, 91, k])
        batches = []
        for _ in range(NB):
            chosen = g.choice(ids, k, replace=False)
            rows = chosen[g.permutation(np.arange(T) % k)]
            batches.append(pool.slots_of(rows))

        def step(i):
            b, l = i % NB, i % R
            plan = pool.plan(None, None, batches[b], stream=st)
            pool.linear(plan, l, 0, xp[l], wp[l], yp[l], stream=st)
            hg.lora_plan_destroy(plan)

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        pool.set_timing(TIMING_PERIOD)
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(args.warmup + i)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        tim = pool.timing()
        pool.set_timing(False)
        kern = {name: round(1e3 * ms / n, 2) for name, (ms, n) in tim.items() if n}
        points.append({"distinct_adapters": k, "ms_per_step": el * 1e3 / args.steps,
                       "tokens_per_s": T * args.steps / el, "kernel_avg_us": kern})
        log(f"k={k}: {el * 1e6 / args.steps:.1f} us/step {kern}")
    base = points[0]["tokens_per_s"]
    for pt in points:
        pt["throughput_vs_one_adapter"] = pt["tokens_per_s"] / base
    print(json.dumps({"sweep": "distinct adapters per batch", "workload": WORKLOADS["c2"], "steps": args.steps,
                      "warmup": args.warmup, "points": points}), flush=True)


def run_stack(args):
    """The Llama-7B stack step: per step, one page-in of 16 cold adapters on a
    side stream (the copy engine into a device staging area, up to 4 layers
    per copy, then one scatter kernel per copy into the pages), one plan and
    the 224 LoRA-linear projections on the compute stream (per layer one
    lora_linear_multi call for q, k, v and one for gate, up, single calls for o
    and down; --single-calls: 224 lora_linear calls; each layer waits only for
    its own cold pages), KV blocks for the requests from the same pool, and
    the previous step's cold adapters evicted.  By default the page-in of step
    s + 1's cold adapters runs while step s computes (the pages' look-ahead:
    the next batch's adapters are copied during the current step); with
    --no-prefetch step s's copy starts when step s - 1's last call ends.
    Every (layer, projection) has its own W0, x and y buffers in HBM (copies
    of one draw per projection), so no step finds the previous step's data in
    the caches."""
    import torch

    import heterogeneous_adapter_gemm_amd as hg
    from heterogeneous_adapter_gemm_amd import host_tensor
    from workloads import make_workload
    from workloads.device import batch_index, build_pool

    wl = make_workload("c5", cache=False)
    T, L, P = wl.T, wl.n_layers, wl.n_proj
    log(f"config c5: T={T}, {L} layers x {P} projections, {len(wl.adapters)} adapters ({len(wl.cold_adapters)} cold)")
    t_setup = time.perf_counter()
    groups = [[p] for p in range(P)] if args.single_calls else wl.proj_groups()
    pool, _ = build_pool(wl, max_tokens=T, max_segments=16, stage_bytes=STACK_STAGE_BYTES,
                         max_multi=max(len(g) for g in groups))
    cold = list(wl.cold_adapters)
    blobs = {}
    for a in cold:
        A, B = wl.adapter_host_blob(a)
        blobs[a] = (host_tensor(A), host_tensor(B))
    cold_bytes = sum(x.numel() * 2 + y.numel() * 2 for x, y in blobs.values())
    xs, ws, ys = {}, {}, {}
    for p in range(P):
        w1 = hg.device_tensor(wl.w0(0, p))
        for l in range(L):
            ws[(l, p)] = w1.clone()
        del w1
    for src in sorted(set(wl.x_input_of_proj)):
        p = wl.x_input_of_proj.index(src)
        x1 = hg.device_tensor(wl.x(0, p))
        for l in range(L):
            xs[(l, src)] = x1.clone()
        del x1
    for l in range(L):
        for p in range(P):
            ys[(l, p)] = torch.empty((T, wl.d_out[p]), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s; pool {wl.num_pages} pages; cold set {cold_bytes / 1e9:.2f} GB")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    st, sst = main.cuda_stream, side.cuda_stream
    kv_sizes = [2 * r.n_tokens * L for r in wl.requests]
    cold_items = [(a, wl.adapters[a].rank, wl.adapters[a].alpha, blobs[a][0], blobs[a][1]) for a in cold]
    calls = [(l, g, xs[(l, wl.x_input_of_proj[g[0]])].data_ptr(), [ws[(l, p)].data_ptr() for p in g],
              [ys[(l, p)].data_ptr() for p in g]) for l in range(L) for g in groups]

    def run_calls(plan):
        for l, g, xp, wps, yps in calls:
            if len(g) == 1:
                pool.linear(plan, l, g[0], xp, wps[0], yps[0], stream=st)
            else:
                pool.linear_multi(plan, l, g, xp, wps, yps, stream=st)

    # KV blocks: the step's requests take kv_total pages (their blocks in request order, one
    # allocation of the batch); the next step's are taken, and this step's returned, while the
    # GPU still runs this step, so that host bookkeeping does not sit between the steps' GPU work
    kv_total = sum(kv_sizes)
    kv = [pool.alloc_kv(kv_total)]
    # Steps follow each other without a host wait, as an engine's would: step s pages the cold
    # weights in under ids a + ALIAS * (s % 2), and the cold set of step s - 1 is evicted once step
    # s's work is enqueued (the eviction waits for step s - 1's work only).  The copy of step s
    # still runs during step s: the side stream waits for the end of step s - 1's last call.
    ALIAS = 1 << 20
    cold_sets = [[(a + k * ALIAS, rk, al, hA, hB) for a, rk, al, hA, hB in cold_items] for k in (0, 1)]
    pre, dec = wl.prefill_requests(), wl.decode_requests()
    seg_start = np.concatenate([[0], np.cumsum([r.n_tokens for r in pre])]).astype(np.int32)

    def index_for(k):
        m = {a: a + k * ALIAS for a in cold}
        return (seg_start, pool.slots_of([m.get(r.adapter_id, r.adapter_id) for r in pre]),
                pool.slots_of([m.get(r.adapter_id, r.adapter_id) for r in dec]))

    state = {"s": 0, "end": None, "host_calls": 0.0, "host_rest": 0.0}
    prefetch = not args.no_prefetch

    def step():
        k = state["s"] % 2
        if prefetch:
            # look-ahead (the pages' prefetch during the current step): this step's cold set
            # was paged in while the previous step ran; the next step's goes in now, after the
            # set of the step before this one is evicted (the eviction waits for that step's work)
            if state["s"] == 0:
                pool.page_in_pinned_batch(cold_sets[k], stream=sst)
        else:
            if state["end"] is not None:
                side.wait_event(state["end"])      # this step's copy starts when the previous step ends
            pool.page_in_pinned_batch(cold_sets[k], stream=sst)   # in layer order across the cold adapters
        h0 = time.perf_counter()
        plan = pool.plan(*index_for(k), stream=st)
        run_calls(plan)
        hg.lora_plan_destroy(plan)
        h1 = time.perf_counter()
        end = torch.cuda.Event()
        end.record(main)
        state["end"] = end
        kv.append(pool.alloc_kv(kv_total))   # the next step's blocks
        pool.free_kv(kv.pop(0))
        if state["s"] > 0:
            for a in cold:
                pool.evict(a + (1 - k) * ALIAS)   # the previous step's cold set
        if prefetch:
            pool.page_in_pinned_batch(cold_sets[1 - k], stream=sst)   # the next step's
        state["host_calls"] += h1 - h0
        state["host_rest"] += time.perf_counter() - h1
        state["s"] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    pool.set_timing(TIMING_PERIOD)
    state["host_calls"] = state["host_rest"] = 0.0
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    host = {"plan_and_calls_ms": state["host_calls"] * 1e3 / args.steps,
            "evict_kv_page_in_ms": state["host_rest"] * 1e3 / args.steps,
            "note": f"host time per step enqueueing the plan and its {len(calls)} calls, then returning KV blocks, evicting "
                    "the previous cold set (which waits for that step's GPU work) and issuing the next page-in"}
    tim = pool.timing()
    pool.set_timing(False)
    torch.cuda.synchronize()
    for a in cold:
        pool.evict(a + ((state["s"] - 1) % 2) * ALIAS)
        if prefetch:
            pool.evict(a + (state["s"] % 2) * ALIAS)   # the next step's set, paged in ahead

    # the same step with every adapter resident (the cold ones paged in once, before timing)
    def step_resident():
        plan = pool.plan(*index_for(0), stream=st)
        run_calls(plan)
        hg.lora_plan_destroy(plan)
        kv.append(pool.alloc_kv(kv_total))
        pool.free_kv(kv.pop(0))

    pool.page_in_pinned_batch(cold_sets[0], stream=sst)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step_resident()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step_resident()
    torch.cuda.synchronize()
    el_res = time.perf_counter() - t1
    all_resident = {"value": T * args.steps / el_res, "unit": "tokens/s", "ms_per_step": el_res * 1e3 / args.steps,
                    "note": "the same step with the 16 cold adapters resident (no page-in in the step)"}
    # pinned host -> device copy rate of the runtime's copy engine, for the page-in rate beside it
    hbuf = torch.empty(256 << 20, dtype=torch.uint8).pin_memory()
    dbuf = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dbuf.copy_(hbuf, non_blocking=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(4):
        dbuf.copy_(hbuf, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    h2d_gbs = 4 * hbuf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del hbuf, dbuf

    # the timed calls: the library brackets call i of the timed region (counted from
    # set_timing) when i % TIMING_PERIOD == 0; a step's calls run in (layer, group) order
    n_calls = len(calls)
    sampled = [i % len(groups) for i in range(0, args.steps * n_calls, TIMING_PERIOD)]
    work, launches = stack_call_work(wl, groups)
    kern = {}
    for name, (ms, n) in tim.items():
        if not n:
            continue
        k = {"avg_us": 1e3 * ms / n, "launches": n}
        if name in work[0]:
            want_n = sum(launches[c][name] for c in sampled)
            if n != want_n:
                raise RuntimeError(f"{name}: {n} timed launches, expected {want_n}")
            byt = sum(work[c][name] for c in sampled)
            k["alg_bytes_per_launch"] = byt / n
            k["GBps"] = byt / (ms * 1e-3) / 1e9
            k["frac_hbm_peak"] = k["GBps"] / HBM_PEAK_GBS
        kern[name] = k
    g = kern["gemm"]
    fl = sum(work[c]["gemm_flops"] for c in sampled)
    g["TFLOPs"] = fl / (tim["gemm"][0] * 1e-3) / 1e12
    g["frac_mfma_peak"] = g["TFLOPs"] / BF16_PEAK_TFLOPS
    dk = [k for k in ("bgmv_shrink", "bgmv_expand", "sgmv_shrink", "sgmv_expand") if k in kern]
    d_ms = sum(tim[k][0] for k in dk)
    d_b = sum(sum(work[c][k] for c in sampled) for k in dk)
    n_proj_sampled = sum(len(groups[c]) for c in sampled)
    delta = {"kernels": dk, "us_per_projection": 1e3 * d_ms / n_proj_sampled,
             "alg_bytes_per_projection": d_b / n_proj_sampled,
             "GBps": d_b / (d_ms * 1e-3) / 1e9, "frac_hbm_peak": d_b / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
             "distinct_adapters": len({int(a) for a in wl.row_adapter() if a >= 0})}
    span = kern.get("page_in_batch")
    page_in = None
    if span:
        span_us = span["avg_us"] * span["launches"] / args.steps
        page_in = {"bytes_per_step": cold_bytes, "us_per_step": span_us,
                   "GBps_pcie": cold_bytes / (span_us * 1e-6) / 1e9, "pinned_h2d_copy_GBps": h2d_gbs,
                   "path": f"copy engine into a {STACK_STAGE_BYTES >> 20} MB device staging area, up to 4 layers "
                           "per copy, then one scatter kernel per copy; us_per_step spans the first copy to the last "
                           "page written",
                   "lookahead": not args.no_prefetch}
    traffic = measured_traffic("c5", "gemm")
    roof = {"bound": "mfma", "achieved": g["TFLOPs"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": g["frac_mfma_peak"], "traffic": traffic, "kernel": "gemm",
            "note": "the base GEMM launches of the timed calls (one per projection, all 7 projection shapes; "
                    "long-batch kernel with the prefill expand fused): their flops over their summed event durations"}
    if traffic is not None:
        roof["traffic_unit"] = ("HBM bytes per projection's GEMM (both launches of a split GEMM together), mean over the "
                                f"step's {L * P} projections (counters)")
        roof["alg_bytes"] = sum(w["gemm"] for w in work) / P
    out = {"metric": METRIC, "value": T * args.steps / el, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": el * 1e3 / args.steps, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": WORKLOADS["c5"], "name": "c5", "tokens_per_step": T,
                      "lora_linear_calls_per_step": len(calls), "projections_per_call": [len(g) for g in groups],
                      "parallelism": "none (1 GPU)"},
           "roofline": roof, "kernels": kern, "delta": delta, "page_in": page_in, "all_resident": all_resident, "host": host,
           "kernel_timing": KERNEL_TIMING}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = stack_cpu_baseline(wl)
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(line + "\n")


def run_peaks(args):
    """Sustained rates next to the published peaks: HBM by a device copy of 1 GiB (bytes read
    plus written over the copy's event time, best of 10) and by the read probe at the delta
    kernels' access shape (read_shape_rates), matrix cores by the library's probe
    (4 waves x 8 independent bf16 chains per workgroup; 16x16x32 ops with 8 workgroups per CU,
    32x32x16 ops with 2, the best settings of a sweep; best of 5)."""
    import torch

    import heterogeneous_adapter_gemm_amd as hg
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    best_copy = 0.0
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best_copy = max(best_copy, 2 * src.numel() * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rates = {}
    for shape, wg_per_cu in ((16, 8), (32, 2)):
        blocks, iters = wg_per_cu * cus, 80000 // wg_per_cu
        out = torch.empty(4 * blocks, dtype=torch.float32, device="cuda")
        hg.lora_probe_mfma(shape, 100, blocks, out)
        best = 0.0
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fl = hg.lora_probe_mfma(shape, iters, blocks, out)
            e1.record()
            torch.cuda.synchronize()
            best = max(best, fl / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        assert torch.isfinite(out).all()
        rates[shape] = best
    reads = read_shape_rates(torch, hg)
    line = json.dumps({"metric": "sustained rates", "hbm_copy_GBps": best_copy, "hbm_peak_GBps": HBM_PEAK_GBS,
                       "copy_frac": best_copy / HBM_PEAK_GBS,
                       "mfma_bf16_16x16x32_TFLOPs": rates[16], "mfma_bf16_32x32x16_TFLOPs": rates[32],
                       "mfma_bf16_peak_TFLOPs": BF16_PEAK_TFLOPS,
                       "mfma_16x16x32_frac": rates[16] / BF16_PEAK_TFLOPS,
                       "mfma_32x32x16_frac": rates[32] / BF16_PEAK_TFLOPS, "compute_units": cus,
                       "chunked_reads": reads})
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(line + "\n")


def run_gemm_vs_library(args):
    """The base product alone: the library's base_gemm against hipBLASLt (torch.matmul of the
    same bf16 operands, x [M, K] times W0 [N, K] transposed) on the stack step's three
    projection shapes (2,961 rows) and the 9,551-row prefill batch.  Warm inputs (the same
    buffers every launch), interleaved rounds, best of 8 x 10 launches by events each."""
    import torch

    import heterogeneous_adapter_gemm_amd as hg
    torch.manual_seed(0)
    shapes = [(2961, 4096, 4096), (2961, 11008, 4096), (2961, 4096, 11008), (9551, 4096, 4096)]
    layer = {(2961, 4096, 4096): 4, (2961, 11008, 4096): 2, (2961, 4096, 11008): 1}   # q, k, v, o; gate, up; down
    out = {}
    for M, N, K in shapes:
        x = torch.randn(M, K, device="cuda").to(torch.bfloat16)
        w = (torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16)
        y0 = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
        y1 = torch.empty_like(y0)
        runs = {"library": lambda: hg.base_gemm(hg.LORA_BF16, x, w, y0, M, N, K),
                "hipblaslt": lambda: torch.matmul(x, w.t(), out=y1)}
        for f in runs.values():
            for _ in range(3):
                f()
        torch.cuda.synchronize()
        best = {k: 1e30 for k in runs}
        for r in range(8):
            for name in (list(runs) if r % 2 == 0 else list(runs)[::-1]):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(10):
                    runs[name]()
                e1.record()
                torch.cuda.synchronize()
                best[name] = min(best[name], e0.elapsed_time(e1) * 1e3 / 10)
        err = float((y0.float() - y1.float()).abs().max())
        fl = 2.0 * M * N * K
        out[f"{M}x{N}x{K}"] = {"library_us": best["library"], "hipblaslt_us": best["hipblaslt"],
                               "library_TFLOPs": fl / best["library"] / 1e6,
                               "hipblaslt_TFLOPs": fl / best["hipblaslt"] / 1e6,
                               "max_abs_diff": err}
        log(f"{M}x{N}x{K}: library {best['library']:.1f} us, hipBLASLt {best['hipblaslt']:.1f} us")
    lay = {k: sum(n * out[f"{m}x{nn}x{kk}"][k] for (m, nn, kk), n in layer.items()) for k in ("library_us", "hipblaslt_us")}
    line = json.dumps({"metric": "base GEMM against hipBLASLt", "shapes": out,
                       "llama7b_layer_us": {"library": lay["library_us"], "hipblaslt": lay["hipblaslt_us"],
                                            "note": "4 x (2961, 4096, 4096) + 2 x (2961, 11008, 4096) + (2961, 4096, 11008)"}})
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(line + "\n")


def read_shape_rates(torch, hg):
    """HBM read rate of the delta kernels' access shape (the library's read probe: one 8 KiB
    chunk per wave, as a shrink wave reads one adapter row in its page) at several launch
    sizes, the chunks at random offsets of a buffer the size of the stack step's pool
    (21.8 GB) or consecutive; before each launch a 512 MB read evicts the caches.  Best of
    10 launches by events on the launch stream."""
    pool_bytes = 2656256 * 8192
    buf = torch.ones(pool_bytes, dtype=torch.uint8, device="cuda")
    flush = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    n_whole = pool_bytes // 8192
    g = np.random.default_rng(3)
    out = []
    for mb in (8.0, 16.0, 30.8, 53.0, 128.0, 512.0):
        n = int(mb * 1e6 / 8192)
        res = {"MB": n * 8192 / 1e6, "chunks": n}
        for order in ("random", "consecutive"):
            idx = g.integers(0, n_whole, n) if order == "random" else np.arange(n) + int(g.integers(0, n_whole - n))
            chunk = torch.from_numpy(idx.astype(np.int64)).cuda()
            sink = torch.empty(n, dtype=torch.float32, device="cuda")
            best = 1e30
            for r in range(12):
                flush.sum(dtype=torch.int64)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                hg.lora_probe_read(buf, pool_bytes, chunk, n, sink)
                e1.record()
                torch.cuda.synchronize()
                if r >= 2:
                    best = min(best, e0.elapsed_time(e1) * 1e3)
            res[order] = {"best_us": best, "GBps": n * 8192 / (best * 1e-6) / 1e9}
        out.append(res)
    del buf, flush
    torch.cuda.empty_cache()
    return out


def run_engine_trace(args):
    """Requests arrive Poisson(8) per step with adapters Zipf(1.0) over the stack workload's
    2000-adapter universe (ranks {8,16,32,64}, Llama-7B shapes, 32 layers x 7 projections),
    prompts U[128,512], U[8,40] tokens to generate.  The engine layer schedules them: a pinned
    host cache below a pool of --trace-slots slots that also holds every running request's KV
    pages (2 per token per layer), page-ins on a copy stream through a 512 MB staging area,
    requests admitted while their adapter is still copying.  Each step runs its plan's 224
    LoRA-linear projections as the stack step does (lora_linear_multi for q, k, v and for
    gate, up; 128 calls).  The host stays at most one step ahead of the GPU (a server needs step
    k's tokens before it schedules step k + 2).  Storage is a memory copy from one random blob
    (values do not matter here: parity of engine-built plans is a test).  Reports the tiers'
    hit rates and the page-in latency distribution after --warmup steps."""
    import torch

    import heterogeneous_adapter_gemm_amd as hg
    from workloads.gen import (LLAMA7B_DIN, LLAMA7B_DOUT, LLAMA7B_XSRC, bf16_bits_from_f32, c5_universe_ranks,
                               engine_trace, proj_groups_of)

    L, P, PAGE, MAX_T = 32, 7, 4096, 4096
    ranks = c5_universe_ranks()
    num_pages = int(args.trace_pool_gb * (1 << 30)) // (PAGE * 2)
    t_setup = time.perf_counter()
    free = np.random.default_rng(0).permutation(num_pages).astype(np.int32)
    groups = proj_groups_of(LLAMA7B_XSRC)
    pool = hg.DevicePool(hg.LORA_BF16, PAGE, num_pages, free, L, LLAMA7B_DIN, LLAMA7B_DOUT, args.trace_slots, 64,
                         MAX_T, 64, stage_bytes=STACK_STAGE_BYTES, max_multi=max(len(g) for g in groups))
    del free
    a_row, b_row = L * sum(LLAMA7B_DIN), L * sum(LLAMA7B_DOUT)
    src = bf16_bits_from_f32(np.random.default_rng(1).standard_normal(64 * max(a_row, b_row)).astype(np.float32)
                             * 0.01)

    def info(a):
        return int(ranks[a]), 2.0 * int(ranks[a]), 0

    def fill(a, A, B):
        A[:] = src[:A.size]
        B[:] = src[:B.size]

    log(f"engine trace: pool of {num_pages} pages ready ({time.perf_counter() - t_setup:.1f} s); pinning the host "
        f"cache ...")
    copy = torch.cuda.Stream()
    eng = hg.AdapterEngine(pool, info, fill, int(args.trace_host_gb * (1 << 30)), MAX_T, args.trace_distinct,
                           max_running=256, prefetch_window=64, admit_in_flight=True, max_wait_steps=16,
                           kv_pages_per_token=2 * L, copy_stream=copy)
    xs = {src_: torch.randn((MAX_T, LLAMA7B_DIN[LLAMA7B_XSRC.index(src_)]), device="cuda").to(torch.bfloat16)
          for src_ in sorted(set(LLAMA7B_XSRC))}
    ws = {}
    for p in range(P):
        w1 = (torch.randn((LLAMA7B_DOUT[p], LLAMA7B_DIN[p]), device="cuda") * 0.02).to(torch.bfloat16)
        for l in range(L):
            ws[(l, p)] = w1.clone()
        del w1
    ys = [torch.empty((MAX_T, LLAMA7B_DOUT[p]), dtype=torch.bfloat16, device="cuda") for p in range(P)]
    calls = [(l, g, xs[LLAMA7B_XSRC[g[0]]].data_ptr(), [ws[(l, p)].data_ptr() for p in g], [ys[p].data_ptr() for p in g])
             for l in range(L) for g in groups]
    torch.cuda.synchronize()
    log(f"engine trace: setup {time.perf_counter() - t_setup:.1f} s; pool {num_pages} pages, {args.trace_slots} "
        f"slots, host cache {args.trace_host_gb} GB")
    n_steps = args.warmup + args.steps
    trace = engine_trace(n_steps)
    main = torch.cuda.current_stream()
    st = main.cuda_stream
    ends = []
    rows, distinct, prefill, host_ms = [], [], [], []
    t0 = None
    for k in range(n_steps):
        if k == args.warmup:
            torch.cuda.synchronize()
            eng.reset_stats()
            rows, distinct, prefill, host_ms = [], [], [], []
            t0 = time.perf_counter()
        if len(ends) >= 2:
            ends.pop(0).synchronize()          # at most one step ahead of the GPU
        for rid, a, pr, mn in trace[k]:
            eng.submit(rid, a, pr, mn)
        th = time.perf_counter()
        b, plan = eng.step(stream=main)
        host_ms.append((time.perf_counter() - th) * 1e3)
        if plan is not None:
            for l, g, xp, wps, yps in calls:
                if len(g) == 1:
                    pool.linear(plan, l, g[0], xp, wps[0], yps[0], stream=st)
                else:
                    pool.linear_multi(plan, l, g, xp, wps, yps, stream=st)
        eng.step_done()
        ev = torch.cuda.Event()
        ev.record(main)
        ends.append(ev)
        rows.append(b["n_rows"])
        distinct.append(b["n_distinct"])
        prefill.append(b["n_prefill"])
        if k % 50 == 0:
            log(f"step {k}: {b['n_prefill']} prompts + {b['n_requests'] - b['n_prefill']} decode rows, "
                f"{b['n_distinct']} adapters, {b['n_rows']} rows")
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    s = eng.stats()
    arr = s["arrivals_resident"] + s["arrivals_missing"]
    pins = s["host_hits"] + s["host_misses"]
    out = {"metric": "engine trace: adapter-tier hit rates and page-in latency under load", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": el * 1e3 / args.steps,
           "rows_per_s": sum(rows) / el, "data": "synthetic",
           "config": {"workload": "Poisson(8) arrivals per step, adapters Zipf(1.0) over 2000 of ranks {8,16,32,64}, "
                                  "Llama-7B 32 layers x 7 projections, prompts U[128,512], U[8,40] new tokens; "
                                  "KV 2 pages per token per layer in the same pool",
                      "slots": args.trace_slots, "pool_GB": args.trace_pool_gb, "host_cache_GB": args.trace_host_gb,
                      "max_distinct_adapters": args.trace_distinct, "max_step_tokens": MAX_T, "max_running": 256,
                      "prefetch_window": 64, "admit_in_flight": True, "max_wait_steps": 16},
           "per_step": {"rows_mean": float(np.mean(rows)), "prompts_mean": float(np.mean(prefill)),
                        "distinct_mean": float(np.mean(distinct)), "distinct_max": int(np.max(distinct)),
                        "engine_step_host_ms_p50": float(np.percentile(host_ms, 50)),
                        "engine_step_host_ms_p99": float(np.percentile(host_ms, 99))},
           "gpu_tier": {"arrivals": arr, "hit_rate": s["arrivals_resident"] / max(1, arr),
                        "evictions": s["gpu_evictions"], "room_stalls": s["room_stalls"],
                        "kv_stalls": s["kv_stalls"]},
           "host_tier": {"page_ins": pins, "hit_rate": s["host_hits"] / max(1, pins),
                         "drops": s["host_evictions"], "storage_ms_p50": s["storage_ms_p50"],
                         "storage_ms_p99": s["storage_ms_p99"]},
           "page_in": {"adapters": s["page_ins"], "GB_per_step": s["page_in_bytes"] / args.steps / 1e9,
                       "ms_p50": s["page_in_ms_p50"], "ms_p99": s["page_in_ms_p99"], "ms_max": s["page_in_ms_max"],
                       "copy_batch_ms_p50": s["copy_ms_p50"], "copy_batch_ms_p99": s["copy_ms_p99"],
                       "latency": "issue (an event on an idle stream when the step issues it) to the copy's last "
                                  "page written, GPU clock, one sample per adapter"},
           "admission_wait": {"ms_p50_resident": s["wait_ms_hit_p50"], "ms_p99_resident": s["wait_ms_hit_p99"],
                              "ms_p50_missing": s["wait_ms_miss_p50"], "ms_p99_missing": s["wait_ms_miss_p99"],
                              "steps_p99": s["wait_steps_p99"], "steps_max": s["wait_steps_max"],
                              "note": "submit to the step that admits the request, host clock, split by whether "
                                      "the adapter was on the GPU at arrival"},
           "finished": s["finished"], "admitted": s["admitted"]}
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(line + "\n")
    eng.close()
    pool.close()


def stack_call_work(wl, groups):
    """Algorithmic work of one call of the stack step, per call shape (a run of
    projections that share x), and the launches each kernel class makes in it
    (the shrinks and the decode rows' expand serve all of the call's projections
    in one launch each).
    Bytes the method must move: W0, x and y once per projection; the distinct
    adapters' A or B rows once; v as fp32; the decode rows' y read and written
    once by the expand, in bf16; x once per shrink launch, which serves every
    projection of the call.  Flops: the base products'."""
    e = wl.elem_bytes
    T = wl.T
    dec = [r.adapter_id for r in wl.decode_requests() if r.adapter_id >= 0]
    pre = [r for r in wl.prefill_requests() if r.adapter_id >= 0]
    rk = lambda a: wl.adapters[a].rank
    dec_rd = sum(rk(a) for a in set(dec))                  # distinct decode adapters' rank-rows
    dec_rr = sum(rk(a) for a in dec)                       # rank-rows over the decode rows
    pre_rd = sum(rk(a) for a in {r.adapter_id for r in pre})
    pre_rows = sum(r.n_tokens for r in pre)
    pre_rr = sum(rk(r.adapter_id) * r.n_tokens for r in pre)
    work, launches = [], []
    for g in groups:
        di = wl.d_in[g[0]]
        w = {"gemm": 0.0, "gemm_flops": 0.0, "bgmv_shrink": len(dec) * di * e, "bgmv_expand": 0.0,
             "sgmv_shrink": pre_rows * di * e, "sgmv_expand": 0.0}
        for p in g:
            do = wl.d_out[p]
            w["gemm"] += (do * di + T * di + T * do) * e + pre_rd * do * e + 4 * pre_rr
            w["gemm_flops"] += 2.0 * T * di * do
            w["bgmv_shrink"] += dec_rd * di * e + 4 * dec_rr
            w["bgmv_expand"] += dec_rd * do * e + 2 * len(dec) * do * e + 4 * dec_rr
            w["sgmv_shrink"] += pre_rd * di * e + 4 * pre_rr
            w["sgmv_expand"] += pre_rd * do * e + 2 * pre_rows * do * e + 4 * pre_rr
        work.append(w)
        n = len(g)
        launches.append({"gemm": n, "bgmv_expand": 1, "sgmv_expand": n, "bgmv_shrink": 1, "sgmv_shrink": 1})
    return work, launches


def stack_cpu_baseline(wl, n_rows=1280):
    """The oracle on the host cores for the stack: n_rows sampled rows through
    the 7 projections of layer 0, scaled to the 32 layers."""
    import oracle
    ra = wl.row_adapter()
    rows = np.sort(np.random.default_rng(5).choice(wl.T, n_rows, replace=False))
    ids = sorted({int(ra[t]) for t in rows if ra[t] >= 0})
    ra_s = np.where(np.isin(ra, ids), ra, -1)
    inputs = []
    for p in range(wl.n_proj):
        ad = {}
        for a in ids:
            A, B = wl.adapter_AB(a, 0, p)
            ad[a] = (wl.adapters[a].rank, wl.adapters[a].alpha, A, B)
        inputs.append((wl.x(0, p), wl.w0(0, p), ad))
    t0 = time.perf_counter()
    for x, w0, ad in inputs:
        oracle.lora_linear(x, w0, ra_s, ad, rows=rows)
    el = time.perf_counter() - t0
    per_token_s = el * wl.n_layers / n_rows
    return {"value": 1.0 / per_token_s, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n_rows} rows through the 7 projections of layer 0 ({el:.1f} s), scaled to {wl.n_layers} "
                      "layers; fp64 loops, OpenMP over rows"}

if __name__ == "__main__":
    main()
