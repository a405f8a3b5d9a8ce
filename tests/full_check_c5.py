"""Every row of every one of the 224 (layer, projection) outputs of the Llama-7B
stack step against the oracle, full output and delta alone.

Too long for the GPU test suite (about five minutes, most of it the oracle on
the host), so pytest does not collect it; run it on a GPU machine from the
repository root:

    python -u -m tests.full_check_c5

The step is the stack benchmark's: the resident adapters paged in first, KV
blocks from the same pool, the 16 cold adapters paged in on a side stream
through a 512 MB staging area while the layers run, and per layer one
lora_linear_multi call for q, k, v and one for gate, up, single calls for o
and down.  The delta alone (w0 = NULL into a zeroed output) is checked on
every row for layers 0, 15 and 31; the full output on every row of all 32
layers.

The oracle (the plain definition in fp64) gives each output as the base term
x W0^T plus the layer's delta.  Projection p reads the same x and W0 in every
layer (only the adapters differ per layer), so the base term is computed once
per projection (oracle with no adapter rows) and the delta once per (layer,
projection) (oracle with w0 = NULL); their fp64 sum is the definition's value.
Bar: max |err| <= 2e-2 x RMS of the oracle's output, per output, as in the
parity tests.
"""
from __future__ import annotations

import sys
import time

import numpy as np

import oracle
from tests.gpu_helpers import parity, to_np
from workloads import make_workload
from workloads.device import batch_index, build_pool, replay

STAGE_BYTES = 512 << 20
DELTA_LAYERS = (0, 15, 31)


def say(*a):
    print("[full]", *a, flush=True)


def main() -> int:
    import torch

    import heterogeneous_adapter_gemm_amd as hg
    from workloads.gen import _executor
    if not torch.cuda.is_available():
        say("needs a GPU")
        return 2
    hg.library()
    t0 = time.perf_counter()
    wl = make_workload("c5", cache=False)
    T, L, P = wl.T, wl.n_layers, wl.n_proj
    groups = wl.proj_groups()
    pool, _ = build_pool(wl, max_tokens=T, max_segments=16, stage_bytes=STAGE_BYTES,
                         max_multi=max(len(g) for g in groups))
    say(f"T = {T}, {L} layers x {P} projections, groups {groups}; resident adapters paged in "
        f"({time.perf_counter() - t0:.1f} s)")
    side = torch.cuda.Stream()
    replay(wl, pool, wl.step_ops, stream=side.cuda_stream, settle=False, batch=True)
    ix = batch_index(wl, pool)
    main_s = torch.cuda.current_stream()
    plan = pool.plan(ix.get("seg_start"), ix.get("seg_slot"), ix.get("token_slot"), stream=main_s.cuda_stream)
    xs = {src: hg.device_tensor(wl.x(0, p)) for p, src in enumerate(wl.x_input_of_proj)}
    ws = [hg.device_tensor(wl.w0(0, p)) for p in range(P)]
    ys = {(l, p): torch.empty((T, wl.d_out[p]), dtype=torch.bfloat16, device="cuda") for l in range(L) for p in range(P)}
    yd = {(l, p): torch.zeros((T, wl.d_out[p]), dtype=torch.bfloat16, device="cuda")
          for l in DELTA_LAYERS for p in range(P)}
    torch.cuda.synchronize()
    for l in range(L):
        for g in groups:
            x = xs[wl.x_input_of_proj[g[0]]]
            pool.linear_multi(plan, l, g, x, [ws[p] for p in g], [ys[(l, p)] for p in g], stream=main_s.cuda_stream)
            if l in DELTA_LAYERS:
                pool.linear_multi(plan, l, g, x, [None] * len(g), [yd[(l, p)] for p in g], stream=main_s.cuda_stream)
    torch.cuda.synchronize()
    hg.lora_plan_destroy(plan)
    pool.drop_host_copies()
    say(f"step done ({time.perf_counter() - t0:.1f} s)")

    ra = wl.row_adapter()
    ids = sorted({int(a) for a in ra if a >= 0})
    null = np.full(T, -1, np.int32)
    base = {}
    for p in range(P):
        base[p] = oracle.lora_linear(wl.x(0, p), wl.w0(0, p), null, {})
        say(f"oracle base term of {wl.proj_names[p]} ({time.perf_counter() - t0:.1f} s)")
    worst = worst_d = 0.0
    for l in range(L):
        for p in range(P):
            ab = list(_executor().map(lambda a: wl.adapter_AB(a, l, p), ids))
            ads = {a: (wl.adapters[a].rank, wl.adapters[a].alpha, A, B) for a, (A, B) in zip(ids, ab)}
            delta = oracle.lora_linear(wl.x(0, p), None, ra, ads)
            name = f"layer {l} {wl.proj_names[p]}"
            worst = max(worst, parity(to_np(ys[(l, p)]), base[p] + delta, what=f"{name}, all {T} rows"))
            if (l, p) in yd:
                got_d = to_np(yd[(l, p)])
                worst_d = max(worst_d, parity(got_d, delta, what=f"{name} delta, all {T} rows"))
                assert np.all(got_d[ra < 0] == 0.0), "rows with no adapter must not be touched"
    say(f"all {L * P} outputs, every row: worst max|err| / RMS = {worst:.3e}; delta alone ({len(yd)} outputs) "
        f"{worst_d:.3e} ({time.perf_counter() - t0:.1f} s)")
    pool.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
