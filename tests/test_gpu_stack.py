"""The Llama-7B stack step on the GPU at full size (32 layers x q, k, v, o, gate,
up, down; 8 prefill segments + 192 decode rows), checked against the oracle on
sampled rows of every one of the 224 LoRA-linear calls.

The step follows the pages' engine step ("Multi-LoRA serving: S-LoRA, Punica
and adapter batching", What the engine does each step): the adapters of the
step are resident except 16 cold ones, which are paged in from pinned host
memory on a side stream while the layers run; every layer's call waits only
for that layer's pages.  KV blocks (2 pages per token per layer) are taken from
the same pool first.

The base weights and inputs of projection p are the same arrays in every layer
(the adapters differ per layer); the calls still run over their own layer's
adapter pages, which is what the check is about.
"""
from __future__ import annotations

import time

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import parity, to_np
from workloads import make_workload
from workloads.device import batch_index, build_pool, replay

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print("[case]", *a, flush=True)


def test_llama7b_stack_step_with_cold_page_in():
    import heterogeneous_adapter_gemm_amd as hg
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hg.library()
    t0 = time.perf_counter()
    wl = make_workload("c5", cache=False)
    T = wl.T
    say("c5: T =", T, "rows,", len(wl.adapters), "adapters,", len(wl.cold_adapters), "cold,", wl.num_pages, "pages")
    pool, _ = build_pool(wl, max_tokens=T, max_segments=16)
    say(f"c5: resident adapters paged in ({time.perf_counter() - t0:.1f} s)")

    # the step: KV blocks, then the cold adapters' page-in on a side stream
    side = torch.cuda.Stream()
    kv = replay(wl, pool, wl.step_ops, stream=side.cuda_stream, settle=False, batch=True)
    assert sum(b.size for b in kv) == 2 * T * wl.n_layers
    ix = batch_index(wl, pool)
    main = torch.cuda.current_stream()
    plan = pool.plan(ix.get("seg_start"), ix.get("seg_slot"), ix.get("token_slot"), stream=main.cuda_stream)

    xs = {src: hg.device_tensor(wl.x(0, p)) for p, src in enumerate(wl.x_input_of_proj)}
    ws = [hg.device_tensor(wl.w0(0, p)) for p in range(wl.n_proj)]
    ys = {(l, p): torch.empty((T, wl.d_out[p]), dtype=torch.bfloat16, device="cuda")
          for l in range(wl.n_layers) for p in range(wl.n_proj)}
    for l in range(wl.n_layers):
        for p in range(wl.n_proj):
            pool.linear(plan, l, p, xs[wl.x_input_of_proj[p]], ws[p], ys[(l, p)], stream=main.cuda_stream)
    torch.cuda.synchronize()
    hg.lora_plan_destroy(plan)
    pool.drop_host_copies()
    say(f"c5: 224 calls done ({time.perf_counter() - t0:.1f} s)")

    # sampled rows: both ends of every prefill segment, decode rows, and rows of cold adapters
    ra = wl.row_adapter()
    n_pre = wl.n_prefill_rows
    st = np.concatenate([[0], np.cumsum([r.n_tokens for r in wl.prefill_requests()])])
    cold = set(wl.cold_adapters)
    g = np.random.default_rng(55)
    base_rows = sorted({int(st[s]) for s in range(len(st) - 1)} | {int(st[s + 1] - 1) for s in range(len(st) - 1)})
    cold_rows = [int(t) for t in np.nonzero([a in cold for a in ra])[0]]
    assert cold_rows, "the step must route rows to cold adapters"
    worst = 0.0
    x_np = {src: wl.x(0, p) for p, src in enumerate(wl.x_input_of_proj)}
    w_np = [wl.w0(0, p) for p in range(wl.n_proj)]
    for l in range(wl.n_layers):
        for p in range(wl.n_proj):
            rows = sorted(set(g.choice(base_rows, 2, replace=False).tolist())
                          | set(g.integers(n_pre, T, 2).tolist())
                          | set(g.choice(cold_rows, 2, replace=False).tolist()))
            ids = sorted({int(ra[t]) for t in rows})
            ad = {}
            for a in ids:
                A, B = wl.adapter_AB(a, l, p)
                ad[a] = (wl.adapters[a].rank, wl.adapters[a].alpha, A, B)
            # rows outside the sample are not computed; their adapters need not be given
            ra_s = np.where(np.isin(ra, ids), ra, -1)
            want = oracle.lora_linear(x_np[wl.x_input_of_proj[p]], w_np[p], ra_s, ad, rows=rows)
            got = to_np(ys[(l, p)][rows])
            worst = max(worst, parity(got, want, what=f"c5 layer {l} {wl.proj_names[p]}"))
    say(f"c5: worst max|err| / RMS = {worst:.3e} ({time.perf_counter() - t0:.1f} s)")
