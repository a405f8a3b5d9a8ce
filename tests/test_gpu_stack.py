"""The Llama-7B stack step on the GPU at full size (32 layers x q, k, v, o, gate,
up, down; 8 prefill segments + 192 decode rows), checked against the oracle
on every one of the 224 (layer, projection) outputs.

The step follows the pages' engine step ("Multi-LoRA serving: S-LoRA, Punica
and adapter batching", What the engine does each step): the adapters of the
step are resident except 16 cold ones, which are paged in from pinned host
memory on a side stream while the layers run (the copy engine into a 512 MB
staging area, layer by layer, then a scatter kernel into the pages); every
layer's call waits only for that layer's pages.  KV blocks (2 pages per token
per layer) are taken from the same pool first.

Checks:
  * every call, full output on at least 64 rows: both ends of every prefill
    segment, a row of every 256-row tile of the prefill rows (the base GEMM's
    row tiles), every decode row routed to a cold adapter, a row of every
    prefill segment routed to one, and random decode and prefill rows;
  * layers 0, 15 and 31 (all 7 projections; layer 31's cold pages arrive
    last): the delta alone (w0 = NULL into a zeroed output, enqueued right
    after the layer's full call, so it waits on the same page-in) on every
    row, against the oracle's delta with its own bar, 2e-2 x RMS(delta): a
    wrong rank-row or page that the base term hides fails it.

The calls are the ones the stack benchmark times: one lora_linear_multi call per
run of projections that read the same input (q, k, v; gate, up), single
projections (o, down) through the same entry point.

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

DELTA_LAYERS = (0, 15, 31)
STAGE_BYTES = 512 << 20   # page-ins through the copy engine and a device staging area
ROWS_PER_CALL = 64


def say(*a):
    print("[case]", *a, flush=True)


def _adapters(wl, ids, layer, proj):
    """{id: (rank, alpha, A, B)} of (layer, proj), drawn in parallel."""
    from workloads.gen import _executor
    ids = sorted(ids)
    ab = list(_executor().map(lambda a: wl.adapter_AB(a, layer, proj), ids))
    return {a: (wl.adapters[a].rank, wl.adapters[a].alpha, A, B) for a, (A, B) in zip(ids, ab)}


def test_llama7b_stack_step_with_cold_page_in():
    import heterogeneous_adapter_gemm_amd as hg
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hg.library()
    t0 = time.perf_counter()
    wl = make_workload("c5", cache=False)
    T = wl.T
    say("c5: T =", T, "rows,", len(wl.adapters), "adapters,", len(wl.cold_adapters), "cold,", wl.num_pages, "pages")
    groups = wl.proj_groups()
    pool, _ = build_pool(wl, max_tokens=T, max_segments=16, stage_bytes=STAGE_BYTES,
                         max_multi=max(len(g) for g in groups))
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
    yd = {(l, p): torch.zeros((T, wl.d_out[p]), dtype=torch.bfloat16, device="cuda")
          for l in DELTA_LAYERS for p in range(wl.n_proj)}
    torch.cuda.synchronize()   # (the zero fills) before the step's calls
    for l in range(wl.n_layers):
        for g in groups:
            x = xs[wl.x_input_of_proj[g[0]]]
            pool.linear_multi(plan, l, g, x, [ws[p] for p in g], [ys[(l, p)] for p in g], stream=main.cuda_stream)
            if l in DELTA_LAYERS:
                pool.linear_multi(plan, l, g, x, [None] * len(g), [yd[(l, p)] for p in g], stream=main.cuda_stream)
    torch.cuda.synchronize()
    hg.lora_plan_destroy(plan)
    pool.drop_host_copies()
    say(f"c5: {len(ys) + len(yd)} projection outputs done ({time.perf_counter() - t0:.1f} s)")

    ra = wl.row_adapter()
    n_pre = wl.n_prefill_rows
    st = np.concatenate([[0], np.cumsum([r.n_tokens for r in wl.prefill_requests()])])
    cold = set(wl.cold_adapters)
    ends = {int(st[s]) for s in range(len(st) - 1)} | {int(st[s + 1] - 1) for s in range(len(st) - 1)}
    cold_dec = {int(t) for t in np.nonzero([a in cold for a in ra[n_pre:]])[0] + n_pre}
    cold_seg = [s for s in range(len(st) - 1) if int(ra[st[s]]) in cold]
    assert cold_dec and cold_seg, "the step must route decode rows and a segment to cold adapters"
    g = np.random.default_rng(55)
    x_np = {src: wl.x(0, p) for p, src in enumerate(wl.x_input_of_proj)}
    w_np = [wl.w0(0, p) for p in range(wl.n_proj)]
    worst = worst_d = 0.0
    for l in range(wl.n_layers):
        for p in range(wl.n_proj):
            rows = set(ends) | cold_dec
            rows |= {int(g.integers(t0_, min(t0_ + 256, n_pre))) for t0_ in range(0, n_pre, 256)}
            rows |= {int(g.integers(st[s], st[s + 1])) for s in cold_seg}
            while len(rows) < ROWS_PER_CALL:
                rows.add(int(g.integers(n_pre, T)) if len(rows) % 2 else int(g.integers(0, n_pre)))
            rows = sorted(rows)
            ids = {int(ra[t]) for t in rows if ra[t] >= 0}
            ad = _adapters(wl, ids, l, p)
            # rows outside the sample are not computed; their adapters need not be given
            ra_s = np.where(np.isin(ra, sorted(ids)), ra, -1)
            x, w = x_np[wl.x_input_of_proj[p]], w_np[p]
            want = oracle.lora_linear(x, w, ra_s, ad, rows=rows)
            got = to_np(ys[(l, p)][rows])
            worst = max(worst, parity(got, want, what=f"c5 layer {l} {wl.proj_names[p]} ({len(rows)} rows)"))
            if (l, p) in yd:
                ad_all = _adapters(wl, {int(a) for a in ra if a >= 0}, l, p)
                want_d = oracle.lora_linear(x, None, ra, ad_all)
                got_d = to_np(yd[(l, p)])
                worst_d = max(worst_d, parity(got_d, want_d, what=f"c5 layer {l} {wl.proj_names[p]} delta, all rows"))
                assert np.all(got_d[ra < 0] == 0.0), "rows with no adapter must not be touched"
    say(f"c5: worst max|err| / RMS = {worst:.3e}, delta only {worst_d:.3e} ({time.perf_counter() - t0:.1f} s)")
