"""The engine layer on the GPU: plans built by lora_engine_step, with adapters
brought in from the engine's pinned host cache while earlier steps run, give
LoRA-linear outputs equal to the oracle's on every row of every step.

Small model (2 layers x 2 projections, 1024/2048 -> 1536/1024), 16 adapters of
ranks {8, 16, 32, 64}, a pool with room for about four of them (so adapters
are evicted and paged in again), a host cache for six (so some come from
storage more than once), page-ins through a device staging area on a copy
stream, and requests admitted while their adapter is still being copied
(each layer's call then waits for that layer's pages).  Bar: max |err| <=
2e-2 x RMS of the oracle's output per call.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import bf16_bits, parity, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_LAYERS, P = 2, 512
D_IN, D_OUT = (1024, 2048), (1536, 1024)
N_ADAPTERS = 16


def say(*a):
    print("[case]", *a, flush=True)


class Store:
    """Storage: seeded bf16 factors per adapter, (layer, projection) pieces in blob order."""

    def __init__(self, seed=5):
        g = np.random.default_rng(seed)
        self.ranks = {a: int(g.choice([8, 16, 32, 64])) for a in range(N_ADAPTERS)}
        self.ab = {}
        for a, r in self.ranks.items():
            for l in range(N_LAYERS):
                for p in range(2):
                    A = bf16_bits((g.standard_normal((r, D_IN[p])) * D_IN[p] ** -0.5).astype(np.float32))
                    B = bf16_bits((g.standard_normal((r, D_OUT[p])) * 0.05).astype(np.float32))
                    self.ab[(a, l, p)] = (A, B)
        self.loads = 0

    def info(self, a):
        return self.ranks[a], 2.0 * self.ranks[a], 0

    def fill(self, a, A, B):
        ao = bo = 0
        for l in range(N_LAYERS):
            for p in range(2):
                x, y = self.ab[(a, l, p)]
                A[ao:ao + x.size] = x.reshape(-1)
                B[bo:bo + y.size] = y.reshape(-1)
                ao += x.size
                bo += y.size
        assert ao == A.size and bo == B.size
        self.loads += 1

    def adapters(self, ids, l, p):
        return {a: (self.ranks[a], 2.0 * self.ranks[a], *self.ab[(a, l, p)]) for a in ids}


def test_engine_steps_match_oracle_with_in_flight_page_ins():
    import heterogeneous_adapter_gemm_amd as hg
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hg.library()
    store = Store()
    per_rank = N_LAYERS * sum(-(-i // P) + -(-o // P) for i, o in zip(D_IN, D_OUT))
    num_pages = per_rank * 4 * 30
    g = np.random.default_rng(11)
    pool = hg.DevicePool(hg.LORA_BF16, P, num_pages, g.permutation(num_pages), N_LAYERS, D_IN, D_OUT, 6, 64, 256, 16,
                         stage_bytes=4 << 20)
    unit = N_LAYERS * (sum(D_IN) + sum(D_OUT)) * 2
    copy = torch.cuda.Stream()
    eng = hg.AdapterEngine(pool, store.info, store.fill, 180 * unit, max_step_tokens=192, max_distinct_adapters=4,
                           max_running=48, prefetch_window=6, admit_in_flight=True, max_wait_steps=4,
                           copy_stream=copy)
    zipf = 1.0 / np.arange(1, N_ADAPTERS + 1)
    zipf /= zipf.sum()
    main = torch.cuda.current_stream()
    ws = {(l, p): bf16_bits((g.standard_normal((D_OUT[p], D_IN[p])) * 0.02).astype(np.float32))
          for l in range(N_LAYERS) for p in range(2)}
    wd = {k: hg.device_tensor(v) for k, v in ws.items()}
    rid, steps_checked, rows_checked = 0, 0, 0
    for step in range(200):
        if step >= 24:
            left = eng.stats()
            if left["waiting"] == 0 and left["running"] == 0:
                break
        if step < 24:
            for _ in range(int(g.integers(2, 6))):
                a = -1 if g.random() < 0.1 else int(g.choice(N_ADAPTERS, p=zipf))
                eng.submit(rid, a, int(g.integers(1, 41)), int(g.integers(1, 5)))
                rid += 1
        b, plan = eng.step(stream=main)
        if plan is None:
            eng.step_done()
            continue
        ra = eng.row_adapter()
        T = b["n_rows"]
        assert ra.size == T
        say(f"step {step}: {b['n_prefill']} prefill + {b['n_requests'] - b['n_prefill']} decode requests, "
            f"{T} rows, {b['n_distinct']} adapters")
        xs, ys = {}, {}
        for l in range(N_LAYERS):
            for p in range(2):
                xs[(l, p)] = bf16_bits(g.standard_normal((T, D_IN[p])).astype(np.float32))
                ys[(l, p)] = torch.empty((T, D_OUT[p]), dtype=torch.bfloat16, device="cuda")
                pool.linear(plan, l, p, hg.device_tensor(xs[(l, p)]), wd[(l, p)], ys[(l, p)], stream=main)
        torch.cuda.synchronize()
        eng.step_done()
        ids = {int(a) for a in ra if a >= 0}
        for (l, p), y in ys.items():
            want = oracle.lora_linear(xs[(l, p)], ws[(l, p)], ra, store.adapters(ids, l, p))
            parity(to_np(y), want, what=f"engine step {step} layer {l} proj {p}")
        steps_checked += 1
        rows_checked += T
    st = eng.stats()
    say("engine stats:", {k: st[k] for k in ("page_ins", "gpu_evictions", "host_misses", "host_evictions",
                                             "page_in_ms_p50", "page_in_ms_p99", "copy_ms_p50")})
    assert st["finished"] == rid, "every request finished"
    assert st["gpu_evictions"] > 0 and st["host_evictions"] > 0, "the trace must evict from both tiers"
    assert st["page_ins"] > N_ADAPTERS // 2 and st["page_in_ms_p99"] > 0.0 and st["copy_ms_p50"] > 0.0
    assert steps_checked >= 20 and rows_checked > 500
    eng.close()
    pool.close()
