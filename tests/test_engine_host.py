"""The engine layer (host cache tier, GPU-tier LRU, look-ahead page-ins,
admission) on host-only pools, no GPU.

Two kinds of checks:
  * the reference model of the policy (oracle.engine_model) against what the
    pages fix, on hand-made scenarios and on random traces: an adapter a
    running request uses is never evicted; the victim is the least recently
    used unused adapter; the step's caps hold; look-ahead brings in the
    adapters of waiting requests; the host cache is least recently used; no
    request starves once it has waited max_wait_steps steps;
  * the library's engine against that model, decision for decision: the
    step's requests in row order, the pool's slots and free list, the
    counters, and the storage loads.
"""
from __future__ import annotations

import numpy as np
import pytest

from heterogeneous_adapter_gemm_amd import _lib as L
from heterogeneous_adapter_gemm_amd.runtime import AdapterEngine, DevicePool
from oracle.engine_model import EngineModel
from oracle.pool_model import PoolModel

P = 512
N_LAYERS = 2
D_IN = (512, 1024)
D_OUT = (512, 1536)
MAX_RANK = 16
ELEM = 2                                   # bf16
PAGES_PER_RANK = N_LAYERS * sum(-(-i // P) + -(-o // P) for i, o in zip(D_IN, D_OUT))   # 14
UNIT = N_LAYERS * (sum(D_IN) + sum(D_OUT)) * ELEM                                          # host bytes per rank-row


class Storage:
    """The storage tier: adapter metadata and a pattern fill, with a log of the loads."""

    def __init__(self, ranks, base_id=0):
        self.ranks = dict(ranks)
        self.base_id = base_id
        self.loads = []
        self.fail = set()

    def info(self, a):
        return self.ranks[a], 2.0 * self.ranks[a], self.base_id

    def fill(self, a, A, B):
        if a in self.fail:
            raise IOError(f"adapter {a} is not in storage")
        r = self.ranks[a]
        assert A.size == r * N_LAYERS * sum(D_IN) and B.size == r * N_LAYERS * sum(D_OUT)
        A[:] = a & 0xFFFF
        B[:] = (a + 1) & 0xFFFF
        self.loads.append(a)


def make(ranks, num_pages, max_slots=8, host_units=48, max_step_tokens=48, max_distinct=4, max_running=16,
         window=8, max_wait=0, kvpt=0, max_segments=16, free_seed=1, base_id=0):
    """The library's engine on a host-only pool and the model on a PoolModel, same settings."""
    free = np.random.default_rng(free_seed).permutation(num_pages).astype(np.int32)
    pool = DevicePool(L.LORA_BF16, P, num_pages, free, N_LAYERS, D_IN, D_OUT, max_slots, MAX_RANK, 256,
                      max_segments, base_id=base_id, device=None)
    store = Storage(ranks, base_id)
    eng = AdapterEngine(pool, store.info, store.fill, host_units * UNIT, max_step_tokens, max_distinct, max_running,
                        window, True, max_wait, kvpt)
    pm = PoolModel(num_pages, P, free, N_LAYERS, D_IN, D_OUT, max_slots, MAX_RANK, base_id=base_id)
    mstore = Storage(ranks, base_id)
    model = EngineModel(pm, ELEM, host_units * UNIT, max_step_tokens, max_distinct, max_running, window, max_wait,
                        kvpt, max_segments, mstore.info)
    return pool, eng, store, model


COUNTERS = ("steps", "rows", "admitted", "finished", "arrivals_resident", "arrivals_missing", "host_hits",
            "host_misses", "page_ins", "gpu_evictions", "host_evictions", "room_stalls", "kv_stalls", "cancelled")


def step_both(pool, eng, model):
    b, plan = eng.step()
    pre, dec = model.step()
    want = pre + dec
    assert list(b["requests"]) == want, f"step {model.step_no}: requests differ"
    assert b["n_prefill"] == len(pre)
    assert list(b["rows"]) == [model.req[q]["prompt"] for q in pre] + [1] * len(dec)
    assert b["n_rows"] == sum(b["rows"])
    assert (plan is None) == (len(want) == 0)
    for a in set(int(x) for x in b["adapters"] if x >= 0):
        assert pool.slot_of(a) == model.pool.slot_of(a)
    assert list(pool.free_list()) == model.pool.free_list()
    st = eng.stats()
    for k in COUNTERS:
        assert st[k] == model.c[k], f"step {model.step_no}: counter {k}: {st[k]} != {model.c[k]}"
    return b, pre, dec


def done_both(eng, model):
    eng.step_done()
    model.step_done()


def zipf_trace(seed, n_steps, n_adapters=40, rate=2.5, null_frac=0.1, max_prompt=24, max_new=6):
    g = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, n_adapters + 1)
    p /= p.sum()
    trace, rid = [], 0
    for _ in range(n_steps):
        arr = []
        for _ in range(g.poisson(rate)):
            a = -1 if g.random() < null_frac else int(g.choice(n_adapters, p=p))
            arr.append((rid, a, int(g.integers(1, max_prompt + 1)), int(g.integers(1, max_new + 1))))
            rid += 1
        trace.append(arr)
    return trace


def ranks_of(n, seed=7):
    g = np.random.default_rng(seed)
    return {a: int(g.choice([2, 4, 8, 16])) for a in range(n)}


SETTINGS = {
    "caps": dict(num_pages=PAGES_PER_RANK * 64, max_slots=8, host_units=48, max_step_tokens=48, max_distinct=4,
                 max_running=16, window=8),
    "aging": dict(num_pages=PAGES_PER_RANK * 48, max_slots=6, host_units=40, max_step_tokens=32, max_distinct=3,
                  max_running=12, window=4, max_wait=3),
    "kv": dict(num_pages=PAGES_PER_RANK * 40 + 300, max_slots=8, host_units=64, max_step_tokens=40, max_distinct=6,
               max_running=10, window=6, max_wait=5, kvpt=4),
    "narrow": dict(num_pages=PAGES_PER_RANK * 20, max_slots=3, host_units=20, max_step_tokens=24, max_distinct=1,
                   max_running=4, window=1, max_wait=2),
    "tiny_host": dict(num_pages=PAGES_PER_RANK * 80, max_slots=16, host_units=16, max_step_tokens=64,
                      max_distinct=16, max_running=32, window=16),
}


def run_trace(setting, seed, n_steps=60, max_drain=3000):
    ranks = ranks_of(40, seed)
    pool, eng, store, model = make(ranks, **SETTINGS[setting])
    trace = zipf_trace(seed, n_steps)
    for t in range(n_steps + max_drain):
        for rid, a, pr, mn in (trace[t] if t < n_steps else []):
            eng.submit(rid, a, pr, mn)
            model.submit(rid, a, pr, mn)
        step_both(pool, eng, model)
        done_both(eng, model)
        if t >= n_steps and not model.waiting and not model.running:
            break
    st = eng.stats()
    assert st["finished"] == sum(len(x) for x in trace), "every request finishes once arrivals stop"
    assert len(store.loads) == st["host_misses"]
    return eng, model, st


# -- the library's engine against the model ---------------------------------------------------------

@pytest.mark.parametrize("setting", sorted(SETTINGS))
@pytest.mark.parametrize("seed", [0, 1])
def test_engine_matches_model_on_zipf_traces(setting, seed):
    eng, model, st = run_trace(setting, seed)
    assert st["page_ins"] > 0 and st["admitted"] > 0


def test_trace_settings_exercise_every_path():
    """The traces above reach evictions, host drops, room stalls, KV stalls and aged requests."""
    seen = {}
    for setting in SETTINGS:
        for seed in (0, 1):
            _, model, st = run_trace(setting, seed)
            for k in ("gpu_evictions", "host_evictions", "room_stalls", "kv_stalls"):
                seen[k] = seen.get(k, 0) + st[k]
    assert all(v > 0 for v in seen.values()), seen


# -- the model against what the pages fix ----------------------------------------------------------------

def model_only(ranks, **kw):
    s = dict(num_pages=PAGES_PER_RANK * 64, max_slots=8, host_units=48, max_step_tokens=48, max_distinct=4,
             max_running=16, window=8, max_wait=0, kvpt=0, max_segments=16)
    s.update(kw)
    pm = PoolModel(s["num_pages"], P, None, N_LAYERS, D_IN, D_OUT, s["max_slots"], MAX_RANK)
    return EngineModel(pm, ELEM, s["host_units"] * UNIT, s["max_step_tokens"], s["max_distinct"], s["max_running"],
                       s["window"], s["max_wait"], s["kvpt"], s["max_segments"], Storage(ranks).info)


@pytest.mark.parametrize("setting", sorted(SETTINGS))
def test_model_invariants_on_traces(setting):
    """Never evict an adapter a running request uses; every adapter of the step resident; caps
    per step; every request admitted exactly once."""
    kw = dict(SETTINGS[setting])
    m = model_only(ranks_of(40, 3), **{k: v for k, v in kw.items()})
    trace = zipf_trace(3, 80)
    admitted = set()
    for t in range(3000):
        if t >= 80 and not m.waiting and not m.running:
            break
        for rid, a, pr, mn in (trace[t] if t < 80 else []):
            m.submit(rid, a, pr, mn)
        n_ev = len(m.evicted)
        pre, dec = m.step()
        in_use = {m.req[q]["adapter"] for q in pre + dec if m.req[q]["adapter"] >= 0}
        running = {m.req[q]["adapter"] for q in dec if m.req[q]["adapter"] >= 0}
        assert not running & set(m.evicted[n_ev:]), "evicted the adapter of a running request"
        for a in in_use:
            assert a in m.pool.adapter_slot
        assert sum(m.req[q]["prompt"] for q in pre) + len(dec) <= kw["max_step_tokens"]
        assert len(in_use) <= kw["max_distinct"]
        assert len(pre) + len(dec) <= kw["max_running"] and len(pre) <= 16
        assert not admitted & set(pre)
        admitted |= set(pre)
        m.step_done()
    assert admitted == {r[0] for arr in trace for r in arr}


def test_model_lru_victim_by_hand():
    """Room for two rank-16 adapters.  a0 and a1 run and finish, a0 runs again, then a2 comes:
    the least recently used unused adapter is a1, which is evicted."""
    m = model_only({0: 16, 1: 16, 2: 16}, num_pages=PAGES_PER_RANK * 16 * 2, max_slots=4)
    for rid, a in ((0, 0), (1, 1), (2, 0), (3, 2)):
        m.submit(rid, a, 4, 1)
        pre, dec = m.step()
        assert pre == [rid] and dec == []
        m.step_done()
    assert m.evicted == [1]
    assert sorted(m.pool.adapter_slot) == [0, 2]


def test_model_never_evicts_running_by_hand():
    """Room for two rank-16 adapters.  a0 runs for a long time; a1 finishes; a2 evicts a1 (a0
    is older but in use); a3 then finds no candidate and waits until a2's request finishes."""
    m = model_only({0: 16, 1: 16, 2: 16, 3: 16}, num_pages=PAGES_PER_RANK * 16 * 2, max_slots=4, max_distinct=4)
    m.submit(0, 0, 4, 100)
    m.step()
    m.step_done()
    m.submit(1, 1, 4, 1)
    m.step()
    m.step_done()
    m.submit(2, 2, 4, 3)
    pre, _ = m.step()
    m.step_done()
    assert pre == [2] and m.evicted == [1]
    m.submit(3, 3, 4, 1)
    waited = 0
    while True:
        pre, dec = m.step()
        m.step_done()
        if 3 in pre:
            break
        waited += 1
        assert 0 in {q for q in dec} and 0 not in m.evicted
    assert m.evicted == [1, 2] and waited == 2 and m.c["room_stalls"] == 2


def test_model_host_lru_by_hand():
    """Host cache for two rank-8 adapters, GPU room for one: a0 a1 a0 a2 a1 loads a0, a1, a2
    (dropping a1, the least recently used), then a1 again (dropping a0)."""
    m = model_only({0: 8, 1: 8, 2: 8}, num_pages=PAGES_PER_RANK * 8, max_slots=2, host_units=16)
    for rid, a in enumerate((0, 1, 0, 2, 1)):
        m.submit(rid, a, 4, 1)
        assert m.step()[0] == [rid]
        m.step_done()
    assert (m.c["host_misses"], m.c["host_hits"], m.c["host_evictions"]) == (4, 1, 2)
    assert sorted(i for i, a in m.ad.items() if a["host_at"] >= 0) == [1, 2]


def test_model_look_ahead_pages_in_waiting_adapters():
    """The row cap keeps the second request out of step 1, yet its adapter comes in during
    step 1 (look-ahead window 2); in step 2 it joins with no page-in."""
    m = model_only({0: 4, 1: 4}, max_step_tokens=8, window=2)
    m.submit(0, 0, 8, 1)
    m.submit(1, 1, 8, 1)
    assert m.step() == ([0], [])
    assert 1 in m.pool.adapter_slot and m.c["page_ins"] == 2
    m.step_done()
    assert m.step() == ([1], [])
    assert m.c["page_ins"] == 2
    m.step_done()
    m1 = model_only({0: 4, 1: 4}, max_step_tokens=8, window=1)
    m1.submit(0, 0, 8, 1)
    m1.submit(1, 1, 8, 1)
    m1.step()
    assert 1 not in m1.pool.adapter_slot


def test_model_distinct_cap_and_fcfs():
    """With room everywhere, requests join in arrival order; the distinct-adapter cap holds back
    a request of a new adapter but lets later requests of the step's adapters join."""
    m = model_only({a: 2 for a in range(4)}, max_distinct=2)
    for rid, a in enumerate((0, 1, 2, 0, 1, 3)):
        m.submit(rid, a, 2, 1)
    pre, _ = m.step()
    assert pre == [0, 1, 3, 4]
    m.step_done()
    assert m.step()[0] == [2, 5]


def test_model_no_starvation_with_aging():
    """A 10-row prompt behind a stream of short requests (10 rows a step): without aging it
    never fits next to the running decode rows; with max_wait_steps 4 it joins within the
    bound (4 steps of waiting + 3 for the running requests to finish + 1)."""
    def run(max_wait):
        m = model_only({0: 2}, max_step_tokens=10, max_running=10, max_wait=max_wait, max_distinct=1)
        rid = 0
        for t in range(40):
            for _ in range(2):
                m.submit(rid, 0, 2, 3)
                rid += 1
            if t == 3:
                m.submit(1000, 0, 10, 1)
            pre, _ = m.step()
            m.step_done()
            if 1000 in pre:
                return m.step_no - 4
        return None
    assert run(0) is None
    joined = run(4)
    assert joined is not None and joined <= 4 + 3 + 1


def test_model_kv_pages_compete_with_adapters():
    """KV pages come from the same pool: a long request's KV evicts an unused adapter."""
    m = model_only({0: 16, 1: 16}, num_pages=PAGES_PER_RANK * 16 * 2 + 40, max_slots=4, kvpt=4)
    m.submit(0, 0, 4, 1)
    m.step()
    m.step_done()
    m.submit(1, 1, 4, 1)
    m.step()
    m.step_done()
    assert m.evicted == [] and len(m.pool.free) == 40
    m.submit(2, 1, 20, 10)     # 120 KV pages: a0 (unused, not wanted) goes
    pre, _ = m.step()
    assert pre == [2] and m.evicted == [0] and len(m.req[2]["kv"]) == 120


# -- the hand scenarios through the library -----------------------------------------------------------------

def test_engine_hand_scenarios_match_model():
    pool, eng, store, model = make({0: 16, 1: 16, 2: 16, 3: 16}, num_pages=PAGES_PER_RANK * 16 * 2, max_slots=4)
    for rid, a, mn in ((0, 0, 30), (1, 1, 1), (2, 2, 3), (3, 3, 1)):
        eng.submit(rid, a, 4, mn)
        model.submit(rid, a, 4, mn)
        step_both(pool, eng, model)
        done_both(eng, model)
    for _ in range(4):
        step_both(pool, eng, model)
        done_both(eng, model)
    assert model.evicted == [1, 2] and eng.stats()["room_stalls"] == 2
    assert eng.kv_pages(0).size == 0


# -- the library's own checks ------------------------------------------------------------------------------

def test_engine_errors():
    pool, eng, store, model = make({0: 4, 1: 4, 2: 99, 3: 4}, num_pages=PAGES_PER_RANK * 32)
    with pytest.raises(L.LoraError) as e:
        eng.submit(0, 0, 0, 1)                  # empty prompt
    assert e.value.code == L.LORA_EINVAL
    with pytest.raises(L.LoraError):
        eng.submit(0, 0, 49, 1)                 # prompt above max_step_tokens
    with pytest.raises(L.LoraError):
        eng.submit(0, 0, 4, 0)                  # nothing to generate
    with pytest.raises(L.LoraError):
        eng.submit(0, 2, 4, 1)                  # rank above the pool's max_rank
    with pytest.raises(L.LoraError):
        eng.submit(0, 7, 4, 1)                  # info fails (unknown adapter)
    eng.submit(0, 0, 4, 1)
    with pytest.raises(L.LoraError):
        eng.submit(0, 1, 4, 1)                  # request id in use
    store.fail.add(3)
    eng.submit(1, 3, 4, 1)
    with pytest.raises(L.LoraError) as e:
        eng.step()                              # storage load fails: no batch
    assert e.value.code == L.LORA_EINVAL and "storage" in str(e.value)
    eng.cancel(1)
    with pytest.raises(L.LoraError) as e:
        eng.cancel(1)
    assert e.value.code == L.LORA_ENOTRESIDENT
    b, plan = eng.step()
    assert list(b["requests"]) == [0] and plan is not None
    with pytest.raises(L.LoraError) as e:
        eng.step()                              # previous step not done
    assert e.value.code == L.LORA_EBUSY
    with pytest.raises(ValueError):
        L.lora_plan_destroy(plan)               # the engine owns it
    eng.step_done()
    eng.step_done()                             # no step: nothing to do
    b, plan = eng.step()
    assert b["n_requests"] == 0 and plan is None
    st = eng.stats()
    assert st["cancelled"] == 1 and st["finished"] == 1
    eng.reset_stats()
    assert eng.stats()["finished"] == 0


def test_engine_base_mismatch():
    pool, eng, store, model = make({0: 4}, num_pages=PAGES_PER_RANK * 8, base_id=5)
    store.base_id = 6
    with pytest.raises(L.LoraError) as e:
        eng.submit(0, 0, 4, 1)
    assert e.value.code == L.LORA_EBASE


@pytest.mark.parametrize("bad", [dict(max_step_tokens=0), dict(max_step_tokens=257), dict(max_distinct=0),
                                 dict(max_running=0), dict(max_running=49), dict(window=0), dict(max_wait=-1),
                                 dict(kvpt=-1), dict(host_units=15)])
def test_engine_create_checks(bad):
    with pytest.raises(L.LoraError) as e:
        make({0: 4}, num_pages=PAGES_PER_RANK * 8, **bad)
    assert e.value.code == L.LORA_EINVAL


def test_engine_kv_pages_and_adoption():
    """KV pages held by a running request come back when it finishes; an adapter paged in
    through the pool before its first request is adopted (a GPU hit, no load)."""
    pool, eng, store, model = make({0: 4, 1: 4}, num_pages=PAGES_PER_RANK * 16, kvpt=2)
    pool.page_in(1, 4, 8.0)
    free0 = len(pool.free_list())
    eng.submit(0, 1, 5, 2)
    b, plan = eng.step()
    assert list(b["requests"]) == [0]
    kv = eng.kv_pages(0)
    assert kv.size == (5 + 2) * 2 and len(pool.free_list()) == free0 - kv.size
    eng.step_done()
    eng.step()
    eng.step_done()
    assert len(pool.free_list()) == free0
    st = eng.stats()
    assert st["arrivals_resident"] == 1 and st["host_misses"] == 0 and store.loads == []
    with pytest.raises(L.LoraError):
        eng.kv_pages(0)


def test_pool_closed_before_engine():
    """Closing the pool first destroys its engine first; the engine's own close is then a no-op."""
    pool, eng, store, model = make({0: 4}, num_pages=PAGES_PER_RANK * 8)
    eng.submit(0, 0, 4, 3)
    eng.step()
    eng.step_done()
    pool.close()
    eng.close()
