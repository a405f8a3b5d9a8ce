"""Host logic of the C library against the oracle's pool and index models,
bit for bit, using host-only pools (no GPU): page tables and free lists
after each workload's op log, every error path, all-or-nothing behaviour,
and the plan's decode grouping."""
import numpy as np
import pytest

from heterogeneous_adapter_gemm_amd import _lib as L
from heterogeneous_adapter_gemm_amd.runtime import DevicePool
from oracle import index_model
from oracle.pool_model import PoolError, PoolModel
from workloads import make_workload

DT = {"f32": L.LORA_F32, "bf16": L.LORA_BF16}


def host_pool(wl, max_tokens=None, max_segments=16, base_id=0):
    return DevicePool(DT[wl.dtype], wl.page_elems, wl.num_pages, wl.free_order, wl.n_layers, wl.d_in, wl.d_out,
                      wl.max_slots, wl.max_rank, max_tokens or max(wl.T, 1), max_segments, base_id=base_id,
                      device=None)


def model_of(wl, base_id=0):
    return PoolModel(wl.num_pages, wl.page_elems, wl.free_order, wl.n_layers, wl.d_in, wl.d_out, wl.max_slots,
                     wl.max_rank, base_id=base_id)


def replay_both(wl, pool, model, ops):
    kv_lib, kv_model = [], []
    for op in ops:
        if op[0] == "page_in":
            a = wl.adapters[op[1]]
            s1 = pool.page_in(a.adapter_id, a.rank, a.alpha)
            s2 = model.page_in(a.adapter_id, a.rank, a.alpha)
            assert s1 == s2
        elif op[0] == "alloc_kv":
            kv_lib.append(pool.alloc_kv(op[1]))
            kv_model.append(model.alloc_kv(op[1]))
            assert list(kv_lib[-1]) == kv_model[-1]
        elif op[0] == "evict":
            pool.evict(op[1])
            model.evict(op[1])
        elif op[0] == "free_kv":
            pool.free_kv(kv_lib[op[1]])
            model.free_kv(kv_model[op[1]])
    return kv_lib


def assert_same_tables(wl, pool, model):
    assert list(pool.free_list()) == model.free_list()
    for aid, slot in model.adapter_slot.items():
        assert pool.slot_of(aid) == slot
        for l in range(wl.n_layers):
            for p in range(wl.n_proj):
                a1, b1 = pool.page_table(slot, l, p)
                a2, b2 = model.page_table(slot, l, p)
                assert np.array_equal(a1, a2) and np.array_equal(b1, b2)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_op_log_tables_bit_exact(name):
    wl = make_workload(name)
    pool, model = host_pool(wl), model_of(wl)
    replay_both(wl, pool, model, wl.setup_ops)
    assert_same_tables(wl, pool, model)
    free, resident, kv = pool.stats()
    assert free == len(model.free) and resident == len(model.slot_adapter) and kv == len(model.kv_pages)


def test_c5_reduced_layers_step_ops():
    wl = make_workload("c5", n_layers=2)
    pool, model = host_pool(wl), model_of(wl)
    replay_both(wl, pool, model, wl.setup_ops + wl.step_ops)
    assert_same_tables(wl, pool, model)
    # end of step: evict the cold adapters again, in reverse order
    for a in reversed(wl.cold_adapters):
        pool.evict(a)
        model.evict(a)
    assert_same_tables(wl, pool, model)


def test_error_paths_match_model_and_leave_pool_unchanged():
    rng = np.random.default_rng(3)
    kw = dict(dtype=L.LORA_F32, page_elems=256, num_pages=200, free_order=rng.permutation(200), n_layers=2,
              d_in=[256, 512], d_out=[768, 256], max_slots=3, max_rank=8)
    pool = DevicePool(kw["dtype"], kw["page_elems"], kw["num_pages"], kw["free_order"], kw["n_layers"], kw["d_in"],
                      kw["d_out"], kw["max_slots"], kw["max_rank"], max_tokens=64, max_segments=4, base_id=7,
                      device=None)
    model = PoolModel(200, 256, kw["free_order"], 2, kw["d_in"], kw["d_out"], 3, 8, base_id=7)
    assert pool.page_in(100, 4, 8.0) == model.page_in(100, 4, 8.0)
    kvl, kvm = pool.alloc_kv(30), model.alloc_kv(30)
    assert list(kvl) == kvm
    assert pool.page_in(101, 8, 1.0) == model.page_in(101, 8, 1.0)

    def same_error(call_lib, call_model):
        with pytest.raises(L.LoraError) as e1:
            call_lib()
        with pytest.raises(PoolError) as e2:
            call_model()
        assert e1.value.code == e2.value.code
        assert list(pool.free_list()) == model.free_list()

    same_error(lambda: pool.page_in(102, 1, 1.0), lambda: model.page_in(102, 1, 1.0))            # ENOPAGES
    same_error(lambda: pool.alloc_kv(3), lambda: model.alloc_kv(3))                                # ENOPAGES
    same_error(lambda: pool.page_in(100, 1, 1.0), lambda: model.page_in(100, 1, 1.0))            # EEXIST
    same_error(lambda: pool.page_in(103, 1, 1.0, base_id=8), lambda: model.page_in(103, 1, 1.0, base_id=8))  # EBASE
    same_error(lambda: pool.page_in(104, 9, 1.0), lambda: model.page_in(104, 9, 1.0))            # EINVAL rank
    same_error(lambda: pool.page_in(104, 0, 1.0), lambda: model.page_in(104, 0, 1.0))
    same_error(lambda: pool.page_in(-1, 1, 1.0), lambda: model.page_in(-1, 1, 1.0))
    same_error(lambda: pool.page_in(104, 1, float("nan")), lambda: model.page_in(104, 1, float("nan")))
    same_error(lambda: pool.free_kv([kvl[0], kvl[0]]), lambda: model.free_kv([kvm[0], kvm[0]]))  # EINVAL dup
    same_error(lambda: pool.free_kv([pool.page_table(0, 0, 0)[0][0, 0]]),
               lambda: model.free_kv([model.page_table(0, 0, 0)[0][0, 0]]))                       # not KV
    same_error(lambda: pool.evict(555), lambda: model.evict(555))                                 # ENOTRESIDENT
    # in use: a plan holds a reference
    plan = pool.plan(token_slot=[0, -1, 0])
    with pytest.raises(L.LoraError) as e:
        pool.evict(100)
    assert e.value.code == L.LORA_EBUSY
    L.lora_plan_destroy(plan)
    L.lora_pool_acquire(pool.pool, 0)
    with pytest.raises(L.LoraError) as e:
        pool.evict(100)
    assert e.value.code == L.LORA_EBUSY
    L.lora_pool_release(pool.pool, 0)
    pool.evict(100)
    model.evict(100)
    assert list(pool.free_list()) == model.free_list()
    # slots run out
    assert pool.page_in(105, 1, 1.0) == model.page_in(105, 1, 1.0)
    pool.evict(101), model.evict(101)
    pool.page_in(106, 1, 1.0), model.page_in(106, 1, 1.0)
    pool.page_in(107, 1, 1.0), model.page_in(107, 1, 1.0)
    same_error(lambda: pool.page_in(108, 1, 1.0), lambda: model.page_in(108, 1, 1.0))            # ENOSLOT


def test_plan_validation():
    wl = make_workload("c1")
    pool = host_pool(wl, max_tokens=16, max_segments=4)
    for op in wl.setup_ops:
        a = wl.adapters[op[1]]
        pool.page_in(a.adapter_id, a.rank, a.alpha)
    bad = [dict(seg_start=[1, 3], seg_slot=[0]), dict(seg_start=[0, 3, 2], seg_slot=[0, 1]),
           dict(seg_start=[0, 17], seg_slot=[0]), dict(token_slot=[0, 9]), dict(token_slot=[-2]),
           dict(seg_start=[0, 1, 2, 3, 4, 5], seg_slot=[0, 0, 0, 0, 0]), dict(token_slot=[0] * 17)]
    for kw in bad:
        with pytest.raises(L.LoraError) as e:
            pool.plan(**kw)
        assert e.value.code == L.LORA_EINVAL, kw
    pool.evict(3)
    with pytest.raises(L.LoraError) as e:
        pool.plan(token_slot=[3])
    assert e.value.code == L.LORA_ENOTRESIDENT
    # empty batches are fine
    L.lora_plan_destroy(pool.plan())
    L.lora_plan_destroy(pool.plan(seg_start=[0, 0], seg_slot=[1]))


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_plan_grouping_matches_index_model(name):
    wl = make_workload(name)
    pool, model = host_pool(wl), model_of(wl)
    replay_both(wl, pool, model, wl.setup_ops)
    ra = wl.row_adapter()
    ts_lib = pool.slots_of(ra)
    ts_model = index_model.token_slots(ra, model.slot_of)
    assert np.array_equal(ts_lib, ts_model)
    plan = pool.plan(token_slot=ts_lib)
    gs, gb, gc, rows = L.lora_plan_groups(plan, len(ra))
    got = {int(s): list(rows[b:b + c]) for s, b, c in zip(gs, gb, gc)}
    assert got == index_model.decode_groups(ts_model)
    # every non-null row appears exactly once
    assert sorted(int(r) for r in rows[: int(gc.sum())]) == [t for t in range(len(ra)) if ts_model[t] >= 0]
    L.lora_plan_destroy(plan)


def test_segments_from_requests_match_index_model():
    wl = make_workload("c4")
    pool, model = host_pool(wl), model_of(wl)
    replay_both(wl, pool, model, wl.setup_ops)
    lens = [r.n_tokens for r in wl.requests]
    ids = [r.adapter_id for r in wl.requests]
    st, ss = index_model.segments(lens, ids, model.slot_of)
    assert np.array_equal(pool.slots_of(ids), ss)
    assert st[-1] == wl.T
    plan = pool.plan(seg_start=st, seg_slot=ss)
    L.lora_plan_destroy(plan)


def test_batch_page_in_equals_calls_in_order():
    """A batch page-in takes the slots and pages that the same page-ins, one by
    one in request order, take in the oracle's pool model."""
    wl = make_workload("c5", n_layers=2)
    pool, model = host_pool(wl), model_of(wl)
    replay_both(wl, pool, model, wl.setup_ops)
    kv = [pool.alloc_kv(n) for n in (5, 17)]
    kvm = [model.alloc_kv(n) for n in (5, 17)]
    assert [list(k) for k in kv] == kvm
    items = [(a, wl.adapters[a].rank, wl.adapters[a].alpha, None, None) for a in wl.cold_adapters]
    slots = pool.page_in_batch(items)
    assert list(slots) == [model.page_in(a, r, al) for a, r, al, _, _ in items]
    assert_same_tables(wl, pool, model)
    pool.page_in_batch([])   # empty batch: nothing happens
    assert_same_tables(wl, pool, model)


def test_batch_page_in_errors_leave_pool_unchanged():
    rng = np.random.default_rng(4)
    order = rng.permutation(120)
    pool = DevicePool(L.LORA_F32, 256, 120, order, 2, [256, 512], [768, 256], 3, 8, max_tokens=16, max_segments=4,
                      base_id=7, device=None)
    model = PoolModel(120, 256, order, 2, [256, 512], [768, 256], 3, 8, base_id=7)
    # pages per rank-row: 2 layers x (1 + 3 + 2 + 1) = 14
    assert pool.page_in(10, 2, 4.0) == model.page_in(10, 2, 4.0)
    before = list(pool.free_list())

    def fails(items, code):
        with pytest.raises(L.LoraError) as e:
            pool.page_in_batch(items)
        assert e.value.code == code
        assert list(pool.free_list()) == before and pool.stats()[1] == 1

    fails([(11, 1, 1.0, None, None), (11, 2, 1.0, None, None)], L.LORA_EEXIST)     # same adapter twice
    fails([(11, 1, 1.0, None, None), (10, 2, 1.0, None, None)], L.LORA_EEXIST)     # already resident
    fails([(11, 4, 1.0, None, None), (12, 4, 1.0, None, None)], L.LORA_ENOPAGES)   # 56 + 56 > 92 free
    fails([(11, 1, 1.0, None, None), (12, 1, 1.0, None, None), (13, 1, 1.0, None, None)], L.LORA_ENOSLOT)
    fails([(11, 1, 1.0, None, None), (12, 9, 1.0, None, None)], L.LORA_EINVAL)     # rank above max_rank
    # a batch that fits
    got = pool.page_in_batch([(11, 4, 1.0, None, None), (12, 2, 1.0, None, None)])
    assert list(got) == [model.page_in(11, 4, 1.0), model.page_in(12, 2, 1.0)]
    assert list(pool.free_list()) == model.free_list()
