"""Pins of the pool and index models (integer side of the oracle).

* The pages' printed size accounting ("Multi-LoRA serving: S-LoRA, Punica and
  adapter batching", worked example and "The bottleneck"), recomputed from
  the model's page geometry (tests/golden/pofe_worked_example.json).
* Invariants that hold whatever the allocation order: every page is owned by
  exactly one of {free list, one adapter, KV}; failed calls change nothing;
  evicting returns exactly the adapter's pages; tables list each page once.
* The index model: segment prefix sums and the decode grouping partition.
"""
import json
import os

import numpy as np
import pytest

from oracle import index_model
from oracle.pool_model import (EBASE, EBUSY, EEXIST, EINVAL, ENOPAGES, ENOSLOT, ENOTRESIDENT, PoolError,
                               PoolModel)
from workloads import make_workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_worked_example_size_accounting():
    with open(os.path.join(GOLDEN, "pofe_worked_example.json")) as f:
        g = json.load(f)
    s, pr = g["shape"], g["printed"]
    # 1024-element pages divide every width of this shape, so pages x page size = exact elements
    m = PoolModel(10 ** 6, 1024, None, s["n_layers"], s["d_in"], s["d_out"], max_slots=1, max_rank=64)
    per_layer = m.pages_per_rank() // s["n_layers"] * 1024
    assert per_layer == pr["per_layer_sum_din_plus_dout"]
    params_per_rank = m.pages_per_rank() * 1024
    assert round(params_per_rank / 1e6, 2) == pr["params_per_rank_millions"]
    r = pr["rank"]
    params = params_per_rank * r
    assert round(params / 1e6, 1) == pr["params_rank16_millions"]
    nbytes = 2 * params
    assert round(nbytes / 1e6, 1) == pr["bytes_rank16_MB_bf16"]
    assert round(1000 * nbytes / 1e9) == pr["adapters_1000_GB"]
    assert round(64 * nbytes / 1e9, 1) == pr["slots_64_GB"]
    assert round(nbytes / (pr["pcie_GBps"] * 1e9) * 1e3, 1) == pr["copy_ms_rank16"]
    assert round(4 * nbytes / (pr["pcie_GBps"] * 1e9) * 1e3, 1) == pr["copy_ms_rank64"]
    assert round(nbytes / (pr["hbm_TBps"] * 1e12) * 1e6) == pr["per_adapter_decode_us"]
    assert round(44 * nbytes / (pr["hbm_TBps"] * 1e12) * 1e3, 1) == pr["distinct_44_added_ms"]
    # one 4096 x 4096 projection, rank 16: adapter elements / base elements = 0.78 %
    m1 = PoolModel(10 ** 4, 4096, None, 1, [4096], [4096], max_slots=1, max_rank=64)
    ratio = 16 * m1.pages_per_rank() * 4096 / (4096 * 4096)
    assert round(100 * ratio, 2) == pr["extra_bytes_ratio_4096sq_r16_percent"]


def _owners(m: PoolModel):
    owner = {}
    for p in m.free:
        assert p not in owner
        owner[p] = "free"
    for s, pages in m.slot_pages.items():
        for p in pages:
            assert p not in owner, f"page {p} owned twice"
            owner[p] = ("slot", s)
    for p in m.kv_pages:
        assert p not in owner
        owner[p] = "kv"
    assert sorted(owner) == list(range(m.num_pages))
    return owner


def _snapshot(m: PoolModel):
    return (list(m.free), dict(m.slot_adapter), {k: list(v) for k, v in m.slot_pages.items()},
            set(m.kv_pages), dict(m.refcount))


def test_pool_partition_and_all_or_nothing():
    rng = np.random.default_rng(0)
    m = PoolModel(200, 256, rng.permutation(200), 2, [256, 512], [768, 256], max_slots=3, max_rank=8, base_id=7)
    # per rank-row: 2 layers x ((1 + 3) + (2 + 1)) = 14 pages
    assert m.pages_per_rank() == 14
    s0 = m.page_in(100, 4, 8.0)
    assert s0 == 0 and len(m.slot_pages[0]) == 56
    kv = m.alloc_kv(30)
    s1 = m.page_in(101, 8, 1.0)          # 112 pages, 2 left
    assert s1 == 1
    _owners(m)
    before = _snapshot(m)
    for call, code in [(lambda: m.page_in(102, 1, 1.0), ENOPAGES), (lambda: m.alloc_kv(3), ENOPAGES),
                       (lambda: m.page_in(100, 1, 1.0), EEXIST), (lambda: m.page_in(103, 1, 1.0, base_id=8), EBASE),
                       (lambda: m.page_in(104, 9, 1.0), EINVAL), (lambda: m.page_in(104, 0, 1.0), EINVAL),
                       (lambda: m.page_in(-1, 1, 1.0), EINVAL), (lambda: m.free_kv([kv[0], kv[0]]), EINVAL),
                       (lambda: m.free_kv([m.slot_pages[0][0]]), EINVAL), (lambda: m.evict(555), ENOTRESIDENT)]:
        with pytest.raises(PoolError) as e:
            call()
        assert e.value.code == code
        assert _snapshot(m) == before, "a failed call must leave the pool unchanged"
    # in-use adapters are not evicted
    m.acquire(s0)
    with pytest.raises(PoolError) as e:
        m.evict(100)
    assert e.value.code == EBUSY
    m.release(s0)
    pages0 = list(m.slot_pages[0])
    tail_before = list(m.free)
    m.evict(100)
    assert list(m.free) == tail_before + pages0, "evicted pages go to the tail in list order"
    _owners(m)
    # the freed slot is reused first
    assert m.page_in(105, 2, 4.0) == 0
    m.free_kv(kv)
    _owners(m)
    # slots run out
    m2 = PoolModel(100, 256, None, 1, [256], [256], max_slots=1, max_rank=4)
    m2.page_in(1, 1, 1.0)
    with pytest.raises(PoolError) as e:
        m2.page_in(2, 1, 1.0)
    assert e.value.code == ENOSLOT


def test_page_table_geometry_and_contents():
    m = PoolModel(64, 4, np.arange(64)[::-1], 1, [6], [10], max_slots=2, max_rank=4)
    s = m.page_in(3, 2, 4.0)
    a, b = m.page_table(s, 0, 0)
    assert a.shape == (2, 2) and b.shape == (2, 3)                 # ceil(6/4) = 2, ceil(10/4) = 3
    flat = list(a.reshape(-1)) + list(b.reshape(-1))
    assert flat == list(range(63, 63 - 10, -1)), "pages taken from the front of the free list, A then B"
    A = np.arange(12, dtype=np.float32).reshape(2, 6) + 1
    B = np.arange(20, dtype=np.float32).reshape(2, 10) + 100
    pages = m.expected_pages(s, 0, 0, A, B)
    assert len(pages) == 10
    assert np.array_equal(pages[int(a[1, 1])], np.array([11, 12, 0, 0], np.float32))      # zero tail
    assert np.array_equal(pages[int(b[0, 2])], np.array([108, 109, 0, 0], np.float32))
    # reassembling the chunks gives the rows back
    for mat, tab in ((A, a), (B, b)):
        for j in range(2):
            row = np.concatenate([pages[int(p)] for p in tab[j]])[: mat.shape[1]]
            assert np.array_equal(row, mat[j])


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_workload_op_logs_replay(name):
    wl = make_workload(name)
    m = PoolModel(wl.num_pages, wl.page_elems, wl.free_order, wl.n_layers, wl.d_in, wl.d_out,
                  wl.max_slots, wl.max_rank)
    ranks = {a: s.rank for a, s in wl.adapters.items()}
    alphas = {a: s.alpha for a, s in wl.adapters.items()}
    m.replay(wl.setup_ops, ranks, alphas)
    owner = _owners(m)
    used = sum(1 for o in owner.values() if o != "free")
    assert used <= wl.num_pages and len(m.free) == wl.num_pages - used
    if name == "c3":
        # 11008-wide B rows take 3 pages: r * (1 + 3) pages per adapter
        for a, spec in list(wl.adapters.items())[:20]:
            assert len(m.slot_pages[m.slot_of(a)]) == 4 * spec.rank


def test_index_model():
    slot_of = {5: 2, 9: 0}.__getitem__
    st, ss = index_model.segments([3, 0, 4], [5, -1, 9], slot_of)
    assert list(st) == [0, 3, 3, 7] and list(ss) == [2, -1, 0]
    assert np.array_equal(np.diff(st), [3, 0, 4])
    ts = index_model.token_slots([9, -1, 5, 9, 5], slot_of)
    assert list(ts) == [0, -1, 2, 0, 2]
    g = index_model.decode_groups(ts, row_offset=10)
    assert g == {0: [10, 13], 2: [12, 14]}
    assert sorted(r for rows in g.values() for r in rows) == [10 + t for t in range(5) if ts[t] >= 0]
