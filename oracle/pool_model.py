"""Reference model of the unified page pool (integer side).  Test infrastructure.

Follows "S-LoRA: Serving Thousands of Concurrent LoRA Adapters" (Unified
paging): one pool of fixed-size pages, each page one hidden-size vector,
holding both adapter weights (rank x hidden) and KV blocks (tokens x hidden),
so adapters of different ranks need no padding.  "Multi-LoRA serving:
S-LoRA, Punica and adapter batching" ("What the engine does each step")
adds that an adapter in use is never evicted; its "Failure modes" section
adds the check of the base-model identity at load.

Readings where the pages leave the allocation open:
  * the free list starts as the given physical page order and is popped from
    the front; freed pages are appended to its tail in list order;
  * a vector longer than a page takes ceil(len / page) pages of consecutive
    chunks, the last one zero-filled past the vector's end;
  * an adapter's pages are taken in the order layer, projection, A before B,
    rank-row j, chunk c; all of them at once or none;
  * a page-in takes the lowest free slot index;
  * argument checks run in the order: malformed -> base mismatch -> already
    resident -> no slot -> not enough pages; a failed call changes nothing.
"""
from __future__ import annotations

import math
from collections import deque
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

OK = 0
EINVAL = -1
ENOPAGES = -2
ENOTRESIDENT = -3
EBUSY = -4
EEXIST = -5
EBASE = -6
ENOSLOT = -8


class PoolError(Exception):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


class PoolModel:
    def __init__(self, num_pages: int, page_elems: int, free_order: Optional[Sequence[int]],
                 n_layers: int, d_in: Sequence[int], d_out: Sequence[int],
                 max_slots: int, max_rank: int, base_id: int = 0):
        self.num_pages = int(num_pages)
        self.page_elems = int(page_elems)
        order = range(self.num_pages) if free_order is None else [int(p) for p in free_order]
        if sorted(order) != list(range(self.num_pages)):
            raise PoolError(EINVAL, "free_order must be a permutation of the pages")
        self.free: deque = deque(order)
        self.n_layers = int(n_layers)
        self.d_in = [int(d) for d in d_in]
        self.d_out = [int(d) for d in d_out]
        self.max_slots = int(max_slots)
        self.max_rank = int(max_rank)
        self.base_id = int(base_id)
        self.slot_adapter: Dict[int, int] = {}
        self.adapter_slot: Dict[int, int] = {}
        self.slot_rank: Dict[int, int] = {}
        self.slot_alpha: Dict[int, float] = {}
        self.slot_pages: Dict[int, List[int]] = {}
        self.refcount: Dict[int, int] = {}
        self.kv_pages: set = set()

    # -- geometry -------------------------------------------------------------
    @property
    def n_proj(self) -> int:
        return len(self.d_in)

    def chunks(self, length: int) -> int:
        return -(-length // self.page_elems)

    def pages_per_rank(self) -> int:
        return self.n_layers * sum(self.chunks(i) + self.chunks(o) for i, o in zip(self.d_in, self.d_out))

    def _lp_offset(self, rank: int, layer: int, proj: int) -> int:
        """Index, within a slot's page list, of the first page of (layer, proj)."""
        per_layer = sum(self.chunks(i) + self.chunks(o) for i, o in zip(self.d_in, self.d_out))
        before = layer * per_layer + sum(self.chunks(self.d_in[p]) + self.chunks(self.d_out[p]) for p in range(proj))
        return rank * before

    # -- adapters ---------------------------------------------------------------
    def page_in(self, adapter_id: int, rank: int, alpha: float, base_id: Optional[int] = None) -> int:
        base_id = self.base_id if base_id is None else int(base_id)
        if adapter_id < 0 or not (1 <= rank <= self.max_rank) or not math.isfinite(alpha):
            raise PoolError(EINVAL, "malformed page-in")
        if base_id != self.base_id:
            raise PoolError(EBASE, "adapter trained on another base")
        if adapter_id in self.adapter_slot:
            raise PoolError(EEXIST, "adapter already resident")
        slot = next((s for s in range(self.max_slots) if s not in self.slot_adapter), None)
        if slot is None:
            raise PoolError(ENOSLOT, "no free slot")
        need = rank * self.pages_per_rank()
        if need > len(self.free):
            raise PoolError(ENOPAGES, "not enough free pages")
        pages = [self.free.popleft() for _ in range(need)]
        self.slot_adapter[slot] = adapter_id
        self.adapter_slot[adapter_id] = slot
        self.slot_rank[slot] = rank
        self.slot_alpha[slot] = float(alpha)
        self.slot_pages[slot] = pages
        self.refcount[slot] = 0
        return slot

    def slot_of(self, adapter_id: int) -> int:
        if adapter_id not in self.adapter_slot:
            raise PoolError(ENOTRESIDENT, "adapter not resident")
        return self.adapter_slot[adapter_id]

    def acquire(self, slot: int) -> None:
        if slot not in self.slot_adapter:
            raise PoolError(ENOTRESIDENT, "empty slot")
        self.refcount[slot] += 1

    def release(self, slot: int) -> None:
        if slot not in self.slot_adapter or self.refcount[slot] == 0:
            raise PoolError(EINVAL, "release without acquire")
        self.refcount[slot] -= 1

    def evict(self, adapter_id: int) -> None:
        slot = self.slot_of(adapter_id)
        if self.refcount[slot] > 0:
            raise PoolError(EBUSY, "adapter in use")
        self.free.extend(self.slot_pages[slot])
        for d in (self.slot_adapter, self.slot_rank, self.slot_alpha, self.slot_pages, self.refcount):
            del d[slot]
        del self.adapter_slot[adapter_id]

    # -- KV blocks --------------------------------------------------------------
    def alloc_kv(self, n: int) -> List[int]:
        if n < 0:
            raise PoolError(EINVAL, "negative count")
        if n > len(self.free):
            raise PoolError(ENOPAGES, "not enough free pages")
        pages = [self.free.popleft() for _ in range(n)]
        self.kv_pages.update(pages)
        return pages

    def free_kv(self, pages: Sequence[int]) -> None:
        pages = [int(p) for p in pages]
        if len(set(pages)) != len(pages) or any(p not in self.kv_pages for p in pages):
            raise PoolError(EINVAL, "not a KV page, or listed twice")
        self.kv_pages.difference_update(pages)
        self.free.extend(pages)

    # -- tables -------------------------------------------------------------------
    def page_table(self, slot: int, layer: int, proj: int) -> Tuple[np.ndarray, np.ndarray]:
        """Pages of (slot, layer, proj): A as [r][chunks(d_in)], B as [r][chunks(d_out)]."""
        if slot not in self.slot_adapter:
            raise PoolError(ENOTRESIDENT, "empty slot")
        r = self.slot_rank[slot]
        ci, co = self.chunks(self.d_in[proj]), self.chunks(self.d_out[proj])
        base = self._lp_offset(r, layer, proj)
        pages = self.slot_pages[slot]
        a = np.array(pages[base: base + r * ci], np.int32).reshape(r, ci)
        b = np.array(pages[base + r * ci: base + r * ci + r * co], np.int32).reshape(r, co)
        return a, b

    def free_list(self) -> List[int]:
        return list(self.free)

    def expected_pages(self, slot: int, layer: int, proj: int, A: np.ndarray, B: np.ndarray) -> Dict[int, np.ndarray]:
        """Expected content of every page of (slot, layer, proj) given the
        logical factors A [r, d_in] and B [r, d_out]: consecutive chunks of
        each rank-row, zero past the row's end."""
        a_pages, b_pages = self.page_table(slot, layer, proj)
        out: Dict[int, np.ndarray] = {}
        P = self.page_elems
        for mat, tab in ((A, a_pages), (B, b_pages)):
            for j in range(tab.shape[0]):
                for c in range(tab.shape[1]):
                    page = np.zeros(P, dtype=mat.dtype)
                    chunk = mat[j, c * P: (c + 1) * P]
                    page[: chunk.shape[0]] = chunk
                    out[int(tab[j, c])] = page
        return out

    # -- replay -------------------------------------------------------------------
    def replay(self, ops: Sequence[tuple], ranks: Dict[int, int], alphas: Dict[int, float]) -> List[List[int]]:
        """Run an op log; returns the page lists of the KV allocations in order."""
        kv: List[List[int]] = []
        for op in ops:
            kind = op[0]
            if kind == "page_in":
                self.page_in(op[1], ranks[op[1]], alphas[op[1]])
            elif kind == "evict":
                self.evict(op[1])
            elif kind == "alloc_kv":
                kv.append(self.alloc_kv(op[1]))
            elif kind == "free_kv":
                self.free_kv(kv[op[1]])
            else:
                raise ValueError(f"unknown op {kind}")
        return kv
