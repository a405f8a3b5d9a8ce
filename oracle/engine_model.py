"""Reference model of the engine layer's decisions (integer side).  Test
infrastructure: only tests import it.

What it follows:
  * "S-LoRA: Serving Thousands of Concurrent LoRA Adapters" (Host memory for
    adapters): every adapter has a home in host memory; the GPU holds the ones
    the running batch uses; the next batch's adapters are predicted from the
    waiting queue and brought in during the current step.
  * "Multi-LoRA serving: S-LoRA, Punica and adapter batching" (What the engine
    does each step): a missing adapter comes from the host cache, or from
    storage into it first; room on the GPU comes from evicting the least
    recently used adapter no request is using; a request is ready once its
    adapter's copy is done; a step picks requests under a row cap and a cap on
    distinct adapters; finished requests let go of their adapter and KV pages.
    Its paragraph after the step adds fairness: one hot adapter must not starve
    the tail.

Readings where the pages leave the policy open:
  * requests have a prompt (one prefill segment in the step that admits them)
    and a number of tokens to generate (one decode row per later step);
  * page-ins start at the step after arrival, for the adapters of the first
    `prefetch_window` waiting requests, in scheduling order; an adapter that
    finds no room stops the page-ins behind it;
  * scheduling order: requests that have waited `max_wait_steps` steps or more
    first, then the rest, each in arrival order; admission skips a request
    that does not fit, except that an aged request that cannot get room stops
    the admissions behind it;
  * eviction candidates are resident adapters with no running request; room
    for the request at queue position i may not evict the adapters of the
    requests ahead of it (so the head of the queue is always served once
    running requests let go); among candidates, those the look-ahead window
    does not want go first, each group least recently used first (ties: the
    smaller adapter id); "used" means admitted, given a decode row or paged
    in, counted in steps;
  * the host cache is an arena of units (one rank-row of A and B over every
    layer and projection, 256-byte aligned); an adapter takes consecutive
    units, first fit; the least recently used entry (ties: smaller id) that no
    copy still reads is dropped until the adapter fits;
  * KV pages (when the engine manages them) are taken whole at admission for
    prompt + generated tokens, evicting candidates if needed.

The model runs on a host-only pool (oracle.pool_model.PoolModel), where a copy
is done as soon as it is issued.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Tuple

from .pool_model import EBUSY, ENOPAGES, PoolError, PoolModel


def _align(x: int, a: int) -> int:
    return -(-x // a) * a


class EngineModel:
    def __init__(self, pool: PoolModel, elem_bytes: int, host_cache_bytes: int, max_step_tokens: int,
                 max_distinct_adapters: int, max_running: int, prefetch_window: int, max_wait_steps: int,
                 kv_pages_per_token: int, max_segments: int, info: Callable[[int], Tuple[int, float, int]]):
        self.pool = pool
        self.max_step_tokens = max_step_tokens
        self.max_distinct = max_distinct_adapters
        self.max_running = max_running
        self.window = prefetch_window
        self.max_wait = max_wait_steps
        self.kvpt = kv_pages_per_token
        self.max_segments = max_segments
        self.info = info
        self.a_row = sum(pool.n_layers * d for d in pool.d_in) * elem_bytes
        self.b_row = sum(pool.n_layers * d for d in pool.d_out) * elem_bytes
        self.unit = _align(self.a_row + self.b_row, 256)
        self.free_runs: List[List[int]] = [[0, host_cache_bytes // self.unit]]   # [start, length], by start
        self.ad: Dict[int, dict] = {}
        self.req: Dict[int, dict] = {}
        self.waiting: List[int] = []
        self.running: List[int] = []
        self.step_no = 0
        self.step_prefill: List[int] = []
        self.step_decode: List[int] = []
        self.c = {k: 0 for k in ("steps", "rows", "admitted", "finished", "arrivals_resident", "arrivals_missing",
                                 "host_hits", "host_misses", "page_ins", "gpu_evictions", "host_evictions",
                                 "room_stalls", "kv_stalls", "cancelled")}
        self.evicted: List[int] = []       # adapters evicted from the GPU, in order
        self.wait_steps: List[int] = []

    # -- host cache ----------------------------------------------------------------------------
    def entry_units(self, rank: int) -> int:
        return -(-(_align(rank * self.a_row, 256) + rank * self.b_row) // self.unit)

    def _take(self, n: int) -> int:
        for i, (start, length) in enumerate(self.free_runs):
            if length >= n:
                if length == n:
                    del self.free_runs[i]
                else:
                    self.free_runs[i] = [start + n, length - n]
                return start
        return -1

    def _give(self, start: int, n: int) -> None:
        self.free_runs.append([start, n])
        self.free_runs.sort()
        merged: List[List[int]] = []
        for s, l in self.free_runs:
            if merged and merged[-1][0] + merged[-1][1] == s:
                merged[-1][1] += l
            else:
                merged.append([s, l])
        self.free_runs = merged

    def _host_drop_one(self, reading: set) -> bool:
        cached = [(a["host_last_use"], i) for i, a in self.ad.items() if a["host_at"] >= 0 and i not in reading]
        if not cached:
            return False
        _, victim = min(cached)
        a = self.ad[victim]
        self._give(a["host_at"], self.entry_units(a["rank"]))
        a["host_at"] = -1
        self.c["host_evictions"] += 1
        return True

    # -- GPU tier --------------------------------------------------------------------------------
    def _evict_one(self, protect: set, skip: set, wanted: set) -> bool:
        """Evict the least recently used unused adapter the window does not want, else the least
        recently used unused one it wants (never one in `protect`)."""
        while True:
            cands = [(i in wanted, a["last_use"], i) for i, a in self.ad.items()
                     if a["resident"] and a["users"] == 0 and i not in protect and i not in skip]
            if not cands:
                return False
            victim = min(cands)[2]
            try:
                self.pool.evict(victim)
            except PoolError as e:
                if e.code != EBUSY:
                    raise
                skip.add(victim)
                continue
            self.ad[victim]["resident"] = False
            self.c["gpu_evictions"] += 1
            self.evicted.append(victim)
            return True

    # -- requests ----------------------------------------------------------------------------------
    def submit(self, rid: int, adapter: int, prompt: int, max_new: int) -> None:
        resident = False
        if adapter >= 0:
            if adapter not in self.ad:
                rank, alpha, _base = self.info(adapter)
                self.ad[adapter] = dict(rank=rank, alpha=alpha, resident=adapter in self.pool.adapter_slot,
                                        users=0, last_use=-1, host_at=-1, host_last_use=-1)
            resident = self.ad[adapter]["resident"]
            self.c["arrivals_resident" if resident else "arrivals_missing"] += 1
        self.req[rid] = dict(adapter=adapter, prompt=prompt, max_new=max_new, generated=0,
                             submit_step=self.step_no, slot=-1, kv=[])
        self.waiting.append(rid)

    def cancel(self, rid: int) -> None:
        self.waiting.remove(rid)
        del self.req[rid]
        self.c["cancelled"] += 1

    def _aged(self, r: dict) -> bool:
        return self.max_wait > 0 and self.step_no - r["submit_step"] >= self.max_wait

    def step(self):
        """-> (prefill request ids, decode request ids) of the step, in row order."""
        self.step_no += 1
        self.c["steps"] += 1
        order = [q for q in self.waiting if self._aged(self.req[q])] + \
                [q for q in self.waiting if not self._aged(self.req[q])]
        window = order[:self.window]
        wanted = {self.req[q]["adapter"] for q in window if self.req[q]["adapter"] >= 0}

        # page-ins for the window, in window order; the adapter of the request at position i
        # may evict any candidate but the adapters of the requests ahead of it
        batch: List[int] = []
        skip: set = set()
        claim_pages = 0
        for i, q in enumerate(window):
            a = self.req[q]["adapter"]
            if a < 0 or self.ad[a]["resident"] or a in batch:
                continue
            ahead = {self.req[w]["adapter"] for w in window[:i]}
            st = self.ad[a]
            need = st["rank"] * self.pool.pages_per_rank()
            room = True
            while (len(self.pool.adapter_slot) + len(batch) + 1 > self.pool.max_slots
                   or len(self.pool.free) - claim_pages < need):
                if not self._evict_one(ahead, skip, wanted):
                    room = False
                    break
            if not room:
                self.c["room_stalls"] += 1
                break
            st["host_last_use"] = self.step_no
            if st["host_at"] >= 0:
                self.c["host_hits"] += 1
            else:
                n = self.entry_units(st["rank"])
                at = self._take(n)
                while at < 0 and self._host_drop_one(set(batch) | {a}):
                    at = self._take(n)
                if at < 0:
                    self.c["room_stalls"] += 1
                    break
                st["host_at"] = at
                self.c["host_misses"] += 1
            batch.append(a)
            claim_pages += need
        for a in batch:
            self.pool.page_in(a, self.ad[a]["rank"], self.ad[a]["alpha"])
            self.ad[a]["resident"] = True
            self.ad[a]["last_use"] = self.step_no
            self.c["page_ins"] += 1

        # admission
        distinct = {self.req[q]["adapter"] for q in self.running if self.req[q]["adapter"] >= 0}
        rows_left = self.max_step_tokens - len(self.running)
        n_running = len(self.running)
        admitted: List[int] = []
        for i, q in enumerate(order):
            r = self.req[q]
            aged = self._aged(r)
            a = r["adapter"]
            if a >= 0 and not self.ad[a]["resident"]:
                if aged:
                    break
                continue
            fits = (r["prompt"] <= rows_left and n_running + 1 <= self.max_running
                    and len(admitted) + 1 <= self.max_segments
                    and (a < 0 or a in distinct or len(distinct) + 1 <= self.max_distinct))
            if not fits:
                if aged:
                    break
                continue
            if self.kvpt > 0:
                need = (r["prompt"] + r["max_new"]) * self.kvpt
                keep = {self.req[w]["adapter"] for w in order[:i]} | distinct | {a}
                got = None
                while got is None:
                    try:
                        got = self.pool.alloc_kv(need)
                    except PoolError as e:
                        if e.code != ENOPAGES:
                            raise
                        if not self._evict_one(keep, skip, wanted):
                            break
                if got is None:
                    self.c["kv_stalls"] += 1
                    if aged:
                        break
                    continue
                r["kv"] = got
            if a >= 0:
                slot = self.pool.slot_of(a)
                self.pool.acquire(slot)
                r["slot"] = slot
                self.ad[a]["users"] += 1
                self.ad[a]["last_use"] = self.step_no
                distinct.add(a)
            rows_left -= r["prompt"]
            n_running += 1
            admitted.append(q)
        for q in admitted:
            self.waiting.remove(q)
            self.wait_steps.append(self.step_no - self.req[q]["submit_step"])
        for q in self.running:
            if self.req[q]["adapter"] >= 0:
                self.ad[self.req[q]["adapter"]]["last_use"] = self.step_no
        self.step_prefill = admitted
        self.step_decode = list(self.running)
        self.c["admitted"] += len(admitted)
        self.c["rows"] += sum(self.req[q]["prompt"] for q in admitted) + len(self.running)
        return list(self.step_prefill), list(self.step_decode)

    def step_done(self) -> None:
        for q in self.step_decode:
            self.req[q]["generated"] += 1
        for q in self.step_prefill:
            self.req[q]["generated"] = 1
            self.running.append(q)
        still = []
        for q in self.running:
            r = self.req[q]
            if r["generated"] < r["max_new"]:
                still.append(q)
                continue
            if r["adapter"] >= 0:
                self.pool.release(r["slot"])
                self.ad[r["adapter"]]["users"] -= 1
            if r["kv"]:
                self.pool.free_kv(r["kv"])
            del self.req[q]
            self.c["finished"] += 1
        self.running = still
        self.step_prefill, self.step_decode = [], []
