"""Seeded generator for the five LoRA-linear workloads.

Each workload follows one configuration of the multi-adapter LoRA-linear
layer that the S-LoRA / Punica pages describe: a frozen base weight W0
(stored [d_out, d_in], the layout of the base weight in the PyTorch demo of
"S-LoRA: Serving Thousands of Concurrent Adapters in 2026", Step 2), a set of
LoRA adapters (A: r x d_in, B: r rows of length d_out, scale alpha / r, as in
the same page's "Three Core Pillars" formula and Step 1), a batch of rows
each routed to one adapter or to none, and the unified page pool's physical
page order ("S-LoRA: Serving Thousands of Concurrent LoRA Adapters", Unified
paging).

Only data generation lives here.  Values are drawn with numpy PCG64 from
``SeedSequence([seed, config, tag, ...])`` keys; large tensors are split in
fixed 4 Mi-element chunks, each with its own key, so the values do not depend
on the thread count.  bf16 tensors are returned as uint16 bit patterns,
rounded to nearest-even from float32 draws; fp32 tensors as float32.

Readings of details the configurations leave open: "N(0, s)" names a
standard deviation; popularity is a bounded Zipf p_k ~ k^-s over k = 1..N
(adapter id k-1), drawn i.i.d. per request;
alpha = 2r wherever a configuration does not give it.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5")
_CFG_NO = {n: i + 1 for i, n in enumerate(CONFIG_NAMES)}

# SeedSequence tags (second key word after the config number)
_T_W0, _T_X, _T_A, _T_B, _T_ROWS, _T_RANKS, _T_FREE, _T_KV, _T_REQ, _T_COLD, _T_TRACE = range(11)

_CHUNK = 1 << 22
_EXEC: Optional[ThreadPoolExecutor] = None


def _executor() -> ThreadPoolExecutor:
    global _EXEC
    if _EXEC is None:
        _EXEC = ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
    return _EXEC


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.array(a, dtype=np.float32, copy=True).view(np.uint32)
    bias = u >> np.uint32(16)
    bias &= np.uint32(1)
    bias += np.uint32(0x7FFF)
    u += bias
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def _to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16_bits_from_f32 through torch's CPU conversion (also round to nearest
    even for finite values, and much faster on large arrays)."""
    import torch
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the float32 values they denote (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(n: int, std: float, key: Tuple[int, ...], bf16: bool) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(i: int) -> None:
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        v = _rng(*key, i).standard_normal(hi - lo, dtype=np.float32)
        v *= np.float32(std)
        out[lo:hi] = _to_bf16_bits(v) if bf16 else v

    if nchunks <= 1:
        for i in range(nchunks):
            work(i)
    else:
        list(_executor().map(work, range(nchunks)))
    return out


def zipf_probs(n: int, s: float) -> np.ndarray:
    """Bounded Zipf popularity p_k ~ k^-s, k = 1..n (index k-1)."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-float(s))
    return w / w.sum()


@dataclass(frozen=True)
class AdapterSpec:
    adapter_id: int
    rank: int
    alpha: float


@dataclass(frozen=True)
class Request:
    """One request of the batch: ``n_tokens`` consecutive rows routed to
    ``adapter_id`` (-1 = the un-adapted base model)."""
    n_tokens: int
    adapter_id: int
    kind: str  # "prefill" or "decode"


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str                      # "f32" or "bf16"
    page_elems: int
    n_layers: int
    proj_names: Tuple[str, ...]
    d_in: Tuple[int, ...]
    d_out: Tuple[int, ...]
    w0_std: float
    a_std: Tuple[float, ...]        # per projection
    b_std: float
    adapters: Dict[int, AdapterSpec]
    requests: List[Request]
    num_pages: int
    free_order: np.ndarray          # int32 permutation of [0, num_pages)
    max_slots: int
    max_rank: int
    setup_ops: List[tuple]          # ("page_in", id) | ("alloc_kv", n) | ("free_kv", idx) | ("evict", id)
    step_ops: List[tuple] = field(default_factory=list)
    cold_adapters: Tuple[int, ...] = ()
    x_input_of_proj: Tuple[int, ...] = (0,)   # which layer input feeds each projection
    cache: bool = True
    _memo: dict = field(default_factory=dict, repr=False)

    # ---- shapes -----------------------------------------------------------
    @property
    def n_proj(self) -> int:
        return len(self.proj_names)

    @property
    def bf16(self) -> bool:
        return self.dtype == "bf16"

    @property
    def elem_bytes(self) -> int:
        return 2 if self.bf16 else 4

    @property
    def T(self) -> int:
        return sum(r.n_tokens for r in self.requests)

    @property
    def n_prefill_rows(self) -> int:
        return sum(r.n_tokens for r in self.requests if r.kind == "prefill")

    @property
    def n_decode_rows(self) -> int:
        return sum(r.n_tokens for r in self.requests if r.kind == "decode")

    def row_adapter(self) -> np.ndarray:
        """Adapter id of every row (-1 = none), prefill rows first, then decode rows."""
        return np.concatenate([np.full(r.n_tokens, r.adapter_id, np.int32) for r in self.requests]) \
            if self.requests else np.zeros(0, np.int32)

    def prefill_requests(self) -> List[Request]:
        return [r for r in self.requests if r.kind == "prefill"]

    def decode_requests(self) -> List[Request]:
        return [r for r in self.requests if r.kind == "decode"]

    def proj_groups(self) -> List[List[int]]:
        """Runs of consecutive projections that read the same layer input (q, k, v;
        gate, up): one lora_linear_multi call each."""
        return proj_groups_of(self.x_input_of_proj)

    def pages_per_rank(self) -> int:
        """Pool pages one rank-row of an adapter takes over all (layer, projection) pairs."""
        P = self.page_elems
        return self.n_layers * sum(-(-di // P) + -(-do // P) for di, do in zip(self.d_in, self.d_out))

    def adapter_pages(self, adapter_id: int) -> int:
        return self.adapters[adapter_id].rank * self.pages_per_rank()

    # ---- tensors ----------------------------------------------------------
    def _get(self, key, make):
        if not self.cache:
            return make()
        if key not in self._memo:
            self._memo[key] = make()
        return self._memo[key]

    def w0(self, layer: int = 0, proj: int = 0) -> np.ndarray:
        """Base weight [d_out, d_in]."""
        c = _CFG_NO[self.name]
        di, do = self.d_in[proj], self.d_out[proj]
        return self._get(("w0", layer, proj), lambda: _normal(
            do * di, self.w0_std, (self.seed, c, _T_W0, layer, proj), self.bf16).reshape(do, di))

    def w0_fp8(self, layer: int = 0, proj: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """The base weight as an FP8 base: E4M3 codes uint8 [d_out, d_in] and an fp32
        scale per output row (largest |w| of the row maps to 448, the largest finite
        E4M3 value), from the same fp32 draw the bf16 base rounds.  The codes are the
        nearest (ties to even) of w / scale, by torch's float8_e4m3fn conversion."""
        import torch
        c = _CFG_NO[self.name]
        di, do = self.d_in[proj], self.d_out[proj]

        def make():
            w = _normal(do * di, self.w0_std, (self.seed, c, _T_W0, layer, proj), False).reshape(do, di)
            amax = np.abs(w).max(axis=1).astype(np.float32)
            scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
            q = np.clip(w / scale[:, None], -448.0, 448.0).astype(np.float32)
            codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            return np.ascontiguousarray(codes), scale
        return self._get(("w0fp8", layer, proj), make)

    def x(self, layer: int = 0, proj: int = 0) -> np.ndarray:
        """Layer input [T, d_in] for a projection; projections that share an
        input (q, k, v read the attention block's input; gate, up the MLP
        block's) share the array."""
        c = _CFG_NO[self.name]
        src = self.x_input_of_proj[proj]
        di = self.d_in[proj]
        return self._get(("x", layer, src), lambda: _normal(
            self.T * di, 1.0, (self.seed, c, _T_X, layer, src), self.bf16).reshape(self.T, di))

    def adapter_AB(self, adapter_id: int, layer: int = 0, proj: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Logical (dense) adapter factors: A [r, d_in] and B [r, d_out]."""
        c = _CFG_NO[self.name]
        r = self.adapters[adapter_id].rank
        di, do = self.d_in[proj], self.d_out[proj]

        def make():
            A = _normal(r * di, self.a_std[proj], (self.seed, c, _T_A, adapter_id, layer, proj), self.bf16)
            B = _normal(r * do, self.b_std, (self.seed, c, _T_B, adapter_id, layer, proj), self.bf16)
            return A.reshape(r, di), B.reshape(r, do)
        return self._get(("ab", adapter_id, layer, proj), make)

    def adapter_host_blob(self, adapter_id: int) -> Tuple[np.ndarray, np.ndarray]:
        """All of an adapter's factors as the two dense host arrays a page-in
        reads: A_all = concat over (layer, proj) of A [r, d_in]; B_all likewise.
        The (layer, proj) pieces are drawn in parallel straight into place."""
        r = self.adapters[adapter_id].rank
        pairs = [(l, p) for l in range(self.n_layers) for p in range(self.n_proj)]
        dt = np.uint16 if self.bf16 else np.float32
        a_off, b_off = [0], [0]
        for _, p in pairs:
            a_off.append(a_off[-1] + r * self.d_in[p])
            b_off.append(b_off[-1] + r * self.d_out[p])
        A_all, B_all = np.empty(a_off[-1], dt), np.empty(b_off[-1], dt)

        def fill(i: int) -> None:
            l, p = pairs[i]
            A, B = self.adapter_AB(adapter_id, l, p)
            A_all[a_off[i]:a_off[i + 1]] = A.reshape(-1)
            B_all[b_off[i]:b_off[i + 1]] = B.reshape(-1)

        if len(pairs) == 1:
            fill(0)
        else:
            list(_executor().map(fill, range(len(pairs))))
        return A_all, B_all

    def drop_cache(self) -> None:
        self._memo.clear()


# ---------------------------------------------------------------------------
# the five configurations
# ---------------------------------------------------------------------------

def _slack_pages(used: int) -> int:
    """Pool size: 25 % above the pages a configuration uses, rounded up to 1024."""
    return int(math.ceil(1.25 * used / 1024.0)) * 1024


def _ranks_uniform(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.choice(np.array([8, 16, 32, 64]), size=n)


def make_workload(name: str, seed: int = 0, cache: bool = True, **overrides) -> Workload:
    """Build the named workload (``c1`` .. ``c5``).  ``overrides`` may change a
    few sizes for reduced test variants: ``n_tokens`` (c2/c3 decode rows),
    ``n_layers`` (c5)."""
    if name not in _CFG_NO:
        raise ValueError(f"unknown workload {name!r}; choose from {CONFIG_NAMES}")
    c = _CFG_NO[name]
    return {"c1": _c1, "c2": _c2, "c3": _c3, "c4": _c4, "c5": _c5}[name](seed, c, cache, **overrides)


def _page_in_all(ids: Sequence[int]) -> List[tuple]:
    return [("page_in", int(a)) for a in ids]


def _c1(seed, c, cache, n_tokens: int = 8):
    """Tiny single layer, fp32: 256 -> 256, four adapters of ranks 4, 8, 4, 8,
    a 64-page pool of 256 floats in a seeded random physical order, eight
    decode rows each routed uniformly to {none, 0, 1, 2, 3}."""
    ranks = [4, 8, 4, 8]
    adapters = {i: AdapterSpec(i, r, 2.0 * r) for i, r in enumerate(ranks)}
    choice = _rng(seed, c, _T_ROWS).integers(-1, 4, size=n_tokens)
    reqs = [Request(1, int(a), "decode") for a in choice]
    num_pages = 64
    free = _rng(seed, c, _T_FREE).permutation(num_pages).astype(np.int32)
    return Workload(name="c1", seed=seed, dtype="f32", page_elems=256, n_layers=1,
                    proj_names=("proj",), d_in=(256,), d_out=(256,), w0_std=1.0 / 256,
                    a_std=(1.0 / 256,), b_std=0.02, adapters=adapters, requests=reqs,
                    num_pages=num_pages, free_order=free, max_slots=8, max_rank=8,
                    setup_ops=_page_in_all(range(4)), cache=cache)


def _c2(seed, c, cache, n_tokens: int = 64):
    """Decode, Llama-7B attention projection 4096 x 4096, bf16: 1000 resident
    rank-16 adapters (alpha 32), 64 rows routed Zipf(1.0), pages scattered."""
    n_ad = 1000
    adapters = {i: AdapterSpec(i, 16, 32.0) for i in range(n_ad)}
    ids = _rng(seed, c, _T_ROWS).choice(n_ad, size=n_tokens, p=zipf_probs(n_ad, 1.0))
    reqs = [Request(1, int(a), "decode") for a in ids]
    used = n_ad * 16 * 2
    num_pages = _slack_pages(used)
    free = _rng(seed, c, _T_FREE).permutation(num_pages).astype(np.int32)
    return Workload(name="c2", seed=seed, dtype="bf16", page_elems=4096, n_layers=1,
                    proj_names=("q",), d_in=(4096,), d_out=(4096,), w0_std=0.02,
                    a_std=(1.0 / 64,), b_std=0.01, adapters=adapters, requests=reqs,
                    num_pages=num_pages, free_order=free, max_slots=1024, max_rank=64,
                    setup_ops=_page_in_all(range(n_ad)), cache=cache)


def _c3(seed, c, cache, n_tokens: int = 256):
    """Decode with mixed ranks, Llama-7B MLP up projection 4096 -> 11008, bf16:
    2000 resident adapters of ranks {8,16,32,64} (alpha 2r), 256 rows of which
    exactly 10 % (rounded) are null at seeded positions and the rest Zipf(0.8);
    every adapter page-in is followed by a dummy KV block of U{1..32} pages."""
    n_ad = 2000
    ranks = _ranks_uniform(_rng(seed, c, _T_RANKS), n_ad)
    adapters = {i: AdapterSpec(i, int(r), 2.0 * int(r)) for i, r in enumerate(ranks)}
    rr = _rng(seed, c, _T_ROWS)
    ids = rr.choice(n_ad, size=n_tokens, p=zipf_probs(n_ad, 0.8)).astype(np.int64)
    n_null = int(round(0.1 * n_tokens))
    null_pos = rr.choice(n_tokens, size=n_null, replace=False)
    ids[null_pos] = -1
    reqs = [Request(1, int(a), "decode") for a in ids]
    kv = _rng(seed, c, _T_KV).integers(1, 33, size=n_ad)
    ops: List[tuple] = []
    for i in range(n_ad):
        ops.append(("page_in", i))
        ops.append(("alloc_kv", int(kv[i])))
    used = int(sum(4 * int(r) for r in ranks)) + int(kv.sum())
    num_pages = _slack_pages(used)
    free = _rng(seed, c, _T_FREE).permutation(num_pages).astype(np.int32)
    return Workload(name="c3", seed=seed, dtype="bf16", page_elems=4096, n_layers=1,
                    proj_names=("up",), d_in=(4096,), d_out=(11008,), w0_std=0.02,
                    a_std=(1.0 / 64,), b_std=0.01, adapters=adapters, requests=reqs,
                    num_pages=num_pages, free_order=free, max_slots=2048, max_rank=64,
                    setup_ops=ops, cache=cache)


def _c4(seed, c, cache):
    """Prefill, 4096 x 4096, bf16: 16 requests of U{64..1024} tokens, each one
    contiguous segment routed to one of 500 adapters (ranks {8..64}, uniform
    choice); two seeded segments use no adapter."""
    n_ad = 500
    ranks = _ranks_uniform(_rng(seed, c, _T_RANKS), n_ad)
    adapters = {i: AdapterSpec(i, int(r), 2.0 * int(r)) for i, r in enumerate(ranks)}
    rr = _rng(seed, c, _T_REQ)
    lens = rr.integers(64, 1025, size=16)
    ids = rr.integers(0, n_ad, size=16).astype(np.int64)
    ids[rr.choice(16, size=2, replace=False)] = -1
    reqs = [Request(int(n), int(a), "prefill") for n, a in zip(lens, ids)]
    used = int(sum(2 * int(r) for r in ranks))
    num_pages = _slack_pages(used)
    free = _rng(seed, c, _T_FREE).permutation(num_pages).astype(np.int32)
    return Workload(name="c4", seed=seed, dtype="bf16", page_elems=4096, n_layers=1,
                    proj_names=("q",), d_in=(4096,), d_out=(4096,), w0_std=0.02,
                    a_std=(1.0 / 64,), b_std=0.01, adapters=adapters, requests=reqs,
                    num_pages=num_pages, free_order=free, max_slots=512, max_rank=64,
                    setup_ops=_page_in_all(range(n_ad)), cache=cache)


LLAMA7B_PROJ = ("q", "k", "v", "o", "gate", "up", "down")
LLAMA7B_DIN = (4096, 4096, 4096, 4096, 4096, 4096, 11008)
LLAMA7B_DOUT = (4096, 4096, 4096, 4096, 11008, 11008, 4096)
def proj_groups_of(x_input_of_proj: Sequence[int]) -> List[List[int]]:
    """Runs of consecutive projections with the same layer input."""
    out: List[List[int]] = []
    for p, src in enumerate(x_input_of_proj):
        if out and x_input_of_proj[out[-1][0]] == src:
            out[-1].append(p)
        else:
            out.append([p])
    return out


# layer inputs: 0 = the attention block's normed input (q, k, v), 1 = attention output (o),
# 2 = the MLP block's normed input (gate, up), 3 = MLP activation (down)
LLAMA7B_XSRC = (0, 0, 0, 1, 2, 2, 3)


def _c5(seed, c, cache, n_layers: int = 32):
    """One continuous-batching step over a Llama-7B projection stack (32 layers x
    q, k, v, o, gate, up, down), bf16.  2000-adapter Zipf(1.0) universe with
    ranks {8..64}; 8 prefill requests of U{128..512} tokens and 192 decode rows;
    the step's distinct adapters are resident except 16 seeded cold ones, paged
    in from host memory during the step; KV blocks of 2 pages per token per
    layer are taken from the same pool in the step."""
    n_univ = 2000
    ranks = _ranks_uniform(_rng(seed, c, _T_RANKS), n_univ)
    rr = _rng(seed, c, _T_REQ)
    p = zipf_probs(n_univ, 1.0)
    lens = rr.integers(128, 513, size=8)
    pre_ids = rr.choice(n_univ, size=8, p=p)
    dec_ids = rr.choice(n_univ, size=192, p=p)
    reqs = [Request(int(n), int(a), "prefill") for n, a in zip(lens, pre_ids)]
    reqs += [Request(1, int(a), "decode") for a in dec_ids]
    distinct = sorted(set(int(a) for a in pre_ids) | set(int(a) for a in dec_ids))
    cold = sorted(int(a) for a in _rng(seed, c, _T_COLD).choice(distinct, size=min(16, len(distinct)), replace=False))
    resident = [a for a in distinct if a not in set(cold)]
    adapters = {a: AdapterSpec(a, int(ranks[a]), 2.0 * int(ranks[a])) for a in distinct}
    P = 4096
    per_rank = n_layers * sum(-(-di // P) + -(-do // P) for di, do in zip(LLAMA7B_DIN, LLAMA7B_DOUT))
    T = int(lens.sum()) + 192
    kv_pages = 2 * T * n_layers
    used = per_rank * sum(int(ranks[a]) for a in distinct) + kv_pages
    num_pages = _slack_pages(used)
    free = _rng(seed, c, _T_FREE).permutation(num_pages).astype(np.int32)
    step_ops: List[tuple] = []
    for i, r in enumerate(reqs):
        step_ops.append(("alloc_kv", 2 * r.n_tokens * n_layers))
    step_ops += _page_in_all(cold)
    return Workload(name="c5", seed=seed, dtype="bf16", page_elems=P, n_layers=n_layers,
                    proj_names=LLAMA7B_PROJ, d_in=LLAMA7B_DIN, d_out=LLAMA7B_DOUT, w0_std=0.02,
                    a_std=tuple(1.0 / math.sqrt(d) for d in LLAMA7B_DIN), b_std=0.01,
                    adapters=adapters, requests=reqs, num_pages=num_pages, free_order=free,
                    max_slots=256, max_rank=64, setup_ops=_page_in_all(resident),
                    step_ops=step_ops, cold_adapters=tuple(cold), x_input_of_proj=LLAMA7B_XSRC,
                    cache=cache)


# ---------------------------------------------------------------------------
# arrival traces for the engine layer
# ---------------------------------------------------------------------------

def c5_universe_ranks(seed: int = 0) -> np.ndarray:
    """Ranks of the stack workload's 2000-adapter universe (the draw c5 makes)."""
    return _ranks_uniform(_rng(seed, _CFG_NO["c5"], _T_RANKS), 2000)


def engine_trace(n_steps: int, rate: float = 8.0, n_adapters: int = 2000, zipf_s: float = 1.0,
                 prompt: Tuple[int, int] = (128, 512), max_new: Tuple[int, int] = (8, 40), seed: int = 0
                 ) -> List[List[Tuple[int, int, int, int]]]:
    """Arrivals per step: Poisson(rate) requests, each (request id, adapter id drawn Zipf(zipf_s)
    over n_adapters, prompt tokens U[prompt], tokens to generate U[max_new]).  With the
    defaults a step in steady state holds about 8 prompts and 190 decode rows, the stack
    workload's mix."""
    g = _rng(seed, _CFG_NO["c5"], _T_TRACE)
    p = zipf_probs(n_adapters, zipf_s)
    out, rid = [], 0
    for _ in range(n_steps):
        n = int(g.poisson(rate))
        ads = g.choice(n_adapters, size=n, p=p)
        pr = g.integers(prompt[0], prompt[1] + 1, size=n)
        mn = g.integers(max_new[0], max_new[1] + 1, size=n)
        out.append([(rid + i, int(ads[i]), int(pr[i]), int(mn[i])) for i in range(n)])
        rid += n
    return out
