"""Load a generated workload into a device pool through the library's API.

Moves the generator's arrays to device memory and replays the workload's op
log (page-ins from pinned host memory, KV allocations) through the C ABI.
No arithmetic of the method happens here.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from .gen import Workload


def dtype_code(wl: Workload) -> int:
    from heterogeneous_adapter_gemm_amd import LORA_BF16, LORA_F32
    return LORA_BF16 if wl.bf16 else LORA_F32


def build_pool(wl: Workload, device: str = "cuda", max_tokens: Optional[int] = None, max_segments: int = 32,
               free_order=None, stream=None, stage_bytes: int = 0, max_multi: int = 1):
    """Create the device pool of ``wl`` and replay its setup ops; returns
    (pool, kv_blocks).  ``free_order`` may override the physical page order;
    ``stage_bytes`` > 0 gives the pool a device staging area for page-ins;
    ``max_multi`` is the most projections one lora_linear_multi call takes."""
    from heterogeneous_adapter_gemm_amd import DevicePool
    fo = wl.free_order if free_order is None else free_order
    pool = DevicePool(dtype_code(wl), wl.page_elems, wl.num_pages, fo, wl.n_layers, wl.d_in, wl.d_out,
                      wl.max_slots, wl.max_rank, max_tokens or max(wl.T, 1), max_segments, device=device,
                      stage_bytes=stage_bytes, max_multi=max_multi)
    kv = replay(wl, pool, wl.setup_ops, stream)
    return pool, kv


def replay(wl: Workload, pool, ops, stream=None, settle: bool = True, batch: bool = False) -> List[np.ndarray]:
    """Replay an op log through the pool.  With ``settle`` the pinned host blobs
    of finished page-ins are let go whenever more than 1 GiB is held, and at the
    end; without it they stay with the pool until the caller has synchronised
    and called ``pool.drop_host_copies()`` (page-ins overlapping later work).
    With ``batch`` each run of consecutive page-ins is one batched page-in
    (copied layer by layer across its adapters)."""
    kv: List[np.ndarray] = []
    held = 0
    run = []

    def flush():
        nonlocal held
        if run:
            pool.page_in_batch(run, stream)
            run.clear()
            if settle and pool.device is not None and held > (1 << 30):
                _settle(pool)
                held = 0

    for op in ops:
        if op[0] == "page_in":
            a = wl.adapters[op[1]]
            A, B = wl.adapter_host_blob(a.adapter_id)
            held += A.nbytes + B.nbytes
            if batch:
                run.append((a.adapter_id, a.rank, a.alpha, A, B))
            else:
                pool.page_in(a.adapter_id, a.rank, a.alpha, A, B, stream)
            del A, B
            if not wl.cache:
                wl.drop_cache()
            if not batch and settle and pool.device is not None and held > (1 << 30):
                _settle(pool)
                held = 0
            continue
        flush()
        if op[0] == "alloc_kv":
            kv.append(pool.alloc_kv(op[1]))
        elif op[0] == "free_kv":
            pool.free_kv(kv[op[1]])
        elif op[0] == "evict":
            pool.evict(op[1])
        else:
            raise ValueError(op)
    flush()
    if settle and pool.device is not None:
        _settle(pool)
    return kv


def _settle(pool) -> None:
    """Wait for the enqueued page-ins, then let their pinned host blobs go."""
    import torch
    torch.cuda.synchronize()
    pool.drop_host_copies()


def batch_index(wl: Workload, pool) -> Dict[str, np.ndarray]:
    """The per-step index through the library: slots of the prefill segments
    and of the decode rows (-1 = no adapter)."""
    pre = wl.prefill_requests()
    dec = wl.decode_requests()
    out: Dict[str, np.ndarray] = {}
    if pre:
        lens = np.array([r.n_tokens for r in pre], np.int64)
        out["seg_start"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        out["seg_slot"] = pool.slots_of([r.adapter_id for r in pre])
    if dec:
        out["token_slot"] = pool.slots_of([r.adapter_id for r in dec])
    return out


def oracle_adapters(wl: Workload, layer: int = 0, proj: int = 0, ids=None) -> Dict[int, tuple]:
    """{id: (rank, alpha, A, B)} of the adapters the batch uses, for the oracle."""
    ids = sorted(set(int(a) for a in wl.row_adapter() if a >= 0)) if ids is None else ids
    out = {}
    for a in ids:
        spec = wl.adapters[a]
        A, B = wl.adapter_AB(a, layer, proj)
        out[a] = (spec.rank, spec.alpha, A, B)
    return out
