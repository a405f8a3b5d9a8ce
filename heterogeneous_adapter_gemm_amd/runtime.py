"""Device-memory plumbing around the C ABI.

``DevicePool`` allocates the pool's page buffer and metadata workspace with
PyTorch (the library itself never allocates device memory), pins adapter
host blobs for page-in, and forwards every operation to the library.  A
host-only pool (``device=None``) runs the allocator, tables and plans with
no GPU at all.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import _lib as L


def torch_dtype(dtype: int):
    import torch
    return torch.bfloat16 if dtype == L.LORA_BF16 else torch.float32


def host_tensor(arr: np.ndarray, pin: bool = True):
    """numpy (bf16 bits as uint16, or float32) -> torch CPU tensor of the
    matching dtype, pinned (allocated pinned, not registered) when asked."""
    import torch
    a = np.ascontiguousarray(arr)
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
    if pin:
        p = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
        p.copy_(t)
        return p
    return t


def device_tensor(arr: np.ndarray, device="cuda"):
    return host_tensor(arr, pin=False).to(device)


class DevicePool:
    def __init__(self, dtype: int, page_elems: int, num_pages: int, free_order: Optional[Sequence[int]],
                 n_layers: int, d_in: Sequence[int], d_out: Sequence[int], max_slots: int, max_rank: int,
                 max_tokens: int, max_segments: int, base_id: int = 0, device: Optional[str] = "cuda",
                 stage_bytes: int = 0, max_multi: int = 1):
        """stage_bytes > 0: a device staging area of that size for page-ins (copy engine into
        the staging area, then a scatter kernel); 0: page-ins gather over PCIe.  max_multi: most
        projections one linear_multi call takes."""
        self.dtype = dtype
        self.page_elems = page_elems
        self.num_pages = num_pages
        self.n_layers = n_layers
        self.d_in = list(d_in)
        self.d_out = list(d_out)
        self.base_id = base_id
        self.device = device
        desc, keep = L.make_desc(dtype, page_elems, num_pages, None, free_order, n_layers, d_in, d_out, max_slots,
                                 max_rank, max_tokens, max_segments, None, 0, base_id, max_multi=max_multi)
        self.pages = self.meta = self.stage = None
        if device is not None:
            import torch
            meta_bytes = L.lora_pool_meta_bytes(desc)
            self.pages = torch.empty(num_pages * page_elems, dtype=torch_dtype(dtype), device=device)
            self.meta = torch.empty(meta_bytes, dtype=torch.uint8, device=device)
            desc.pages_dev = self.pages.data_ptr()
            desc.meta_dev = self.meta.data_ptr()
            desc.meta_bytes = meta_bytes
            if stage_bytes > 0:
                self.stage = torch.empty(stage_bytes, dtype=torch.uint8, device=device)
                desc.stage_dev = self.stage.data_ptr()
                desc.stage_bytes = stage_bytes
        self.pool = L.lora_pool_create(desc, keep)
        self._host: Dict[int, tuple] = {}

    # -- adapters ---------------------------------------------------------------
    def page_in(self, adapter_id: int, rank: int, alpha: float, A_blob: Optional[np.ndarray] = None,
                B_blob: Optional[np.ndarray] = None, stream=None, base_id: Optional[int] = None) -> int:
        base = self.base_id if base_id is None else base_id
        if self.device is None:
            return L.lora_pool_page_in(self.pool, adapter_id, rank, alpha, base, None, None, None)
        hA, hB = host_tensor(A_blob), host_tensor(B_blob)
        slot = L.lora_pool_page_in(self.pool, adapter_id, rank, alpha, base, hA, hB, stream)
        self._host[adapter_id] = (hA, hB)   # the copy reads these until it has run
        return slot

    def page_in_pinned(self, adapter_id: int, rank: int, alpha: float, hA, hB, stream=None) -> int:
        """Page in from already-pinned torch host tensors (kept alive by the caller)."""
        return L.lora_pool_page_in(self.pool, adapter_id, rank, alpha, self.base_id, hA, hB, stream)

    def page_in_pinned_batch(self, items, stream=None) -> np.ndarray:
        """Page in several adapters, layer by layer: items = [(adapter_id, rank, alpha, hA, hB)]
        with already-pinned torch host tensors (kept alive by the caller)."""
        return L.lora_pool_page_in_batch(self.pool, [(a, r, al, self.base_id, hA, hB) for a, r, al, hA, hB in items],
                                         stream)

    def page_in_batch(self, items, stream=None) -> np.ndarray:
        """items = [(adapter_id, rank, alpha, A_blob, B_blob)] from host arrays (pinned copies
        are made and kept until drop_host_copies); host-only pools take no blobs."""
        if self.device is None:
            return L.lora_pool_page_in_batch(self.pool, [(a, r, al, self.base_id, None, None)
                                                         for a, r, al, *_ in items], None)
        reqs = []
        for a, r, al, A, B in items:
            hA, hB = host_tensor(A), host_tensor(B)
            self._host[a] = (hA, hB)
            reqs.append((a, r, al, self.base_id, hA, hB))
        return L.lora_pool_page_in_batch(self.pool, reqs, stream)

    def drop_host_copies(self) -> None:
        """Forget the pinned host blobs; call after the page-in work has run."""
        self._host.clear()

    def evict(self, adapter_id: int) -> None:
        L.lora_pool_evict(self.pool, adapter_id)
        self._host.pop(adapter_id, None)

    def slot_of(self, adapter_id: int) -> int:
        return L.lora_pool_slot_of(self.pool, adapter_id)

    def slots_of(self, adapter_ids) -> np.ndarray:
        return L.lora_pool_slots_of(self.pool, adapter_ids)

    def alloc_kv(self, n: int) -> np.ndarray:
        return L.lora_pool_alloc_kv(self.pool, n)

    def free_kv(self, pages) -> None:
        L.lora_pool_free_kv(self.pool, pages)

    def page_table(self, slot: int, layer: int, proj: int):
        return L.lora_pool_page_table(self.pool, slot, layer, proj)

    def free_list(self) -> np.ndarray:
        return L.lora_pool_free_list(self.pool)

    def stats(self):
        return L.lora_pool_stats(self.pool)

    # -- batches ------------------------------------------------------------------
    def plan(self, seg_start=None, seg_slot=None, token_slot=None, stream=None) -> L.Plan:
        return L.lora_plan_create(self.pool, seg_start, seg_slot, token_slot, stream)

    def linear(self, plan: L.Plan, layer: int, proj: int, x, w0, y, stream=None) -> None:
        L.lora_linear(self.pool, plan, layer, proj, x, w0, y, stream)

    def linear_multi(self, plan: L.Plan, layer: int, projs, x, w0s, ys, stream=None) -> None:
        """Projections projs of one layer that share x, their shrinks in shared launches."""
        L.lora_linear_multi(self.pool, plan, layer, projs, x, w0s, ys, stream)

    def linear_fp8(self, plan: L.Plan, layer: int, proj: int, x, w0_code, w0_scale, y, stream=None) -> None:
        L.lora_linear_fp8(self.pool, plan, layer, proj, x, w0_code, w0_scale, y, stream)

    def linear_decode(self, layer: int, proj: int, x, w0, y, token_slot, stream=None) -> None:
        L.lora_linear_decode(self.pool, layer, proj, x, w0, y, token_slot, stream)

    def linear_decode_noalloc(self, layer: int, proj: int, x, w0, y, token_slot, stream=None) -> None:
        L.lora_linear_decode_noalloc(self.pool, layer, proj, x, w0, y, token_slot, stream)

    def linear_prefill(self, layer: int, proj: int, x, w0, y, seg_start, seg_slot, stream=None) -> None:
        L.lora_linear_prefill(self.pool, layer, proj, x, w0, y, seg_start, seg_slot, stream)

    def set_timing(self, enable) -> None:
        """True / 1: time every call's kernels; k > 1: every k-th call; False / 0: off."""
        L.lora_pool_set_timing(self.pool, int(enable))

    def timing(self) -> Dict[str, tuple]:
        """{kernel name: (total ms, launches)} since timing was enabled."""
        return {name: L.lora_pool_timing(self.pool, k) for k, name in enumerate(L.KERNEL_NAMES)}

    def close(self) -> None:
        L.lora_pool_destroy(self.pool)


class AdapterEngine:
    """The engine layer over a DevicePool (host tier, GPU-tier LRU, look-ahead page-ins,
    admission; see lora_engine_* in the C header).

    Storage is two Python callables:
      info(adapter_id) -> (rank, alpha, base_id)
      fill(adapter_id, A, B): write the adapter's A and B blobs (layouts of page-in) into the
        flat host-cache views A and B (uint16 bf16 bits or float32, by the pool's dtype).
    An exception in either becomes a failed call (nonzero status) in the library.
    """

    def __init__(self, pool: DevicePool, info, fill, host_cache_bytes: int, max_step_tokens: int,
                 max_distinct_adapters: int, max_running: Optional[int] = None, prefetch_window: int = 64,
                 admit_in_flight: bool = True, max_wait_steps: int = 0, kv_pages_per_token: int = 0,
                 copy_stream=None):
        import ctypes
        self.pool = pool
        self.errors = errors = []   # the callbacks hold this list, not self (no reference cycle)
        elem = np.uint16 if pool.dtype == L.LORA_BF16 else np.float32
        esize = np.dtype(elem).itemsize

        def _info(_user, adapter_id, rank, alpha, base):
            try:
                r, a, b = info(int(adapter_id))
                rank[0], alpha[0], base[0] = int(r), float(a), int(b)
                return 0
            except Exception as exc:   # reported through the library's status
                errors.append(exc)
                return -1

        def _fill(_user, adapter_id, host_a, a_bytes, host_b, b_bytes):
            try:
                A = np.ctypeslib.as_array((ctypes.c_uint8 * a_bytes).from_address(host_a)).view(elem)
                B = np.ctypeslib.as_array((ctypes.c_uint8 * b_bytes).from_address(host_b)).view(elem)
                assert A.size * esize == a_bytes and B.size * esize == b_bytes
                fill(int(adapter_id), A, B)
                return 0
            except Exception as exc:
                errors.append(exc)
                return -1

        self._cb = (L.INFO_FN(_info), L.FILL_FN(_fill))
        d = L.lora_engine_desc()
        d.host_cache_bytes = int(host_cache_bytes)
        d.max_step_tokens = int(max_step_tokens)
        d.max_distinct_adapters = int(max_distinct_adapters)
        d.max_running = int(max_step_tokens if max_running is None else max_running)
        d.prefetch_window = int(prefetch_window)
        d.admit_in_flight = int(bool(admit_in_flight))
        d.max_wait_steps = int(max_wait_steps)
        d.kv_pages_per_token = int(kv_pages_per_token)
        d.info, d.fill = self._cb
        d.copy_stream = None if copy_stream is None else (copy_stream if isinstance(copy_stream, int)
                                                            else copy_stream.cuda_stream)
        self.engine = L.lora_engine_create(pool.pool, d, list(self._cb))
        self.batch = None

    def submit(self, request_id: int, adapter_id: int, prompt_tokens: int, max_new_tokens: int) -> None:
        L.lora_engine_submit(self.engine, request_id, adapter_id, prompt_tokens, max_new_tokens)

    def cancel(self, request_id: int) -> None:
        L.lora_engine_cancel(self.engine, request_id)

    def step(self, stream=None):
        """-> (batch dict with 'requests', 'adapters', 'rows' arrays added, plan or None)."""
        b, plan = L.lora_engine_step(self.engine, 0 if self.pool.device is None else stream)
        ids, ads, rows = L.lora_engine_batch_requests(self.engine, b["n_requests"])
        b.update(requests=ids, adapters=ads, rows=rows)
        self.batch = b
        return b, plan

    def step_done(self) -> None:
        L.lora_engine_step_done(self.engine)
        self.batch = None

    def row_adapter(self) -> np.ndarray:
        """Adapter id of every row of the current step's plan (-1 = none)."""
        b = self.batch
        return np.repeat(b["adapters"], b["rows"]).astype(np.int32)

    def kv_pages(self, request_id: int) -> np.ndarray:
        return L.lora_engine_kv_pages(self.engine, request_id)

    def stats(self) -> Dict[str, float]:
        return L.lora_engine_get_stats(self.engine)

    def reset_stats(self) -> None:
        L.lora_engine_reset_stats(self.engine)

    def close(self) -> None:
        L.lora_engine_destroy(self.engine)
