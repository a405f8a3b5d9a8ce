"""ctypes binding of ``libhagemm.so`` (the C ABI in include/lora_gemm.h).

Argument marshalling only: every function has the name of the C entry point
it calls, turns tensors and arrays into pointers, the current torch stream
into a ``hipStream_t`` and a negative status into ``LoraError``.  All work
runs in the library's gfx950 kernels; there is no Python or CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# HAGEMM_LIB: another build of the same sources (the host-sanitizer build of the tests)
LIB_PATH = os.environ.get("HAGEMM_LIB") or os.path.join(_HERE, "libhagemm.so")

LORA_OK = 0
LORA_EINVAL = -1
LORA_ENOPAGES = -2
LORA_ENOTRESIDENT = -3
LORA_EBUSY = -4
LORA_EEXIST = -5
LORA_EBASE = -6
LORA_EHIP = -7
LORA_ENOSLOT = -8
LORA_F32 = 0
LORA_BF16 = 1

ERROR_NAMES = {LORA_EINVAL: "EINVAL", LORA_ENOPAGES: "ENOPAGES", LORA_ENOTRESIDENT: "ENOTRESIDENT",
               LORA_EBUSY: "EBUSY", LORA_EEXIST: "EEXIST", LORA_EBASE: "EBASE", LORA_EHIP: "EHIP",
               LORA_ENOSLOT: "ENOSLOT"}


class LoraError(RuntimeError):
    def __init__(self, code: int, func: str, msg: str):
        super().__init__(f"{func}: {ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


class lora_pool_desc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("page_elems", ctypes.c_int32), ("num_pages", ctypes.c_int64),
                ("pages_dev", ctypes.c_void_p), ("free_order", ctypes.POINTER(ctypes.c_int32)),
                ("n_layers", ctypes.c_int32), ("n_proj", ctypes.c_int32),
                ("d_in", ctypes.POINTER(ctypes.c_int32)), ("d_out", ctypes.POINTER(ctypes.c_int32)),
                ("max_slots", ctypes.c_int32), ("max_rank", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("max_segments", ctypes.c_int32), ("meta_dev", ctypes.c_void_p), ("meta_bytes", ctypes.c_int64),
                ("base_id", ctypes.c_uint64), ("stage_dev", ctypes.c_void_p), ("stage_bytes", ctypes.c_int64),
                ("max_multi", ctypes.c_int32)]


_VP = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)

# storage callbacks of the engine layer
INFO_FN = ctypes.CFUNCTYPE(ctypes.c_int, _VP, ctypes.c_int32, _I32P, ctypes.POINTER(ctypes.c_float),
                           ctypes.POINTER(ctypes.c_uint64))
FILL_FN = ctypes.CFUNCTYPE(ctypes.c_int, _VP, ctypes.c_int32, _VP, ctypes.c_int64, _VP, ctypes.c_int64)


class lora_engine_desc(ctypes.Structure):
    _fields_ = [("host_cache_bytes", ctypes.c_int64), ("max_step_tokens", ctypes.c_int32),
                ("max_distinct_adapters", ctypes.c_int32), ("max_running", ctypes.c_int32),
                ("prefetch_window", ctypes.c_int32), ("admit_in_flight", ctypes.c_int32),
                ("max_wait_steps", ctypes.c_int32), ("kv_pages_per_token", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("info", INFO_FN), ("fill", FILL_FN), ("user", _VP),
                ("copy_stream", _VP)]


class lora_engine_batch(ctypes.Structure):
    _fields_ = [("plan", _VP), ("n_requests", ctypes.c_int32), ("n_prefill", ctypes.c_int32),
                ("n_rows", ctypes.c_int32), ("n_distinct", ctypes.c_int32)]


class lora_engine_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "steps", "rows", "admitted", "finished", "waiting", "running", "cancelled", "arrivals_resident",
        "arrivals_missing", "host_hits", "host_misses", "page_ins", "page_in_bytes", "gpu_evictions",
        "host_evictions", "room_stalls", "kv_stalls")] + [(n, ctypes.c_double) for n in (
        "page_in_ms_p50", "page_in_ms_p99", "page_in_ms_max", "copy_ms_p50", "copy_ms_p99", "wait_ms_hit_p50",
        "wait_ms_hit_p99", "wait_ms_miss_p50", "wait_ms_miss_p99", "wait_steps_p99", "wait_steps_max",
        "storage_ms_p50", "storage_ms_p99")]

_SIGS = {
    "lora_pool_meta_bytes": [ctypes.POINTER(lora_pool_desc), _I64P],
    "lora_pool_create": [ctypes.POINTER(lora_pool_desc), ctypes.POINTER(_VP)],
    "lora_pool_destroy": [_VP],
    "lora_pool_page_in": [_VP, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_uint64, _VP, ctypes.c_int64,
                          _VP, ctypes.c_int64, _VP, _I32P],
    "lora_pool_page_in_batch": [_VP, ctypes.c_int32, _VP, _VP, _I32P],
    "lora_pool_evict": [_VP, ctypes.c_int32],
    "lora_pool_slot_of": [_VP, ctypes.c_int32, _I32P],
    "lora_pool_slots_of": [_VP, ctypes.c_int32, _I32P, _I32P],
    "lora_pool_acquire": [_VP, ctypes.c_int32],
    "lora_pool_release": [_VP, ctypes.c_int32],
    "lora_pool_alloc_kv": [_VP, ctypes.c_int32, _I32P],
    "lora_pool_free_kv": [_VP, ctypes.c_int32, _I32P],
    "lora_pool_page_table": [_VP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _I32P, _I32P],
    "lora_pool_stats": [_VP, _I64P, _I32P, _I64P],
    "lora_pool_free_list": [_VP, ctypes.c_int64, _I32P, _I64P],
    "lora_pool_slot_info": [_VP, ctypes.c_int32, _I32P, ctypes.POINTER(ctypes.c_float), _I32P],
    "lora_plan_create": [_VP, _I32P, _I32P, ctypes.c_int32, _I32P, ctypes.c_int32, _VP, ctypes.POINTER(_VP)],
    "lora_plan_destroy": [_VP],
    "lora_plan_groups": [_VP, _I32P, _I32P, _I32P, _I32P, _I32P],
    "lora_linear": [_VP, _VP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP],
    "lora_linear_multi": [_VP, _VP, ctypes.c_int32, ctypes.c_int32, _I32P, _VP, ctypes.POINTER(_VP),
                          ctypes.POINTER(_VP), _VP],
    "lora_linear_decode": [_VP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _I32P, ctypes.c_int32, _VP],
    "lora_linear_prefill": [_VP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _I32P, _I32P, ctypes.c_int32, _VP],
    "lora_linear_decode_noalloc": [_VP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _I32P, ctypes.c_int32, _VP],
    "base_gemm": [ctypes.c_int32, _VP, _VP, _VP, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _VP],
    "base_gemm_fp8": [_VP, _VP, _VP, _VP, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _VP],
    "lora_linear_fp8": [_VP, _VP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP],
    "lora_engine_create": [_VP, ctypes.POINTER(lora_engine_desc), ctypes.POINTER(_VP)],
    "lora_engine_destroy": [_VP],
    "lora_engine_submit": [_VP, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32],
    "lora_engine_cancel": [_VP, ctypes.c_int64],
    "lora_engine_step": [_VP, _VP, ctypes.POINTER(lora_engine_batch)],
    "lora_engine_batch_requests": [_VP, _I64P, _I32P, _I32P],
    "lora_engine_step_done": [_VP],
    "lora_engine_kv_pages": [_VP, ctypes.c_int64, ctypes.c_int32, _I32P, _I32P],
    "lora_engine_get_stats": [_VP, ctypes.POINTER(lora_engine_stats)],
    "lora_engine_reset_stats": [_VP],
    "lora_pool_set_timing": [_VP, ctypes.c_int32],
    "lora_pool_timing": [_VP, ctypes.c_int32, ctypes.POINTER(ctypes.c_double), _I64P],
    "lora_probe_mfma": [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _VP, _VP, ctypes.POINTER(ctypes.c_double)],
    "lora_probe_read": [_VP, ctypes.c_int64, _VP, ctypes.c_int32, _VP, _VP],
    "lora_last_error": [],
    "lora_version": [],
}
EXPORTED = tuple(_SIGS)

_LIB: Optional[ctypes.CDLL] = None


def library() -> ctypes.CDLL:
    """Load the in-tree library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m heterogeneous_adapter_gemm_amd.build` (there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name in ("lora_last_error", "lora_version") else ctypes.c_int
        _LIB = lib
    return _LIB


def _check(rc: int, func: str) -> None:
    if rc != LORA_OK:
        raise LoraError(rc, func, library().lora_last_error().decode())


def _addr(obj) -> Optional[int]:
    """Device/host address of a tensor, array or raw int (None stays NULL)."""
    if obj is None:
        return None
    if isinstance(obj, int):
        return obj
    if hasattr(obj, "data_ptr"):
        return obj.data_ptr()
    if isinstance(obj, np.ndarray):
        return obj.ctypes.data
    raise TypeError(f"cannot take the address of {type(obj)}")


def _i32(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i32p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_I32P)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Pool:
    """Owns a ``lora_pool*``; keeps the descriptor's arrays alive."""

    def __init__(self, handle: int, desc: lora_pool_desc, keep: list):
        self.handle = handle
        self.desc = desc
        self._keep = keep
        self.engines: set = set()   # handles of live engines over this pool, destroyed first

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            for h in list(getattr(self, "engines", ())):
                _LIB.lora_engine_destroy(h)
            self.engines = set()
            _LIB.lora_pool_destroy(self.handle)
            self.handle = None


class Plan:
    def __init__(self, handle: int, pool: Pool, owned: bool = True):
        self.handle = handle
        self.pool = pool
        self.owned = owned   # False: an engine step's plan, destroyed by lora_engine_step_done

    def __del__(self):
        if self.owned and getattr(self, "handle", None) and _LIB is not None:
            _LIB.lora_plan_destroy(self.handle)
            self.handle = None


def make_desc(dtype: int, page_elems: int, num_pages: int, pages_dev, free_order, n_layers: int,
              d_in: Sequence[int], d_out: Sequence[int], max_slots: int, max_rank: int, max_tokens: int,
              max_segments: int, meta_dev=None, meta_bytes: int = 0, base_id: int = 0, stage_dev=None,
              stage_bytes: int = 0, max_multi: int = 1):
    fo = _i32(free_order)
    di, do = _i32(d_in), _i32(d_out)
    d = lora_pool_desc(dtype=dtype, page_elems=page_elems, num_pages=num_pages, pages_dev=_addr(pages_dev),
                       free_order=_i32p(fo), n_layers=n_layers, n_proj=len(di), d_in=_i32p(di), d_out=_i32p(do),
                       max_slots=max_slots, max_rank=max_rank, max_tokens=max_tokens, max_segments=max_segments,
                       meta_dev=_addr(meta_dev), meta_bytes=meta_bytes, base_id=base_id,
                       stage_dev=_addr(stage_dev), stage_bytes=stage_bytes, max_multi=max_multi)
    return d, [fo, di, do]


def lora_pool_meta_bytes(desc: lora_pool_desc) -> int:
    out = ctypes.c_int64()
    _check(library().lora_pool_meta_bytes(ctypes.byref(desc), ctypes.byref(out)), "lora_pool_meta_bytes")
    return out.value


def lora_pool_create(desc: lora_pool_desc, keep: list) -> Pool:
    h = _VP()
    _check(library().lora_pool_create(ctypes.byref(desc), ctypes.byref(h)), "lora_pool_create")
    return Pool(h.value, desc, keep)


def lora_pool_destroy(pool: Pool) -> None:
    if pool.handle:
        for h in list(pool.engines):
            _check(library().lora_engine_destroy(h), "lora_engine_destroy")
        pool.engines = set()
        _check(library().lora_pool_destroy(pool.handle), "lora_pool_destroy")
        pool.handle = None


def lora_pool_page_in(pool: Pool, adapter_id: int, rank: int, alpha: float, base_id: int, host_A, host_B,
                      stream=None, host_A_bytes: Optional[int] = None, host_B_bytes: Optional[int] = None) -> int:
    def nbytes(t):
        if t is None:
            return 0
        return t.numel() * t.element_size() if hasattr(t, "element_size") else t.nbytes
    slot = ctypes.c_int32(-1)
    _check(library().lora_pool_page_in(
        pool.handle, adapter_id, rank, alpha, base_id, _addr(host_A),
        nbytes(host_A) if host_A_bytes is None else host_A_bytes, _addr(host_B),
        nbytes(host_B) if host_B_bytes is None else host_B_bytes, _stream(stream) if host_A is not None else None,
        ctypes.byref(slot)), "lora_pool_page_in")
    return slot.value


class lora_page_in_req(ctypes.Structure):
    _fields_ = [("adapter_id", ctypes.c_int32), ("rank", ctypes.c_int32), ("alpha", ctypes.c_float),
                ("reserved", ctypes.c_int32), ("base_id", ctypes.c_uint64), ("host_A", _VP),
                ("host_A_bytes", ctypes.c_int64), ("host_B", _VP), ("host_B_bytes", ctypes.c_int64)]


def lora_pool_page_in_batch(pool: Pool, reqs, stream=None) -> np.ndarray:
    """reqs: sequence of (adapter_id, rank, alpha, base_id, host_A, host_B) with
    pinned host tensors (or None for both on a host-only pool).  Returns the slots."""
    def nbytes(t):
        if t is None:
            return 0
        return t.numel() * t.element_size() if hasattr(t, "element_size") else t.nbytes
    n = len(reqs)
    arr = (lora_page_in_req * max(n, 1))()
    any_host = False
    for k, (aid, rank, alpha, base, hA, hB) in enumerate(reqs):
        arr[k] = lora_page_in_req(aid, rank, alpha, 0, base, _addr(hA), nbytes(hA), _addr(hB), nbytes(hB))
        any_host = any_host or hA is not None
    slots = np.full(max(n, 1), -1, np.int32)
    _check(library().lora_pool_page_in_batch(pool.handle, n, ctypes.cast(arr, _VP), _stream(stream) if any_host else None,
                                             _i32p(slots)), "lora_pool_page_in_batch")
    return slots[:n]


def lora_pool_evict(pool: Pool, adapter_id: int) -> None:
    _check(library().lora_pool_evict(pool.handle, adapter_id), "lora_pool_evict")


def lora_pool_slot_of(pool: Pool, adapter_id: int) -> int:
    s = ctypes.c_int32()
    _check(library().lora_pool_slot_of(pool.handle, adapter_id, ctypes.byref(s)), "lora_pool_slot_of")
    return s.value


def lora_pool_slots_of(pool: Pool, adapter_ids) -> np.ndarray:
    ids = _i32(adapter_ids)
    out = np.empty_like(ids)
    _check(library().lora_pool_slots_of(pool.handle, ids.size, _i32p(ids), _i32p(out)), "lora_pool_slots_of")
    return out


def lora_pool_acquire(pool: Pool, slot: int) -> None:
    _check(library().lora_pool_acquire(pool.handle, slot), "lora_pool_acquire")


def lora_pool_release(pool: Pool, slot: int) -> None:
    _check(library().lora_pool_release(pool.handle, slot), "lora_pool_release")


def lora_pool_alloc_kv(pool: Pool, n_pages: int) -> np.ndarray:
    out = np.empty(max(n_pages, 0), np.int32)
    _check(library().lora_pool_alloc_kv(pool.handle, n_pages, _i32p(out)), "lora_pool_alloc_kv")
    return out


def lora_pool_free_kv(pool: Pool, pages) -> None:
    p = _i32(pages)
    _check(library().lora_pool_free_kv(pool.handle, p.size, _i32p(p)), "lora_pool_free_kv")


def lora_pool_slot_info(pool: Pool, slot: int):
    r, a, i = ctypes.c_int32(), ctypes.c_float(), ctypes.c_int32()
    _check(library().lora_pool_slot_info(pool.handle, slot, ctypes.byref(r), ctypes.byref(a), ctypes.byref(i)),
           "lora_pool_slot_info")
    return r.value, a.value, i.value


def lora_pool_page_table(pool: Pool, slot: int, layer: int, proj: int):
    rank, _, _ = lora_pool_slot_info(pool, slot)
    P = pool.desc.page_elems
    di, do = pool.desc.d_in[proj], pool.desc.d_out[proj]
    a = np.empty((rank, -(-di // P)), np.int32)
    b = np.empty((rank, -(-do // P)), np.int32)
    _check(library().lora_pool_page_table(pool.handle, slot, layer, proj, _i32p(a), _i32p(b)), "lora_pool_page_table")
    return a, b


def lora_pool_stats(pool: Pool):
    f, r, k = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int64()
    _check(library().lora_pool_stats(pool.handle, ctypes.byref(f), ctypes.byref(r), ctypes.byref(k)), "lora_pool_stats")
    return f.value, r.value, k.value


def lora_pool_free_list(pool: Pool) -> np.ndarray:
    n = ctypes.c_int64()
    _check(library().lora_pool_free_list(pool.handle, 0, None, ctypes.byref(n)), "lora_pool_free_list")
    out = np.empty(n.value, np.int32)
    _check(library().lora_pool_free_list(pool.handle, out.size, _i32p(out), ctypes.byref(n)), "lora_pool_free_list")
    return out


def lora_plan_create(pool: Pool, seg_start=None, seg_slot=None, token_slot=None, stream=None) -> Plan:
    ss, sl, ts = _i32(seg_start), _i32(seg_slot), _i32(token_slot)
    S = 0 if sl is None else sl.size
    nd = 0 if ts is None else ts.size
    h = _VP()
    st = _stream(stream) if pool.desc.meta_dev else None
    _check(library().lora_plan_create(pool.handle, _i32p(ss), _i32p(sl), S, _i32p(ts), nd, st, ctypes.byref(h)),
           "lora_plan_create")
    return Plan(h.value, pool)


def lora_plan_destroy(plan: Plan) -> None:
    if not plan.owned:
        raise ValueError("an engine step's plan is destroyed by lora_engine_step_done")
    if plan.handle:
        _check(library().lora_plan_destroy(plan.handle), "lora_plan_destroy")
        plan.handle = None


def lora_plan_groups(plan: Plan, n_decode: int):
    n = ctypes.c_int32()
    _check(library().lora_plan_groups(plan.handle, ctypes.byref(n), None, None, None, None), "lora_plan_groups")
    gs, gb, gc = (np.empty(n.value, np.int32) for _ in range(3))
    rows = np.empty(n_decode, np.int32)
    _check(library().lora_plan_groups(plan.handle, ctypes.byref(n), _i32p(gs), _i32p(gb), _i32p(gc), _i32p(rows)),
           "lora_plan_groups")
    return gs, gb, gc, rows


def lora_linear(pool: Pool, plan: Plan, layer: int, proj: int, x, w0, y, stream=None) -> None:
    _check(library().lora_linear(pool.handle, plan.handle, layer, proj, _addr(x), _addr(w0), _addr(y), _stream(stream)),
           "lora_linear")


def lora_linear_multi(pool: Pool, plan: Plan, layer: int, projs: Sequence[int], x, w0s, ys, stream=None) -> None:
    """Projections projs of one layer sharing x; w0s and ys per projection (w0s may be all None)."""
    n = len(projs)
    pr = _i32(projs)
    w = (_VP * n)(*[_addr(t) for t in w0s])
    yy = (_VP * n)(*[_addr(t) for t in ys])
    _check(library().lora_linear_multi(pool.handle, plan.handle, layer, n, _i32p(pr), _addr(x), w, yy,
                                       _stream(stream)), "lora_linear_multi")


def lora_linear_decode(pool: Pool, layer: int, proj: int, x, w0, y, token_slot, stream=None) -> None:
    ts = _i32(token_slot)
    _check(library().lora_linear_decode(pool.handle, layer, proj, _addr(x), _addr(w0), _addr(y), _i32p(ts), ts.size,
                                        _stream(stream)), "lora_linear_decode")


def lora_linear_decode_noalloc(pool: Pool, layer: int, proj: int, x, w0, y, token_slot, stream=None) -> None:
    ts = _i32(token_slot)
    _check(library().lora_linear_decode_noalloc(pool.handle, layer, proj, _addr(x), _addr(w0), _addr(y), _i32p(ts),
                                                ts.size, _stream(stream)), "lora_linear_decode_noalloc")


def lora_linear_prefill(pool: Pool, layer: int, proj: int, x, w0, y, seg_start, seg_slot, stream=None) -> None:
    ss, sl = _i32(seg_start), _i32(seg_slot)
    _check(library().lora_linear_prefill(pool.handle, layer, proj, _addr(x), _addr(w0), _addr(y), _i32p(ss), _i32p(sl),
                                         sl.size, _stream(stream)), "lora_linear_prefill")


def base_gemm_fp8(x, w0_code, w0_scale, y, M: int, N: int, K: int, stream=None) -> None:
    _check(library().base_gemm_fp8(_addr(x), _addr(w0_code), _addr(w0_scale), _addr(y), M, N, K, _stream(stream)),
           "base_gemm_fp8")


def lora_linear_fp8(pool: Pool, plan: Plan, layer: int, proj: int, x, w0_code, w0_scale, y, stream=None) -> None:
    _check(library().lora_linear_fp8(pool.handle, plan.handle, layer, proj, _addr(x), _addr(w0_code),
                                     _addr(w0_scale), _addr(y), _stream(stream)), "lora_linear_fp8")


def base_gemm(dtype: int, x, w0, y, M: int, N: int, K: int, stream=None) -> None:
    _check(library().base_gemm(dtype, _addr(x), _addr(w0), _addr(y), M, N, K, _stream(stream)), "base_gemm")


KERNEL_NAMES = ("gemm", "bgmv_shrink", "bgmv_expand", "sgmv_shrink", "sgmv_expand", "page_in", "gemm_bgmv_shrink",
                "page_in_batch")


def lora_pool_set_timing(pool: Pool, enable) -> None:
    _check(library().lora_pool_set_timing(pool.handle, int(enable)), "lora_pool_set_timing")


def lora_pool_timing(pool: Pool, kernel: int):
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(library().lora_pool_timing(pool.handle, kernel, ctypes.byref(ms), ctypes.byref(n)), "lora_pool_timing")
    return ms.value, n.value


def lora_version() -> str:
    return library().lora_version().decode()


# -- engine layer -----------------------------------------------------------------------------------

class Engine:
    """Owns a ``lora_engine*``; keeps its pool and storage callbacks alive.  The pool lists the
    handle: whichever of the two Python objects is finalized first, the engine is destroyed
    before the pool."""

    def __init__(self, handle: int, pool: Pool, keep: list):
        self.handle = handle
        self.pool = pool
        self._keep = keep
        pool.engines.add(handle)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _LIB is not None and h in self.pool.engines:
            self.pool.engines.discard(h)
            _LIB.lora_engine_destroy(h)
        self.handle = None


def lora_engine_create(pool: Pool, desc: lora_engine_desc, keep: list) -> Engine:
    h = _VP()
    _check(library().lora_engine_create(pool.handle, ctypes.byref(desc), ctypes.byref(h)), "lora_engine_create")
    return Engine(h.value, pool, keep + [desc])


def lora_engine_destroy(engine: Engine) -> None:
    h, engine.handle = engine.handle, None
    if h and h in engine.pool.engines:
        engine.pool.engines.discard(h)
        _check(library().lora_engine_destroy(h), "lora_engine_destroy")


def lora_engine_submit(engine: Engine, request_id: int, adapter_id: int, prompt_tokens: int,
                       max_new_tokens: int) -> None:
    _check(library().lora_engine_submit(engine.handle, request_id, adapter_id, prompt_tokens, max_new_tokens),
           "lora_engine_submit")


def lora_engine_cancel(engine: Engine, request_id: int) -> None:
    _check(library().lora_engine_cancel(engine.handle, request_id), "lora_engine_cancel")


def lora_engine_step(engine: Engine, stream=None):
    """-> (batch fields as a dict, Plan or None); the plan belongs to the engine."""
    b = lora_engine_batch()
    _check(library().lora_engine_step(engine.handle, _stream(stream), ctypes.byref(b)), "lora_engine_step")
    plan = Plan(b.plan, engine.pool, owned=False) if b.plan else None
    return {k: getattr(b, k) for k in ("n_requests", "n_prefill", "n_rows", "n_distinct")}, plan


def lora_engine_batch_requests(engine: Engine, n_requests: int):
    """-> (request ids int64, adapter ids int32, rows int32) of the current step, in row order."""
    ids = np.zeros(n_requests, np.int64)
    ads = np.zeros(n_requests, np.int32)
    rows = np.zeros(n_requests, np.int32)
    _check(library().lora_engine_batch_requests(engine.handle, ids.ctypes.data_as(_I64P), _i32p(ads), _i32p(rows)),
           "lora_engine_batch_requests")
    return ids, ads, rows


def lora_engine_step_done(engine: Engine) -> None:
    _check(library().lora_engine_step_done(engine.handle), "lora_engine_step_done")


def lora_engine_kv_pages(engine: Engine, request_id: int) -> np.ndarray:
    n = ctypes.c_int32()
    _check(library().lora_engine_kv_pages(engine.handle, request_id, 0, None, ctypes.byref(n)), "lora_engine_kv_pages")
    out = np.zeros(n.value, np.int32)
    _check(library().lora_engine_kv_pages(engine.handle, request_id, out.size, _i32p(out), ctypes.byref(n)),
           "lora_engine_kv_pages")
    return out


def lora_engine_get_stats(engine: Engine) -> dict:
    s = lora_engine_stats()
    _check(library().lora_engine_get_stats(engine.handle, ctypes.byref(s)), "lora_engine_get_stats")
    return {k: getattr(s, k) for k, _ in lora_engine_stats._fields_}


def lora_engine_reset_stats(engine: Engine) -> None:
    _check(library().lora_engine_reset_stats(engine.handle), "lora_engine_reset_stats")


def lora_probe_mfma(shape: int, iters: int, blocks: int, out, stream=None) -> float:
    """Launch the matrix-core probe (shape 16 or 32); returns the launch's flop count."""
    f = ctypes.c_double()
    _check(library().lora_probe_mfma(shape, iters, blocks, _addr(out), _stream(stream), ctypes.byref(f)),
           "lora_probe_mfma")
    return f.value


def lora_probe_read(buf, buf_bytes: int, chunk, n_chunks: int, out, stream=None) -> None:
    """Launch the read probe: wave w reads the 8 KiB chunk chunk[w] of buf (device buffers)."""
    _check(library().lora_probe_read(_addr(buf), buf_bytes, _addr(chunk), n_chunks, _addr(out), _stream(stream)),
           "lora_probe_read")
