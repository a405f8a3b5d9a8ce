"""Oracle for the multi-adapter LoRA-linear path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this package; the
product library (``heterogeneous_adapter_gemm_amd``) never does, and this
package imports nothing from it.

Parts:
  * ``lora_linear`` - the floating-point result, plain fp64 loops in C
    (``lora_oracle.c``), read from the logical dense adapters, never from the
    page pool; ``lora_linear_fp8base`` the same with the base weight given as
    E4M3 codes and a scale per output channel, ``e4m3_value`` the decoding of
    one code;
  * ``pool_model``  - the integer side: free list, slot and page tables of
    the unified page pool, and the expected bytes of every page;
  * ``index_model`` - the per-batch index: token -> slot, prefill segments and
    the grouping of decode rows by adapter.

Each function cites the passage of the pages it follows.  Pins (tests that
tie the oracle to facts other than itself) live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from . import build as _build

_LIB: Optional[ctypes.CDLL] = None


def load_library(path: str) -> ctypes.CDLL:
    """Load an oracle library built from ``lora_oracle.c`` (or a test's mutant of it)."""
    lib = ctypes.CDLL(path)
    lib.oracle_lora_linear.restype = ctypes.c_int
    lib.oracle_lora_linear.argtypes = [
        ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
    lib.oracle_lora_linear_fp8base.restype = ctypes.c_int
    lib.oracle_lora_linear_fp8base.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    return lib


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        _LIB = load_library(_build.LIB)
    return _LIB


def set_threads(n: int) -> None:
    _lib().oracle_set_threads(int(n))


def num_threads() -> int:
    return int(_lib().oracle_num_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def lora_linear(x: np.ndarray, w0: Optional[np.ndarray], row_adapter: Sequence[int],
                adapters: Dict[int, Tuple[int, float, np.ndarray, np.ndarray]],
                rows: Optional[Sequence[int]] = None, _lib_handle: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """Multi-adapter LoRA-linear output in fp64.

    ``x`` [T, d_in] and ``w0`` [d_out, d_in] (or None: base term zero) are
    float32 arrays or uint16 bf16 bit patterns; ``row_adapter[t]`` is an
    adapter id or -1; ``adapters[id] = (rank, alpha, A [r, d_in], B [r, d_out])``
    in the same element type.  Returns y [len(rows), d_out] (all rows if
    ``rows`` is None).  Follows "S-LoRA: Serving Thousands of Concurrent
    Adapters in 2026" (LoRA formula with scale alpha / r; the Step 2 per-row
    loop that skips rows with no adapter) and "Multi-LoRA serving: S-LoRA,
    Punica and adapter batching" (shrink then expand, "How the kernels work").
    """
    x = np.ascontiguousarray(x)
    bf16 = x.dtype == np.uint16
    if not bf16 and x.dtype != np.float32:
        raise TypeError("x must be float32 or uint16 (bf16 bits)")
    T, d_in = x.shape
    if w0 is not None:
        w0 = np.ascontiguousarray(w0)
        if w0.dtype != x.dtype or w0.shape[1] != d_in:
            raise ValueError("w0 must be [d_out, d_in] of x's element type")
        d_out = w0.shape[0]
    else:
        d_out = None
    ids = sorted(adapters)
    index = {a: i for i, a in enumerate(ids)}
    ranks = np.array([adapters[a][0] for a in ids], np.int32)
    alphas = np.array([adapters[a][1] for a in ids], np.float64)
    As, Bs, a_off, b_off = [], [], [], []
    oa = ob = 0
    for a in ids:
        r, _, A, B = adapters[a]
        A = np.ascontiguousarray(A)
        B = np.ascontiguousarray(B)
        if A.shape != (r, d_in) or A.dtype != x.dtype:
            raise ValueError(f"adapter {a}: A must be [{r}, {d_in}]")
        if d_out is None:
            d_out = B.shape[1]
        if B.shape != (r, d_out) or B.dtype != x.dtype:
            raise ValueError(f"adapter {a}: B must be [{r}, {d_out}]")
        As.append(A.reshape(-1)); Bs.append(B.reshape(-1))
        a_off.append(oa); b_off.append(ob)
        oa += A.size; ob += B.size
    if d_out is None:
        raise ValueError("d_out unknown: give w0 or at least one adapter")
    A_all = np.concatenate(As) if As else np.zeros(1, x.dtype)
    B_all = np.concatenate(Bs) if Bs else np.zeros(1, x.dtype)
    ra = np.array([index[int(a)] if int(a) >= 0 else -1 for a in row_adapter], np.int32)
    if ra.shape[0] != T:
        raise ValueError("row_adapter must have one entry per row")
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n_rows = T if rows_arr is None else rows_arr.shape[0]
    y = np.empty((n_rows, d_out), np.float64)
    lib = _lib() if _lib_handle is None else _lib_handle
    rc = lib.oracle_lora_linear(
        int(bf16), T, d_in, d_out, _ptr(x), _ptr(w0), _ptr(ra), len(ids), _ptr(ranks), _ptr(alphas),
        _ptr(np.array(a_off, np.int64)), _ptr(np.array(b_off, np.int64)), _ptr(A_all), _ptr(B_all),
        _ptr(rows_arr), n_rows, _ptr(y))
    if rc != 0:
        raise ValueError("oracle_lora_linear rejected its arguments")
    return y


def e4m3_value(code: int, _lib_handle: Optional[ctypes.CDLL] = None) -> float:
    """Value of one 8-bit E4M3 code (sign, 4 exponent bits with bias 7, 3
    mantissa bits; subnormals m * 2^-9; all-ones exponent and mantissa is NaN,
    no infinities): the FP8 reading of "Multi-LoRA serving: S-LoRA, Punica and
    adapter batching", section "Interaction with how the adapters were trained"."""
    lib = _lib() if _lib_handle is None else _lib_handle
    return float(lib.oracle_e4m3_value(int(code)))


def lora_linear_fp8base(x: np.ndarray, w0_code: np.ndarray, w0_scale: np.ndarray, row_adapter: Sequence[int],
                        adapters: Dict[int, Tuple[int, float, np.ndarray, np.ndarray]],
                        rows: Optional[Sequence[int]] = None, _lib_handle: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """Multi-adapter LoRA-linear with an FP8 base, in fp64: the base weight is
    W0[n, k] = w0_scale[n] * e4m3(w0_code[n, k]) (codes uint8 [d_out, d_in],
    scales float32 [d_out]); x [T, d_in] and the adapters are bf16 bit
    patterns (uint16) as in ``lora_linear``.  Follows "Multi-LoRA serving:
    S-LoRA, Punica and adapter batching" ("Interaction with how the adapters
    were trained": a quantized base served with 16-bit adapters) and the
    LoRA-linear of ``lora_linear``."""
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("x must be bf16 bit patterns (uint16)")
    w0_code = np.ascontiguousarray(w0_code)
    w0_scale = np.ascontiguousarray(w0_scale, dtype=np.float32)
    T, d_in = x.shape
    if w0_code.dtype != np.uint8 or w0_code.ndim != 2 or w0_code.shape[1] != d_in:
        raise ValueError("w0_code must be uint8 [d_out, d_in]")
    d_out = w0_code.shape[0]
    if w0_scale.shape != (d_out,):
        raise ValueError("w0_scale must be [d_out]")
    ids = sorted(adapters)
    index = {a: i for i, a in enumerate(ids)}
    ranks = np.array([adapters[a][0] for a in ids], np.int32)
    alphas = np.array([adapters[a][1] for a in ids], np.float64)
    As, Bs, a_off, b_off = [], [], [], []
    oa = ob = 0
    for a in ids:
        r, _, A, B = adapters[a]
        A, B = np.ascontiguousarray(A), np.ascontiguousarray(B)
        if A.shape != (r, d_in) or B.shape != (r, d_out) or A.dtype != np.uint16 or B.dtype != np.uint16:
            raise ValueError(f"adapter {a}: A [{r}, {d_in}] and B [{r}, {d_out}] must be bf16 bits")
        As.append(A.reshape(-1)); Bs.append(B.reshape(-1))
        a_off.append(oa); b_off.append(ob)
        oa += A.size; ob += B.size
    A_all = np.concatenate(As) if As else np.zeros(1, np.uint16)
    B_all = np.concatenate(Bs) if Bs else np.zeros(1, np.uint16)
    ra = np.array([index[int(a)] if int(a) >= 0 else -1 for a in row_adapter], np.int32)
    if ra.shape[0] != T:
        raise ValueError("row_adapter must have one entry per row")
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n_rows = T if rows_arr is None else rows_arr.shape[0]
    y = np.empty((n_rows, d_out), np.float64)
    lib = _lib() if _lib_handle is None else _lib_handle
    rc = lib.oracle_lora_linear_fp8base(
        T, d_in, d_out, _ptr(x), _ptr(w0_code), _ptr(w0_scale), _ptr(ra), len(ids), _ptr(ranks), _ptr(alphas),
        _ptr(np.array(a_off, np.int64)), _ptr(np.array(b_off, np.int64)), _ptr(A_all), _ptr(B_all),
        _ptr(rows_arr), n_rows, _ptr(y))
    if rc != 0:
        raise ValueError("oracle_lora_linear_fp8base rejected its arguments")
    return y
