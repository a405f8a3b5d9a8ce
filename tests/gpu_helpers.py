"""Shared helpers of the GPU tests (not collected)."""
from __future__ import annotations

import numpy as np

TOL = 2e-2  # max |err| <= TOL * RMS(oracle output), bf16 in / fp32 accumulate


def to_np(t):
    """torch tensor (bf16 or fp32, any device) -> float64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(t):
    """Raw element bits of a tensor as a numpy integer array (for bitwise checks)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().copy()
    return t.view(torch.int32).numpy().copy()


def parity(got: np.ndarray, want: np.ndarray, tol: float = TOL, what: str = ""):
    rms = float(np.sqrt(np.mean(want ** 2)))
    err = float(np.max(np.abs(got - want)))
    print(f"[parity] {what} max|err| {err:.4e}  rms {rms:.4e}  ratio {err / max(rms, 1e-300):.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= tol * rms, f"{what}: max|err| {err:.4e} > {tol} x RMS {rms:.4e}"
    return err / rms


def bf16_bits(v: np.ndarray) -> np.ndarray:
    from workloads import bf16_bits_from_f32
    return bf16_bits_from_f32(v.astype(np.float32))
