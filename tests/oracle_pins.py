"""Pins of the LoRA-linear oracle: checks against facts other than the oracle.

Each check takes the oracle's ``lora_linear`` entry (so the mutation test can
run them against deliberately broken copies of the oracle) and raises
AssertionError when the oracle disagrees with:

* the base-only special case, which reduces to one library matmul;
* the merged-weight identity W' = W0 + gamma * B A ("Multi-LoRA serving:
  S-LoRA, Punica and adapter batching", "The bottleneck" section: a merged
  fine-tune serves the same function as base plus adapter);
* the delta as a sum over adapters of masked whole-matrix products (the
  looped per-adapter form that "Multi-LoRA serving: S-LoRA, Punica and
  adapter batching" measures in "Measured and simulated"): a different
  route to the same numbers;
* one-hot adapters, whose delta has a closed form by inspection;
* a hand-derived worked example (tests/golden/tiny_by_hand.json);
* exact invariances: row permutation, rows computed alone, row subsets;
* exact bf16 decoding of a few printed bit patterns.
"""
from __future__ import annotations

import json
import os

import numpy as np

from workloads import bf16_bits_from_f32, f32_from_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def random_case(seed=0, T=9, d_in=24, d_out=24, ranks=(3, 5, 1), bf16=False, null_frac=0.3):
    """Small random layer: adapters with random alpha (gamma != 2 on purpose)."""
    g = _rng(seed)

    def arr(*shape, std=1.0):
        v = (g.standard_normal(shape) * std).astype(np.float32)
        return bf16_bits_from_f32(v) if bf16 else v

    x = arr(T, d_in)
    w0 = arr(d_out, d_in, std=0.2)
    adapters = {}
    for i, r in enumerate(ranks):
        adapters[10 + i] = (r, float(g.uniform(0.5, 7.0)), arr(r, d_in, std=0.3), arr(r, d_out, std=0.3))
    ids = list(adapters)
    row_adapter = np.array([-1 if g.random() < null_frac else ids[g.integers(len(ids))] for _ in range(T)], np.int32)
    if not any(row_adapter >= 0):
        row_adapter[0] = ids[0]
    return x, w0, row_adapter, adapters


def _f64(a):
    a = np.asarray(a)
    return f32_from_bf16_bits(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _close(got, want, rel=1e-12):
    scale = max(1.0, float(np.max(np.abs(want)))) if want.size else 1.0
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert err <= rel * scale, f"max |err| {err:.3e} > {rel:.0e} x {scale:.3e}"


def pin_base_only(lora_linear, bf16=False):
    x, w0, _, adapters = random_case(1, bf16=bf16)
    T = x.shape[0]
    y = lora_linear(x, w0, [-1] * T, adapters)
    _close(y, _f64(x) @ _f64(w0).T)


def pin_merged_weight(lora_linear, bf16=False):
    x, w0, _, adapters = random_case(2, bf16=bf16)
    T = x.shape[0]
    for a, (r, alpha, A, B) in adapters.items():
        y = lora_linear(x, w0, [a] * T, adapters)
        merged = _f64(w0) + (alpha / r) * (_f64(B).T @ _f64(A))   # W' = W0 + gamma * B A, B as d_out x r
        _close(y, _f64(x) @ merged.T, rel=1e-11)


def pin_per_adapter_masked(lora_linear, bf16=False):
    """Route the delta through whole-matrix products, one adapter at a time:
    the delta of the batch is the sum over adapters a of
    gamma_a * M_a (X A_a^T) B_a, where the 0/1 diagonal M_a keeps the rows
    routed to a.  No per-row loop, no gather: a different route to the same
    numbers (the merged and looped-matmul forms the pages compare against)."""
    x, w0, row_adapter, adapters = random_case(3, T=17, bf16=bf16)
    got = lora_linear(x, w0, row_adapter, adapters)
    xs = _f64(x)
    routed = np.asarray(row_adapter)
    total = xs @ _f64(w0).T
    for a, (rank, alpha, A, B) in adapters.items():
        keep = (routed == a).astype(np.float64)[:, None]
        low = (keep * xs) @ _f64(A).T            # rows not routed to a give zero
        total = total + (alpha / rank) * (low @ _f64(B))
    _close(got, total, rel=1e-11)


def pin_one_hot(lora_linear):
    d_in, d_out, T = 7, 5, 4
    g = _rng(4)
    x = g.standard_normal((T, d_in)).astype(np.float32)
    w0 = np.zeros((d_out, d_in), np.float32)
    # rank 2: A row j picks input k_j, B row j writes output n_j
    ks, ns, alpha = (3, 6), (4, 1), 3.0
    A = np.zeros((2, d_in), np.float32)
    B = np.zeros((2, d_out), np.float32)
    for j in range(2):
        A[j, ks[j]] = 1.0
        B[j, ns[j]] = 1.0
    y = lora_linear(x, w0, [7] * T, {7: (2, alpha, A, B)})
    want = np.zeros((T, d_out))
    for j in range(2):
        want[:, ns[j]] += (alpha / 2) * x[:, ks[j]].astype(np.float64)
    _close(y, want)
    # and with no adapter the zero base stays exactly zero
    y0 = lora_linear(x, w0, [-1] * T, {7: (2, alpha, A, B)})
    assert np.all(y0 == 0.0)


def pin_golden_by_hand(lora_linear):
    with open(os.path.join(GOLDEN, "tiny_by_hand.json")) as f:
        g = json.load(f)
    x = np.array(g["x"], np.float32)
    w0 = np.array(g["w0"], np.float32)
    adapters = {int(k): (v["rank"], v["alpha"], np.array(v["A"], np.float32), np.array(v["B"], np.float32))
                for k, v in g["adapters"].items()}
    y = lora_linear(x, w0, g["row_adapter"], adapters)
    assert np.array_equal(y, np.array(g["y"], np.float64)), (y, g["y"])


def pin_invariances(lora_linear, bf16=False):
    x, w0, row_adapter, adapters = random_case(5, T=13, bf16=bf16)
    y = lora_linear(x, w0, row_adapter, adapters)
    perm = _rng(6).permutation(x.shape[0])
    yp = lora_linear(x[perm], w0, row_adapter[perm], adapters)
    assert np.array_equal(yp, y[perm]), "row permutation must permute outputs exactly"
    for t in range(x.shape[0]):
        y1 = lora_linear(x[t:t + 1], w0, row_adapter[t:t + 1], adapters)
        assert np.array_equal(y1[0], y[t]), "a row computed alone must equal its batched value"
    rows = [11, 0, 5, 5]
    ys = lora_linear(x, w0, row_adapter, adapters, rows=rows)
    assert np.array_equal(ys, y[rows])


def pin_bf16_decoding(lora_linear):
    # bf16 bit patterns with known values: 0x3F80 = 1, 0xC000 = -2, 0x3F81 = 1 + 2^-7, 0x0001 = 2^-133
    bits = np.array([[0x3F80, 0xC000, 0x3F81, 0x0001]], np.uint16)
    vals = np.array([1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133])
    w0 = np.zeros((4, 4), np.uint16)
    for n in range(4):
        w0[n, n] = 0x3F80
    y = lora_linear(bits, w0, [-1], {})
    assert np.array_equal(y[0], vals), y
    # and bf16 inputs give the same numbers as their exact fp32 images
    x, w, ra, ad = random_case(7, bf16=True)
    yb = lora_linear(x, w, ra, ad)
    ad32 = {a: (r, al, f32_from_bf16_bits(A), f32_from_bf16_bits(B)) for a, (r, al, A, B) in ad.items()}
    yf = lora_linear(f32_from_bf16_bits(x), f32_from_bf16_bits(w), ra, ad32)
    assert np.array_equal(yb, yf)


ALL_PINS = [
    ("base_only", lambda f: pin_base_only(f)),
    ("base_only_bf16", lambda f: pin_base_only(f, bf16=True)),
    ("merged_weight", lambda f: pin_merged_weight(f)),
    ("merged_weight_bf16", lambda f: pin_merged_weight(f, bf16=True)),
    ("per_adapter_masked", lambda f: pin_per_adapter_masked(f)),
    ("per_adapter_masked_bf16", lambda f: pin_per_adapter_masked(f, bf16=True)),
    ("one_hot", pin_one_hot),
    ("golden_by_hand", pin_golden_by_hand),
    ("invariances", lambda f: pin_invariances(f)),
    ("bf16_decoding", pin_bf16_decoding),
]
