"""Pins of the FP8-base oracle (``oracle.lora_linear_fp8base``, ``oracle.e4m3_value``).

The base weight is W0[n, k] = scale[n] * e4m3(code[n, k]), the reading of an
FP8 base with 16-bit adapters ("Multi-LoRA serving: S-LoRA, Punica and adapter
batching", Interaction with how the adapters were trained).  The checks tie it
to facts other than itself:

* decoded values derived by hand from the format's definition
  (tests/golden/e4m3_by_hand.json) and every code against torch's
  float8_e4m3fn conversion (a library routine for the same format);
* the codes' order: 0x00 .. 0x7E increasing, the negative half its mirror;
* with unit scales the FP8 base equals the bf16 oracle run on the decoded
  values written as bf16 (every E4M3 value is exact in bf16), bit for bit;
* a scale per output channel multiplies that channel's base output;
* the delta is the bf16 oracle's delta.
A mutation test plants mistakes in a copy of the oracle's FP8 code (the
exponent bias, the subnormals, the sign, the NaN code, the scale's index) and
checks that a pin rejects each.
"""
import json
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from workloads import bf16_bits_from_f32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "e4m3_by_hand.json")
torch = pytest.importorskip("torch")


def _same(a, b):
    return (np.isnan(a) and np.isnan(b)) or (a == b and np.signbit(a) == np.signbit(b))


def pin_golden(lib):
    g = json.load(open(GOLDEN))
    for c, v in zip(g["codes"], g["values"]):
        want = float("nan") if v == "nan" else float(v)
        got = oracle.e4m3_value(c, _lib_handle=lib)
        assert _same(got, want), f"code {c:#04x}: {got} != {want}"


def pin_library(lib):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        got = oracle.e4m3_value(c, _lib_handle=lib)
        assert _same(got, float(ref[c])), f"code {c:#04x}: {got} != {ref[c]}"


def pin_order(lib):
    pos = [oracle.e4m3_value(c, _lib_handle=lib) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:])), "codes 0x00..0x7E must increase"
    for c in range(0x7F):
        assert oracle.e4m3_value(c | 0x80, _lib_handle=lib) == -pos[c]


def _case(seed, T=7, d_in=40, d_out=24, ranks=(3, 1, 5)):
    g = np.random.default_rng(seed)
    codes = g.integers(0, 256, (d_out, d_in)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] ^= 0x01               # no NaN codes
    x = bf16_bits_from_f32(g.standard_normal((T, d_in)).astype(np.float32))
    ad = {}
    for i, r in enumerate(ranks):
        A = bf16_bits_from_f32(g.standard_normal((r, d_in)).astype(np.float32))
        B = bf16_bits_from_f32(g.standard_normal((r, d_out)).astype(np.float32))
        ad[10 + i] = (r, float(g.uniform(0.5, 8.0)), A, B)
    ra = g.choice([-1, 10, 11, 12], T)
    return x, codes, ad, ra


def pin_reduces_to_bf16(lib):
    x, codes, ad, ra = _case(1)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
    w_bf16 = vals.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(vals.numpy(), vals.to(torch.bfloat16).float().numpy())   # exact in bf16
    got = oracle.lora_linear_fp8base(x, codes, np.ones(codes.shape[0], np.float32), ra, ad, _lib_handle=lib)
    want = oracle.lora_linear(x, w_bf16, ra, ad)
    assert np.array_equal(got, want)


def pin_channel_scale(lib):
    x, codes, ad, ra = _case(2)
    g = np.random.default_rng(3)
    sc = g.uniform(1e-4, 3.0, codes.shape[0]).astype(np.float32)
    none = [-1] * x.shape[0]
    y1 = oracle.lora_linear_fp8base(x, codes, np.ones_like(sc), none, {}, _lib_handle=lib)
    ys = oracle.lora_linear_fp8base(x, codes, sc, none, {}, _lib_handle=lib)
    want = y1 * sc.astype(np.float64)[None, :]
    assert np.allclose(ys, want, rtol=1e-12, atol=1e-300)


def pin_delta(lib):
    x, codes, ad, ra = _case(4)
    sc = np.full(codes.shape[0], 0.01, np.float32)
    full = oracle.lora_linear_fp8base(x, codes, sc, ra, ad, _lib_handle=lib)
    base = oracle.lora_linear_fp8base(x, codes, sc, [-1] * x.shape[0], ad, _lib_handle=lib)
    delta = oracle.lora_linear(x, None, ra, ad)
    assert np.allclose(full - base, delta, rtol=1e-12, atol=1e-9)


FP8_PINS = [("golden", pin_golden), ("library", pin_library), ("order", pin_order),
            ("reduces_to_bf16", pin_reduces_to_bf16), ("channel_scale", pin_channel_scale), ("delta", pin_delta)]


@pytest.mark.parametrize("name,pin", FP8_PINS, ids=[n for n, _ in FP8_PINS])
def test_fp8_pin(name, pin):
    pin(None)


FP8_MUTANTS = {
    "bias_8": ("for (int i = 7; i < e; ++i) v *= 2.0;", "for (int i = 8; i < e; ++i) v *= 2.0;"),
    "subnormal_as_normal": ("} else if (e == 0) {", "} else if (e == 0 && 0) {"),
    "sign_dropped": ("return sign ? -v : v;", "return v;"),
    "nan_code_finite": ("if (e == 15 && m == 7) {", "if (e == 15 && m == 8) {"),
    "scale_by_input_index": ("const double sc = (double)w0_scale[n];", "const double sc = (double)w0_scale[0];"),
    "mantissa_shift": ("v = (1.0 + m / 8.0);", "v = (1.0 + m / 16.0);"),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_pins_reject_planted_mistake(name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = FP8_MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, f"{name}.c")
        open(path, "w").write(src.replace(old, new))
        lib_path = os.path.join(tmp, f"lib{name}.so")
        subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", path, "-o", lib_path], check=True)
        lib = oracle.load_library(lib_path)
        caught = []
        for pin_name, pin in FP8_PINS:
            try:
                pin(lib)
            except (AssertionError, ValueError):
                caught.append(pin_name)
        assert caught, f"no pin caught mutant {name}"
