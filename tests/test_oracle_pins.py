"""The oracle against its pins, and the pins against planted mistakes.

The mutation test copies ``oracle/lora_oracle.c`` to a temporary directory,
plants one plausible mistake (a dropped scale, a sign, a transposed operand,
a wrong shift in the bf16 decode, an off-by-one in the null test), builds it
with gcc and checks that at least one pin rejects it.  The oracle itself is
never modified.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("name,pin", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_pin(name, pin):
    pin(oracle.lora_linear)


MUTANTS = {
    "gamma_without_divide": ("alpha[a] / (double)r", "alpha[a]"),
    "delta_sign": ("yrow[n] += gamma * s", "yrow[n] -= gamma * s"),
    "w0_transposed": ("load_elem(w0, bf16, n * d_in + k)", "load_elem(w0, bf16, k * d_out + n)"),
    "b_transposed": ("b_off[a] + (int64_t)j * d_out + n", "b_off[a] + (int64_t)n * r + j"),
    "a_transposed": ("a_off[a] + (int64_t)j * d_in + k", "a_off[a] + (int64_t)k * r + j"),
    "bf16_shift": ("<< 16;", "<< 15;"),
    "adapter_zero_is_null": ("if (a < 0) continue;", "if (a <= 0) continue;"),
    "shrink_uses_wrong_row": ("* load_elem(x, bf16, xo + k);", "* load_elem(x, bf16, k);"),
}


def _build_mutant(tmp, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(tmp, f"lib{name}.so")
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", path, "-o", lib], check=True)
    return oracle.load_library(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTANTS[name]
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build_mutant(tmp, name, old, new)

        def mutant(*args, **kw):
            return oracle.lora_linear(*args, _lib_handle=lib, **kw)

        caught = []
        for pin_name, pin in ALL_PINS:
            try:
                pin(mutant)
            except (AssertionError, ValueError):
                caught.append(pin_name)
        assert caught, f"no pin caught mutant {name}"


def test_rows_out_of_range_rejected():
    x = np.zeros((2, 3), np.float32)
    w0 = np.zeros((3, 3), np.float32)
    with pytest.raises(ValueError):
        oracle.lora_linear(x, w0, [-1, -1], {}, rows=[2])
