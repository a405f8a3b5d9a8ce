"""Seeded synthetic workloads for the multi-adapter LoRA-linear path.

This package only *generates data*: tensor shapes, value distributions,
adapter popularity, request mixes and the pool's physical page order.  It
contains none of the method's arithmetic.  Both the oracle (``oracle/``) and
the GPU path read the arrays it produces; neither is imported here.
"""
from .gen import (  # noqa: F401
    CONFIG_NAMES,
    AdapterSpec,
    Request,
    Workload,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make_workload,
    zipf_probs,
)
