"""Seeded synthetic inputs for the KDA core (gated delta rule with per-channel decay).

This package only draws random inputs and converts between storage dtypes. It holds
none of the method's arithmetic: the recurrence, its chunked form and everything the
kernels compute live elsewhere. Both the CPU oracle's tests and the GPU path's tests and
benchmark draw their inputs from here, so the two sides always see identical values.
"""

from .gen import (  # noqa: F401
    ROOT_SEED,
    WORKLOADS,
    Workload,
    bf16_bits_to_f32,
    bf16_bits_to_f64,
    conv_params,
    conv_state,
    NORM_EPS,
    f64_to_bf16_bits,
    fused_slab,
    gate_params,
    grad_out,
    grad_state,
    initial_state,
    make_inputs,
    norm_weight,
    seq_lengths,
    slab,
    stored_to_f64,
)
