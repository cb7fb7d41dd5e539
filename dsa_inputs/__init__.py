"""Seeded synthetic workloads for the DSA hot path (input generation only)."""
from .configs import WORKLOADS, Workload, get, visible  # noqa: F401
from .generate import (  # noqa: F401
    DecodeInputs, PrefillInputs, bf16_bits_to_f32, decode_inputs, decode_lengths,
    prefill_inputs, quantize_fp8_rows, to_bf16_bits,
)
