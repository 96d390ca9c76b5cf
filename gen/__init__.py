"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package draws random numbers and lays them out; it performs none of the
Sketch&Walk arithmetic (no block means, no Hadamard transform, no walk, no
selection, no attention).  Both the CPU oracle and the HIP path consume the
tensors it returns.
"""
from .synth import (  # noqa: F401
    CONFIGS,
    Config,
    hadamard_tables,
    layer_inputs,
    seq_tensor,
    block_latents,
    decode_layer_inputs,
    seed_for,
    ragged_lengths,
    cu_offsets,
    page_table,
    to_fp8_e4m3,
)
