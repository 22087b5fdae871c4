"""Seeded synthetic inputs shared by the parity tests, the benchmark and the oracle.

This package only *draws* inputs (weights, activations, upstream gradients and
outlier rows) and converts the float32 samples to bfloat16 bit patterns or to
per-tensor-scaled OCP FP8 codes. It holds none of the method's arithmetic: no
gradient, no optimizer, no rounding of results, no quantisation of states.
"""
from .inputs import (  # noqa: F401
    LayerSpec, WORKLOADS, bf16_bits_from_f32, f32_from_bf16_bits, draw_normal,
    draw_layer_init, draw_layer_batch, outlier_rows, sample_rows, layer_seed, llama8b_stack,
    draw_layer_batch_fp8, fp8_codes, FP8_MAX,
)
