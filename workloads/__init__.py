"""Seeded synthetic workloads for the bandwidth-bound batch-1 decode step.

This module fixes the shapes of the five workloads and generates, from seeds,
everything a decode run consumes: weight tensors, prompt token ids, first
tokens and pre-filled KV-cache values.  The reference decoder (``oracle/``),
the tests and the benchmark all draw their inputs from here, so both sides of
every parity check see identical bits.  Nothing in this package computes any
part of the decode step itself.

The pages describe no trained model that could be run here: the Kog engine's
2B technical-preview model and the 11B full-duplex voice model are not
available, and the pages measure on no public dataset.  Every workload is
therefore a random-init decoder of the stated shape fed with uniform random
token ids, which is what the bytes-per-token accounting of the pages needs
(each token reads every weight and the whole KV cache, per "Kog 3000 tok/s
real-time inference: memory-bandwidth optimisation and request-level
concurrency trade-offs", section "three-layer strategy").
"""

from .presets import ModelShape, Workload, PRESETS, get, TENSORS_PER_LAYER, LAYER_TENSOR_NAMES
from .gen import (
    make_weights,
    make_prompt,
    make_first_tokens,
    kv_prefill_block,
    fill_kv_prefill,
    fill_kv_prefill_device,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    Fp8Matrix,
    quantize_rows_e4m3,
    E4M3_MAX,
    Int8Matrix,
    quantize_rows_int8,
    INT8_MAX,
)

__all__ = [
    "ModelShape",
    "Workload",
    "PRESETS",
    "get",
    "TENSORS_PER_LAYER",
    "LAYER_TENSOR_NAMES",
    "make_weights",
    "make_prompt",
    "make_first_tokens",
    "kv_prefill_block",
    "fill_kv_prefill",
    "fill_kv_prefill_device",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "Fp8Matrix",
    "quantize_rows_e4m3",
    "E4M3_MAX",
    "Int8Matrix",
    "quantize_rows_int8",
    "INT8_MAX",
]
