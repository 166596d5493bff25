"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This package holds no arithmetic of the attention method itself: it draws
random tensors, rotates them with RoPE (the library takes already-rotated
inputs), plants structure, and rounds once to the storage dtype.
"""
from .workloads import (  # noqa: F401
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    rope,
    storage_to_f64,
    tiny_decode,
    gqa_decode,
    dlm_denoise,
    dlm_denoise_steps,
    sparse_prefill,
    threshold_prefill,
    threshold_decode,
    decode_rows,
    decode_batch_shifts,
    shift_sequence,
)
