"""Seeded synthetic inputs shared by the CPU oracle checks, the GPU tests and the bench.

This package holds only random-number generation, bf16 bit conversion and tensor
assembly. It does none of the attention arithmetic, so the oracle and the HIP
path can both draw from it without sharing any of the method's code.
"""
from .inputs import (  # noqa: F401
    TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DO,
    bf16_bits_from_f32, f32_from_bf16_bits, normal_slice, bnhd_tensor,
    varlen_lengths, cu_seqlens_from_lengths, varlen_tensor, decode_query,
    paged_layout, paged_tensor, rademacher_signs, outlier_tensor,
)
