"""Seeded synthetic inputs shared by the oracle tests, the HIP parity tests
and the benchmark.  This package holds input generation only: none of the
attention arithmetic lives here."""
from .workloads import (  # noqa: F401
    PagedBatch, MlaBatch, f32_to_bf16_bits, f32_to_f16_bits, bf16_bits_to_f32,
    config_tiny_f32_decode, config_bf16_decode_batch, config_bf16_chunked_prefill,
    config_bf16_mixed_batch, config_bf16_mla_decode, config_bf16_mla_decode_h128, config_bf16_mla_chunked_prefill, config_bf16_chunked_prefill_d192,
    config_bf16_chunked_prefill_d256, CONFIGS, random_batch, random_mla_batch,
    with_shared_pages,
)
