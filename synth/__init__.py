"""Seeded synthetic inputs shared by the oracle side and the GPU side (no attention arithmetic)."""
from .inputs import (bf16_bits_to_f32, f32_to_bf16_bits, host_threads, make_log_sizes, make_qkv, sample_rows,
                     tokens_per_frame)

__all__ = ["bf16_bits_to_f32", "f32_to_bf16_bits", "host_threads", "make_log_sizes", "make_qkv", "sample_rows",
           "tokens_per_frame"]
