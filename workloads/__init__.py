"""Seeded synthetic inputs shared by the tests, the oracle checks and the bench."""
from .planted import (CHUNK_BF16_64K, FP8_128K, GQA_BF16_16K, PAGED_VARLEN, SHARD_BF16_16K, SWEEP_ALPHAS,
                      SWEEP_BF16_64K, TINY_F32, Inputs, Workload, generate_f32,
                      make_inputs, page_table, quantize_fp8)

__all__ = ["CHUNK_BF16_64K", "FP8_128K", "GQA_BF16_16K", "PAGED_VARLEN", "SHARD_BF16_16K", "SWEEP_ALPHAS",
           "SWEEP_BF16_64K",
           "TINY_F32", "Inputs", "Workload", "generate_f32", "make_inputs", "page_table",
           "quantize_fp8"]
