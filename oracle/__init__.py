"""Plain, slow, float64 CPU oracle for FlashPrefill / FlashPrefill V2 block-sparse
prefill attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test suite, the smoke check of the
package entry and the CPU-baseline leg of the benchmark use it.  It shares no
code with the HIP library and imports nothing from it.

Every function follows the steps the pages state, in their order and notation,
with numpy float64 arithmetic; matrix products (`@`) are the only library
primitive used.  See `flashprefill.py` for the step-by-step citations and
`fp8.py` for the e4m3 decoder used to read fp8 inputs and the encoder of the
online per-tensor quantisation, and `fp8_attention.py` for the FP8 arithmetic
of the attention (e4m3 probabilities against the running maximum, the 2^8
offset, quantised pooled statistics).

Pinned by the `-m "not gpu"` tests in `tests/test_oracle_pins.py`.  One part is
"parity unpinned": the absolute accuracy of the fp8 path against the pages'
model-level tables (their Tab. 8/9) needs model weights and datasets that do
not exist here; only the arithmetic identities of the fp8 path are pinned.
"""
from .flashprefill import (attend_rows, block_scores_row, dense_causal_reference,
                           forced_blocks, merge_partials, n_blocks, packgqa_rows,
                           pool_means, request_oracle, select_row, tile_query_rows,
                           todo_row, wasted_row_fraction)
from .fp8 import decode_e4m3fn, encode_e4m3fn, quantize_per_tensor
from .fp8_attention import attend_rows_fp8, e4m3_round, pooled_code_means, walk

__all__ = ["attend_rows", "block_scores_row", "dense_causal_reference", "forced_blocks",
           "merge_partials", "n_blocks", "packgqa_rows", "pool_means", "request_oracle",
           "select_row", "tile_query_rows", "todo_row", "wasted_row_fraction",
           "decode_e4m3fn", "encode_e4m3fn", "quantize_per_tensor", "attend_rows_fp8",
           "e4m3_round", "pooled_code_means", "walk"]
