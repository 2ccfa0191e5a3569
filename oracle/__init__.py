"""CPU oracle for gated block-sparse prefill attention: test infrastructure only.

Importable only from the test suite, the entry point's smoke check and the benchmark's CPU
baseline. The product path (block_sparse_long_amd) never imports it.
"""
from .bsfa_oracle import (GATE_ABSOLUTE, GATE_DENSE, GATE_RELATIVE, OracleResult, calibrate,
                          gather_pages,
                          effective_threshold, key_block_range, kth_highest, num_blocks,
                          off_diagonal_block_maxima, oracle_prefill, oracle_prefill_varlen,
                          quantize_e4m3, quantize_k_tiles, quantize_q_rows)

__all__ = ["GATE_ABSOLUTE", "GATE_DENSE", "GATE_RELATIVE", "OracleResult", "calibrate",
           "gather_pages",
           "effective_threshold", "key_block_range", "kth_highest", "num_blocks",
           "off_diagonal_block_maxima", "oracle_prefill", "oracle_prefill_varlen",
           "quantize_e4m3", "quantize_k_tiles", "quantize_q_rows"]
