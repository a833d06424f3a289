"""fp64 CPU oracle of the Ulysses per-rank hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path. It shares no code
with the HIP library.
"""
from .ulysses_oracle import *  # noqa: F401,F403
from .ulysses_oracle import (attn_bwd_block_sparse, attn_bwd_block_sparse_head, attn_fwd_block_sparse,  # noqa: F401
                             attn_fwd_block_sparse_head, attn_rows_block_sparse, block_visible, attn_dkv_cols_block_sparse,
                             attn_abs_sums_block_sparse_head, attn_abs_sums_head, attn_bwd, attn_bwd_gqa, attn_bwd_head, attn_fwd_gqa, check_gqa,
                             head_to_seq_kv_grad, kv_replication, seq_to_head_kv, attn_dkv_cols, attn_fwd,  # noqa: F401
                             attn_fwd_head, attn_rows, bf16_bits_to_f64, check_divisible,
                             error_stats, head_to_seq, head_to_seq_part, head_to_seq_source_rows,
                             monolithic_attention_fwd, seq_to_head, seq_to_head_part,
                             seq_to_head_source_rows, to_f64, ulysses_attention_fwd)
