"""CPU oracle for MSA: test infrastructure only (see msa_oracle.py)."""
from .msa_oracle import *  # noqa: F401,F403
from .msa_oracle import (attend, block_partials, block_score, index_scores, kv_block_major_lists, lse_merge,  # noqa: F401
                         num_candidates, paged_decode_attention, request_tokens, selected_kv,
                         sparse_attention, sparse_page_table, topk_blocks, valid_token_count)
