"""fp64 CPU oracle for QSA — test infrastructure only (see qsa_oracle)."""
from .qsa_oracle import (  # noqa: F401
    attend,
    attend_rows,
    block_scores,
    candidate_blocks,
    compress_keys,
    decode,
    index_topk,
    num_complete_blocks,
    prefill,
    select_blocks,
    token_set,
    trailing_tokens,
)
