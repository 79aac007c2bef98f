"""QSA (Qwen Sparse Attention) for AMD MI355X: HIP kernels behind a C ABI.

The binding (``qsa``) loads ``libqsa.so`` lazily on first use and fails loudly
when it is missing; ``synth`` holds the seeded synthetic-input generators.
"""
from .qsa import (  # noqa: F401
    QSAError,
    compress_keys,
    decode,
    decode_workspace,
    decode_workspace_bytes,
    index_topk,
    lib,
    prefill,
    sparse_attn_decode,
    sparse_attn_prefill,
)
