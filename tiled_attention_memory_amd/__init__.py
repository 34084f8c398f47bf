"""Exact causal GQA attention for MI355X (gfx950): HIP kernels behind a C ABI.

The Python names mirror include/attn.h, include/attn_block.h, include/attn_decode.h and
include/attn_dropout.h. The library is loaded on first use
and every call fails loudly if it is missing; nothing here computes attention.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    STATUS,
    BWD_EVENTS,
    MAX_MERGE,
    AttnError,
    attn_bwd_block_begin,
    attn_bwd_block_dkdv,
    attn_bwd_block_dq,
    attn_bwd_block_dq_end,
    attn_bwd_block_workspace_bytes,
    attn_decode,
    attn_decode_workspace_bytes,
    attn_bwd_dropout,
    attn_fwd_dropout,
    attn_fwd_block,
    attn_merge,
    attn_bwd,
    attn_bwd_raw,
    attn_bwd_workspace_bytes,
    attn_fwd,
    attn_fwd_raw,
    attn_status_string,
    attn_version,
    backward,
    forward,
    load,
    workspace_for,
)
