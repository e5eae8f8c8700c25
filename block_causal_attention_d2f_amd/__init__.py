"""block_causal_attention_d2f_amd: the hot path of one D2F denoising step on
MI355X (gfx950), as a C-ABI HIP library (libd2f.so, see include/d2f.h) with a
thin ctypes binding.

    d2f_block_attn          block-causal attention of the active window
    d2f_confidence_commit   max-probability confidence + commit/remask
    d2f_kv_commit           append a completed block to the KV cache
    Window                  the active-window schedule (host)
    d2f_decode_advance      one step's bookkeeping after the commit pass
    d2f_block_attn_paged    attention over a paged cache (one page per block)
    d2f_kv_commit_paged     persist a block by moving its page into the table
    d2f_block_attn_range    the window over a cache key range (outside-block part)
    d2f_attn_combine        exact log-space join of two attention results
    d2f_confidence_commit_noalloc  the commit pass without a workspace argument
"""
from ._binding import (d2f_attn_combine, d2f_block_attn_range,  # noqa: F401
                       AGGRESSIVE, COMMITTED, CONSERVATIVE, D2F_BF16, D2F_F32, EXPORTS,  # noqa: F401
                       LIB_PATH, MASKED, AttnDesc, D2FError, Window, d2f_block_attn,
                       d2f_block_attn_paged, d2f_block_attn_workspace_size, d2f_confidence_commit,
                       d2f_confidence_commit_noalloc, d2f_confidence_commit_workspace_size, d2f_decode_advance,
                       d2f_decode_advance_paged,
                       d2f_kv_commit, d2f_kv_commit_paged, load, make_desc, prophet_threshold,
                       version)
