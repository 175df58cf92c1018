"""KVzip reconstruction-attention scoring, global selection and compaction on
MI355X (gfx950): a C-ABI HIP library (libkvz.so, include/kvz.h) and its
Python binding (kvz.py)."""
from .kvz import (KvzError, kvz_build_id, kvz_compact, kvz_compact_workspace, kvz_decode_packed,  # noqa: F401
                  kvz_decode_workspace, kvz_head_scores, kvz_keep_count, kvz_prof_enable,
                  kvz_prof_read, kvz_score_chunk, kvz_score_chunk_attn,
                  kvz_score_chunk_attn_workspace, kvz_score_chunk_ex, kvz_score_chunk_noalloc, kvz_score_chunk_workspace,
                  kvz_select_heads, kvz_select_heads_workspace, kvz_select_threshold,
                  kvz_select_tokens, kvz_select_tokens_workspace, kvz_select_workspace,
                  kvz_status_string,
                  kvz_token_scores)
