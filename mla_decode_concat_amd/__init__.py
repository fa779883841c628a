"""Fused MLA decode epilogue for AMD MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI of
include/mla_dq.h (the epilogue) and include/mla_attn.h (the decode attention
that consumes its output), both in libmla_dq.so; this package is their Python
binding.
"""
from ._binding import (  # noqa: F401
    ROPE, Q_FP8, KV_FP8, FP16, ROPE_GPTJ, TABLE_BF16, FORCE_SMALL_T, FORCE_LARGE_T, FORCE_STREAM, FORCE_CACHED,
    FORCE_MID_T, Q_ROWS_ONLY, CACHE_ROWS_ONLY,
    MlaDqError, Dims, LaunchPlan, fused_mla_decode_q_concat_kv_cache_insert,
    mla_decode_q_concat_kv_insert, PreparedInsert, plan, strerror, load,
    UkLaunchPlan, uk_plan, mla_decode_uk_q_concat_kv_insert, PreparedUkInsert,
    ATTN_Q_FP8, ATTN_KV_FP8, AttnDims, AttnPlan, PreparedAttention, attn_plan,
    attn_workspace_size, mla_decode_attention, mla_decode_attention_noalloc,
)
