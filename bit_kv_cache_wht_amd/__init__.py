"""UltraQuant FP4 KV-cache hot path for MI355X (gfx950).

Thin Python binding over the C ABI of ``libuq.so`` (declared in include/uq.h):
every function here only marshals torch tensors into pointers and sizes; all
computation runs in the HIP kernels.  Importing the package does not load the
library; the first call does, and raises if ``libuq.so`` is missing (build it
with ``python -m bit_kv_cache_wht_amd.build``).
"""
from ._binding import (  # noqa: F401
    UQ_CHECK_BAD_LEN,
    UQ_CHECK_BAD_PAGE,
    UQ_FLAG_CHECK,
    UQ_FLAG_OUT_ROTATED,
    UQ_FLAG_PV_SCALED,
    UQ_FLAG_SCALE_CONSTOPT,
    UQ_IN_BF16,
    UQ_IN_F32,
    UQ_KV_BF16,
    UQ_KV_FP4,
    UQ_KV_FP8,
    UQ_ROT_K_ONLY,
    UQ_ROT_SIGNS,
    KvCache,
    UqError,
    decode_check_word,
    lib,
    sign_words,
    uq_append_bf16,
    uq_append_fp8,
    uq_append_decode_attention,
    uq_decode_attention,
    uq_decode_attention_bf16,
    uq_decode_attention_fp8,
    uq_decode_attention_noalloc,
    uq_decode_workspace_bytes,
    uq_head_block_bytes,
    uq_last_hip_error,
    uq_page_bytes,
    uq_profile_next_decode,
    uq_profile_next_decode_clock,
    uq_stream_read,
    uq_prefill_attention,
    uq_quantize_append,
    uq_rotate_quantize_query,
    uq_rotate_quantize_query_cache,
    uq_status_string,
)
