"""MI355X (gfx950) KV-cache attention: split-KV decode (plain, with the
current token's cache append, with the rotary embedding in that append, or
over a paged cache), causal prefill against a cached prefix (contiguous or
paged), and top-k sparse scores (encoder and decoder-causal forms), as
hand-written HIP kernels behind a C ABI (``include/attn.h``), plus a
streaming-read probe that measures attainable read bandwidth. This package is
the thin Python binding.
"""
from ._binding import (  # noqa: F401
    ATTN_BF16,
    ATTN_E_ARG,
    ATTN_E_HIP,
    ATTN_E_UNSUPPORTED,
    ATTN_E_WORKSPACE,
    ATTN_F32,
    ATTN_OK,
    EXPORTED,
    LIB_PATH,
    AttnArgError,
    AttnError,
    attn_decode,
    attn_decode_append,
    attn_decode_append_rope,
    attn_decode_noalloc,
    attn_decode_paged,
    attn_decode_workspace_bytes,
    attn_prefill,
    attn_prefill_paged,
    attn_topk,
    attn_topk_causal,
    attn_read_probe,
    lib,
)

__all__ = ["attn_decode", "attn_decode_noalloc", "attn_decode_append",
           "attn_decode_append_rope",
           "attn_decode_paged",
           "attn_prefill", "attn_prefill_paged", "attn_topk", "attn_topk_causal",
           "attn_decode_workspace_bytes", "attn_read_probe", "AttnError",
           "AttnArgError"]
