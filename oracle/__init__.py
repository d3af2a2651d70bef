"""fp64 CPU oracle for KV-cache attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library and its Python binding
never import it, and it imports nothing from them.
"""
from .attention import (  # noqa: F401
    default_scale,
    decode,
    decode_append,
    decode_append_rope,
    decode_paged,
    decode_sequence,
    gather_pages,
    prefill,
    prefill_paged,
    rope_rotate,
    round_to_storage,
    topk_causal_select,
    topk_causal_sparse,
    topk_sparse,
    topk_scores,
    topk_select,
)
