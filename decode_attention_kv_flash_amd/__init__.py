"""MI355X-native single-token decode attention over a KV cache.

The compute lives in hand-written HIP kernels for gfx950 behind the C ABI of
``libdattn.so`` (include/dattn.h); ``api`` is the thin Python binding.
"""
from .api import (  # noqa: F401
    DattnError, decode_attn_gqa, decode_attn_mla, decode_attn_quest, dsa_indexer_topk, dsa_topk,
    kv_append_gqa, kv_append_rows, profile_enable, profile_read, profile_reset, quest_page_minmax,
    sparse_mla_attn,
)
