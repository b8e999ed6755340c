"""Lossless compressed-KV decode attention for AMD MI355X (gfx950).

The compute path is the HIP library libkvz.so (C ABI in include/kvz.h); `kvz` is its thin Python
binding. Importing this package does not load the library; the first call does, and raises when
the library is not built.
"""
from . import kvz  # noqa: F401
from .kvz import (FORMAT_CHANNEL, FORMAT_ESCAPE, FORMAT_ZIPFUSION, Cache, KvzError, append_token,  # noqa: F401
                  chosen_pages_per_split, chosen_split, compact_pool, compress_pages, decode_attention,
                  decode_attention_noalloc,
                  decode_attention_dense, decode_attention_dense_splits, decode_attention_splits,
                  decompress_pages, merge_splits, inline_capacity, meta_bytes, num_splits, payload_bytes, unit_bytes,
                  workspace_bytes, PreparedAttention, prepare_decode_attention, prepare_decode_attention_dense,
                  PreparedAppend, prepare_append_token)
