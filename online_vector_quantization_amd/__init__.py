"""TurboQuant KV-cache compression for AMD MI355X (gfx950).

The compute path lives in libtq.so (hand-written HIP kernels behind a C ABI,
include/tq.h); this package is its thin Python binding.
"""
from .api import (  # noqa: F401
    EXPORTED, LIB_PATH, TQ_BF16, TQ_F32, Codebook, CompressedCache, TQError, alloc_workspace, append_decode,
    alloc_chunk_workspace, attention_logits, chunk_attention, chunk_workspace_bytes,
    compressed_bytes_per_token, decode_attention, decode_attention_static, decode_workspace_bytes, encode_into_cache, encode_kv,
    load_library,
)
