"""TurboQuant key path on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/tq.h`` (libtq.so, built
in-tree by ``kv_cache_vector_rotate_amd.build``).  Every step of the path runs
in the library's HIP kernels; this module only checks tensors and passes
pointers, sizes and the current stream.  If the library is missing the calls
raise instead of falling back to anything else.
"""

from ._binding import (  # noqa: F401
    TQ_F32, TQ_BF16, TQError, Codebook, codebook_tables, encode_keys, append_keys, score_logits,
    score_cache, value_packed_nbytes, encode_values, attention_workspace_nbytes, attention_decode,
    score_topk, score_topk_workspace_nbytes, decode_mse, dense_logits_bf16, packed_nbytes,
    score_workspace_nbytes, rotation_dim, library, library_path, EXPORTED_SYMBOLS,
    clock_probe, stream_probe, score_stream_probe, attention_decode_noalloc,
    attention_noalloc_max_nbytes, paged_pool_nbytes, paged_append_keys, paged_score,
    append_values, attention_cache, paged_value_pool_nbytes, paged_append_values, paged_attention,
)
