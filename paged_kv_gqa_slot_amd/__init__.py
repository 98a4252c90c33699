"""Paged grouped-query attention over a block-allocated KV cache, for MI355X.

The compute lives in ``libfe.so`` (hand-written HIP for gfx950 behind a C ABI
declared in ``include/fe.h``).  :mod:`.binding` marshals torch tensors into
those calls; the library is loaded on first use and a missing or unbuilt
library is an error -- there is no CPU fallback.
"""
from .binding import (  # noqa: F401
    KVAllocator,
    fe_hbm_read_probe,
    fe_mfma_rate_probe,
    fe_kv_allocator_append,
    fe_kv_allocator_batch,
    fe_kv_allocator_create,
    fe_kv_allocator_destroy,
    fe_kv_allocator_num_allocated,
    fe_kv_allocator_num_free,
    fe_kv_allocator_release,
    fe_kv_allocator_seq_len,
    fe_last_error,
    fe_paged_gqa_decode,
    fe_paged_gqa_decode_append,
    fe_paged_gqa_decode_noalloc,
    fe_paged_gqa_decode_norm_rope_append,
    fe_paged_gqa_decode_num_partitions,
    fe_paged_gqa_decode_workspace_size,
    fe_paged_gqa_mixed,
    fe_paged_gqa_mixed_workspace_size,
    fe_paged_gqa_prefill_chunk,
    fe_paged_gqa_prefill_chunk_ex,
    fe_paged_kv_append,
    fe_qk_norm_rope_append,
    fe_sampler_form,
    fe_sampler_softmax_argmax,
    fe_sampler_softmax_argmax_ex,
    fe_sampler_workspace_size,
    fe_status_string,
    library_path,
    load_library,
)
