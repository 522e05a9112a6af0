"""KV-streams hot path on AMD MI355X (gfx950): Python binding of libks.so.

The kernels (RoPE at logical positions, eviction-masked attention forward and
backward, block-table compaction, paged GQA decode with 16-token or single-token
blocks) live in libks.so, built
from ``csrc/`` by ``python -m kv_cache_compaction_amd.build``.  This package
only marshals torch tensors into the C ABI declared in ``include/ks.h``.
"""
from ._lib import (  # noqa: F401
    KS_BF16, KS_BLOCK, KS_F32, KS_NEVER, KSError, LIB_PATH, header_functions,
    ks_append_kv, ks_compact_block_table, ks_compact_block_table_rounds, ks_evict_attn_bwd,
    ks_evict_attn_bwd_workspace, ks_evict_attn_fwd, ks_evict_attn_fwd_workspace,
    ks_evict_attn_fwd_rope, ks_evict_attn_bwd_rope,
    ks_append_kv_bs1, ks_check_block_table, ks_check_eviction_record, ks_paged_decode, ks_paged_decode_bs1, ks_paged_decode_bs1_workspace,
    ks_paged_decode_noalloc, ks_paged_decode_noalloc_max_scratch, ks_paged_decode_rope,
    ks_paged_decode_workspace, ks_rope_logical, load_library, ks_measure_mfma_bf16,
    ks_measure_mfma_flops, ks_measure_dq_atomics,
)
