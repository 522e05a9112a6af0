"""Plain fp64 CPU oracle for the KV-streams hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and never imports it.
"""
from .ks_oracle import (  # noqa: F401
    KS_NEVER, BLOCK, rope, eviction_mask, attn_fwd, attn_fwd_rows, attn_bwd,
    attn_bwd_rows, attn_bwd_keys, compact_block_table, paged_decode,
    live_keys, count_bad_e, count_bad_table,
)
from . import toy_stack  # noqa: F401
