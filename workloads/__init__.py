"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This package builds inputs only: turn boundaries, compaction-event records
(the per-token eviction index e_j), paged block tables with per-round keep
flags, the paged layout of traces continued by decoding, the segment traces of the re-prefill counterfactual, random tensors
and the random weights of a toy decoder stack.  It holds none of the
method's arithmetic (no RoPE, no attention, no table compaction); the oracle
and the HIP library each implement those on their own.
"""
from .traces import (  # noqa: F401
    KS_NEVER, BLOCK, Trace, build_trace, check_trace, Continuation, DecodeBatch, evict_units,
    build_decode_batch, continuation_layout, normal_tensor, reprefill_pack, reprefill_segments,
    trace_blocks_keep,
)
from .configs import (LONG_MIXED_64K, PAGED_DECODE, SUMMARY_32K, TINY_F32,  # noqa: F401
                      TRAIN_4K, TRAINING_WORKLOADS, WORKLOADS, Config, config_trace_batch,
                      stacked_e, workload_rng)
from .toy import ToyShape, toy_tokens, toy_weights  # noqa: F401
