"""The five workload configurations of the KV-streams hot path.

Seeds: a configuration with seed index ``k`` draws its structure from
``numpy.random.default_rng(1000 + k)`` (``workload_rng``); trace ``b`` of a
batch uses child ``b`` of that generator's ``spawn(...)``.  Tensor seeds are
drawn from the same generator, so every input is a pure function of the seed
index.

The shapes stand in for the paper's rollouts (32k-token rollouts, budgets B
and overlap/summary sizes o+s: paper page, Fig. 3; 16-padded turns: wqu.guru
explainer), since the benchmark suites and models the pages train on are not
available here.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .traces import build_trace, check_trace


@dataclass(frozen=True)
class Config:
    seed_index: int
    name: str
    batch: int
    N: int
    Hq: int
    Hkv: int
    D: int
    dtype: str              # "f32" or "bf16"
    P: int
    budget: int
    strategies: tuple       # per trace, cycled
    turn_len: tuple = (64, 512)
    overlap: int = 0
    summary: int = 0
    value_scale: float = 0.5
    backward: bool = True
    rope_base: float = 10000.0


TINY_F32 = Config(1, "tiny-f32", batch=1, N=512, Hq=1, Hkv=1, D=64, dtype="f32",
              P=64, budget=256, strategies=("recent",), turn_len=(64, 64),
              value_scale=1.0, backward=False)
TRAIN_4K = Config(2, "train-4k", batch=1, N=4096, Hq=8, Hkv=2, D=128, dtype="bf16",
              P=256, budget=2048, strategies=("recent",))
SUMMARY_32K = Config(3, "summary-32k", batch=4, N=32768, Hq=32, Hkv=8, D=128,
              dtype="bf16", P=512, budget=8192, strategies=("summary",),
              overlap=1024, summary=512)
PAGED_DECODE = Config(4, "paged-decode", batch=64, N=0, Hq=32, Hkv=8, D=128,
              dtype="bf16", P=16, budget=0, strategies=(), backward=False)
LONG_MIXED_64K = Config(5, "long-mixed-64k", batch=8, N=65536, Hq=64, Hkv=8, D=128,
              dtype="bf16", P=512, budget=16384,
              strategies=("window", "recent", "summary"),
              overlap=2048, summary=1024)

# every workload by name; the training ones (those with traces) in order of size
WORKLOADS = {c.name: c for c in (TINY_F32, TRAIN_4K, SUMMARY_32K, PAGED_DECODE, LONG_MIXED_64K)}
TRAINING_WORKLOADS = (TINY_F32, TRAIN_4K, SUMMARY_32K, LONG_MIXED_64K)


def workload_rng(cfg: Config) -> np.random.Generator:
    """The generator a configuration's structure is drawn from."""
    return np.random.default_rng(1000 + cfg.seed_index)


def config_trace_batch(cfg: Config, check: bool = True):
    """Traces of a training configuration, plus tensor seeds.

    Returns ``(traces, seeds)`` where ``seeds`` maps the tensor names
    q, k, v, do to integer seeds.
    """
    root = workload_rng(cfg)
    seeds = {name: int(root.integers(0, 2**31 - 1)) for name in ("q", "k", "v", "do")}
    children = root.spawn(cfg.batch)
    traces = []
    for b in range(cfg.batch):
        strat = cfg.strategies[b % len(cfg.strategies)]
        tr = build_trace(children[b], cfg.N, cfg.P, cfg.budget, strat,
                         turn_len=cfg.turn_len, overlap=cfg.overlap,
                         summary=cfg.summary)
        if check:
            check_trace(tr)
        traces.append(tr)
    return traces, seeds


def stacked_e(traces) -> np.ndarray:
    """int32 [B, N] eviction record of a batch of equal-length traces."""
    return np.stack([t.e for t in traces]).astype(np.int32)
