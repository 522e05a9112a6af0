"""Seeded random weights and token ids of a small decoder stack.

Input construction only: the weights of a toy model whose attention is the
KV-streams path (no trained checkpoint exists here, so the weights are
random).  Every matrix is N(0, 1) / sqrt(fan_in), drawn in fp32 with numpy
from ``default_rng(seed)`` in a fixed order, so the oracle and the GPU stack
start from identical numbers.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class ToyShape:
    layers: int = 3
    vocab: int = 512
    d_model: int = 512
    Hq: int = 4
    Hkv: int = 2
    D: int = 128
    ffn: int = 1024


def toy_weights(shape: ToyShape, seed: int) -> dict:
    """Embedding ``emb`` [vocab, d_model], unembedding ``unemb`` [d_model,
    vocab] and per layer ``wq`` [d_model, Hq*D], ``wk``/``wv`` [d_model,
    Hkv*D], ``wo`` [Hq*D, d_model], ``w1`` [d_model, ffn], ``w2`` [ffn,
    d_model] (row-vector convention: y = x @ W)."""
    rng = np.random.default_rng(seed)

    def mat(r, c, fan_in):
        return (rng.standard_normal((r, c), dtype=np.float32) / np.sqrt(fan_in)).astype(np.float32)
    s = shape
    w = {"emb": rng.standard_normal((s.vocab, s.d_model), dtype=np.float32)}
    layers = []
    for _ in range(s.layers):
        layers.append({
            "wq": mat(s.d_model, s.Hq * s.D, s.d_model),
            "wk": mat(s.d_model, s.Hkv * s.D, s.d_model),
            "wv": mat(s.d_model, s.Hkv * s.D, s.d_model),
            "wo": mat(s.Hq * s.D, s.d_model, s.Hq * s.D),
            "w1": mat(s.d_model, s.ffn, s.d_model),
            "w2": mat(s.ffn, s.d_model, s.ffn),
        })
    w["layers"] = layers
    w["unemb"] = mat(s.d_model, s.vocab, s.d_model)
    return w


def toy_tokens(shape: ToyShape, N: int, seed: int) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, shape.vocab, size=N).astype(np.int64)
