"""fp64 toy decoder stack over KV-streams attention (CPU, numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The trainer replays recorded compaction events so that every token's
states, at every layer, are the ones it formed during generation: retained
entries keep what they computed while the later-removed turns were still
visible, and later tokens cannot see the removed spans (explainer, trainer
paragraph and the closing paragraph on influence that remains in retained
entries; paper page, Fig. 2A).  With more than one layer this is a claim
about the whole stack, not only one attention call: `train_logits` runs the
masked pass over the rollout, `decode_logits` generates token by token with
per-layer caches from which each event removes the evicted spans, and the
two must agree.

Architecture (the pages fix none; plainest choice): x = emb[token]; per layer
  a = rmsnorm(x); q, k, v = a Wq, a Wk, a Wv split into heads of D;
  q, k rotated at their logical positions; x += attn(q, k, v) Wo;
  x += silu(rmsnorm(x) W1) W2;
logits = rmsnorm(x) U.  rmsnorm has no gain and eps = 1e-6; query head h
reads kv head floor(h / G).
"""
from __future__ import annotations

import numpy as np

from .ks_oracle import attn_fwd, paged_decode, rope

EPS = 1e-6


def rmsnorm(x):
    return x / np.sqrt((x * x).mean(-1, keepdims=True) + EPS)


def silu(x):
    return x / (1.0 + np.exp(-x))


def train_logits(w, tokens, e, Hq, Hkv, D):
    """Logits [N, vocab] of one masked pass over the whole trace (every layer
    uses the eviction record e [N])."""
    N = len(tokens)
    x = np.asarray(w["emb"], np.float64)[tokens]
    pos = np.arange(N)[None]
    ee = np.asarray(e, np.int64)[None]
    for L in w["layers"]:
        a = rmsnorm(x)
        q = (a @ L["wq"].astype(np.float64)).reshape(1, N, Hq, D)
        k = (a @ L["wk"].astype(np.float64)).reshape(1, N, Hkv, D)
        v = (a @ L["wv"].astype(np.float64)).reshape(1, N, Hkv, D)
        o, _ = attn_fwd(rope(q, pos), rope(k, pos), v, ee)
        x = x + o.reshape(N, Hq * D) @ L["wo"].astype(np.float64)
        x = x + silu(rmsnorm(x) @ L["w1"].astype(np.float64)) @ L["w2"].astype(np.float64)
    return rmsnorm(x) @ np.asarray(w["unemb"], np.float64)


def decode_logits(w, tokens, evicted, Hq, Hkv, D):
    """Logits [N, vocab] generated token by token.

    ``evicted`` maps an event index t to the token spans [(a, b)] removed
    before token t is generated.  Each layer keeps the rotated keys and the
    values of its live tokens in order; decode attends them through an
    identity table of single-token blocks.
    """
    N = len(tokens)
    nl = len(w["layers"])
    cache = [{"tok": [], "k": [], "v": []} for _ in range(nl)]
    out = None
    for t in range(N):
        if t in evicted:
            gone = np.zeros(N, bool)
            for (a, b) in evicted[t]:
                gone[a:b] = True
            for c in cache:
                keep = [i for i, j in enumerate(c["tok"]) if not gone[j]]
                for key in ("tok", "k", "v"):
                    c[key] = [c[key][i] for i in keep]
        x = np.asarray(w["emb"], np.float64)[tokens[t]]
        pos = np.array([[t]])
        for L, c in zip(w["layers"], cache):
            a = rmsnorm(x)
            q = (a @ L["wq"].astype(np.float64)).reshape(1, 1, Hq, D)
            k = (a @ L["wk"].astype(np.float64)).reshape(1, 1, Hkv, D)
            v = (a @ L["wv"].astype(np.float64)).reshape(Hkv, D)
            c["tok"].append(t)
            c["k"].append(rope(k, pos)[0, 0])
            c["v"].append(v)
            n = len(c["tok"])
            kp = np.stack(c["k"])[:, :, None]            # [n, Hkv, 1, D]
            vp = np.stack(c["v"])[:, :, None]
            o, _ = paged_decode(rope(q, pos)[:, 0], kp, vp, np.arange(n)[None], np.array([n]))
            x = x + o.reshape(Hq * D) @ L["wo"].astype(np.float64)
            x = x + silu(rmsnorm(x) @ L["w1"].astype(np.float64)) @ L["w2"].astype(np.float64)
        lg = rmsnorm(x) @ np.asarray(w["unemb"], np.float64)
        if out is None:
            out = np.zeros((N, lg.shape[-1]))
        out[t] = lg
    return out


def log_softmax(z):
    z = z - z.max(-1, keepdims=True)
    return z - np.log(np.exp(z).sum(-1, keepdims=True))


def kl_rows(p_logits, q_logits):
    """KL(p || q) per row from two logit arrays."""
    lp, lq = log_softmax(np.asarray(p_logits, np.float64)), log_softmax(np.asarray(q_logits, np.float64))
    return (np.exp(lp) * (lp - lq)).sum(-1)
