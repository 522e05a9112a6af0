"""A small random-weight decoder stack driven by the KV-streams path.

Shows the path as a model uses it: the training pass runs every layer's
attention as one eviction-masked call over the rollout, and generation runs
token by token over paged caches that each compaction event splices
(explainer: trainer paragraph, RoPE and block-table paragraphs).  Both
produce next-token distributions; with the same weights they must agree up
to rounding, because every surviving entry is the one computed before the
event and no later token sees a removed span.

Attention, RoPE, the cache append, decode and the table splice run in
libks; projections, norms and the MLP are plain bf16 GEMMs and elementwise
torch ops (a stand-in model, not part of the path).  Architecture: x =
emb[token]; per layer x += attn(rope(q), rope(k), v) Wo with q, k, v =
rmsnorm(x) W; x += silu(rmsnorm(x) W1) W2; logits = rmsnorm(x) U.  The
residual stream and the norms are fp32, GEMM operands bf16.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as K

BLOCK = K.KS_BLOCK


class ToyStack:
    def __init__(self, weights: dict, Hq: int, Hkv: int, D: int, device="cuda",
                 base: float = 10000.0):
        bf = torch.bfloat16
        self.Hq, self.Hkv, self.D, self.base = Hq, Hkv, D, base
        self.dev = device
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        self.emb = t(weights["emb"]).float()
        self.unemb = t(weights["unemb"]).to(bf)
        self.layers = []
        for L in weights["layers"]:
            self.layers.append({
                "wqkv": torch.cat([t(L["wq"]), t(L["wk"]), t(L["wv"])], 1).to(bf),
                "wo": t(L["wo"]).to(bf), "w1": t(L["w1"]).to(bf), "w2": t(L["w2"]).to(bf)})

    @staticmethod
    def _norm(x):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + 1e-6)

    def _qkv(self, L, x):
        n = x.shape[0]
        y = self._norm(x).to(torch.bfloat16) @ L["wqkv"]
        hq, hk = self.Hq * self.D, self.Hkv * self.D
        q = y[:, :hq].reshape(n, self.Hq, self.D)
        k = y[:, hq:hq + hk].reshape(n, self.Hkv, self.D)
        v = y[:, hq + hk:].reshape(n, self.Hkv, self.D)
        return q, k, v

    def _mlp_out(self, L, x, o):
        x = x + (o.reshape(x.shape[0], -1) @ L["wo"]).float()
        h = torch.nn.functional.silu((self._norm(x).to(torch.bfloat16) @ L["w1"]).float())
        return x + (h.to(torch.bfloat16) @ L["w2"]).float()

    def _logits(self, x):
        return (self._norm(x).to(torch.bfloat16) @ self.unemb).float()

    def train_logits(self, tokens: torch.Tensor, e: torch.Tensor) -> torch.Tensor:
        """fp32 logits [N, vocab] of one masked pass; tokens int64 [N], e int32 [N]."""
        N = tokens.shape[0]
        x = self.emb[tokens]
        pos = torch.arange(N, dtype=torch.int32, device=self.dev)[None]
        e2 = e.reshape(1, N).contiguous()
        for L in self.layers:
            q, k, v = self._qkv(L, x)
            q, k, v = q[None].contiguous(), k[None].contiguous(), v[None].contiguous()
            K.ks_rope_logical(q, k, pos, base=self.base)
            o, _ = K.ks_evict_attn_fwd(q, k, v, e2)
            x = self._mlp_out(L, x, o[0])
        return self._logits(x)

    def decode_logits(self, tokens: torch.Tensor, evicted: dict, block_size: int = BLOCK
                      ) -> torch.Tensor:
        """fp32 logits [N, vocab], generating one token at a time.

        ``evicted`` maps an event index t to the token spans removed before
        token t.  With ``block_size`` 16 (the vLLM setup) the spans must be
        whole 16-token blocks, as padded turns make them; with 1 (SGLang's
        single-token blocks) any span works.  Every layer has its own pool;
        one table serves all of them and is spliced with
        ks_compact_block_table at each event.  The new token's key is rotated
        by the append, its query inside the decode kernel.
        """
        if block_size not in (1, BLOCK):
            raise ValueError(f"block_size {block_size} (1 or {BLOCK})")
        bs = block_size
        N = tokens.shape[0]
        nl = len(self.layers)
        MB = N // bs + 2
        bf = torch.bfloat16
        shape = (nl, MB, self.Hkv, bs, self.D) if bs > 1 else (nl, MB, self.Hkv, self.D)
        kp = torch.zeros(shape, dtype=bf, device=self.dev)
        vp = torch.zeros_like(kp)
        append = K.ks_append_kv if bs > 1 else K.ks_append_kv_bs1
        table_h = []                      # block ids, in order
        first_tok = []                    # logical first token of each listed block
        nxt_block = 0
        live = 0
        table = torch.full((1, MB), -1, dtype=torch.int32, device=self.dev)
        nblk = torch.zeros(1, dtype=torch.int32, device=self.dev)
        pos_all = torch.arange(N, dtype=torch.int32, device=self.dev)
        out = torch.empty((N, self.unemb.shape[1]), dtype=torch.float32, device=self.dev)
        for t in range(N):
            if t in evicted:
                gone = np.zeros(N, bool)
                for (a, b) in evicted[t]:
                    if a % bs or b % bs:
                        raise ValueError(f"evicted spans must be whole {bs}-token blocks")
                    gone[a:b] = True
                keep = np.array([0 if gone[f] else 1 for f in first_tok], np.uint8)
                kp_row = np.zeros((1, MB), np.uint8)
                kp_row[0, :len(keep)] = keep
                nblk.fill_(len(table_h))
                table, nblk, _ = K.ks_compact_block_table(
                    table, nblk, torch.from_numpy(kp_row).to(self.dev))
                live -= int(bs * (len(keep) - keep.sum()))
                table_h = [b for b, k in zip(table_h, keep) if k]
                first_tok = [f for f, k in zip(first_tok, keep) if k]
            if live % bs == 0:            # the new token opens a block
                table_h.append(nxt_block)
                first_tok.append(t)
                table[0, len(table_h) - 1] = nxt_block
                nxt_block += 1
            live += 1
            seq = torch.full((1,), live, dtype=torch.int32, device=self.dev)
            pos = pos_all[t:t + 1]
            x = self.emb[tokens[t:t + 1]]
            for li, L in enumerate(self.layers):
                q, k, v = self._qkv(L, x)
                append(k.contiguous(), v.contiguous(), pos, table, seq, kp[li], vp[li],
                       base=self.base)
                o, _ = K.ks_paged_decode_rope(q.contiguous(), pos, kp[li], vp[li], table, seq,
                                              base=self.base)
                x = self._mlp_out(L, x, o)
            out[t] = self._logits(x)[0]
        return out
