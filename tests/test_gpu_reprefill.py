"""GPU parity of the re-prefill counterfactual: the segments re-prefill
compaction would process (paper page, Fig. 2A), packed end to end so that one
eviction-masked pass computes every segment's own causal attention.  Checked
against the oracle on the same packed input, element by element at the
4k-token size and on sampled rows at the 32k size the bench times."""
import numpy as np
import pytest
import torch

import kv_cache_compaction_amd as ks
import oracle as O
import rounding_model as RM
from parity_util import announce, f64, gate, gate_rows_model
from workloads import (SUMMARY_32K, TRAIN_4K, config_trace_batch, normal_tensor, reprefill_pack,
                       reprefill_segments)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


def _packed_inputs(cfg, pad_to=None):
    traces, seeds = config_trace_batch(cfg)
    packs = [reprefill_pack(tr) for tr in traces]
    L = max(len(p[0]) for p in packs) if pad_to is None else pad_to
    packs = [reprefill_pack(tr, L) for tr in traces]
    B, N, Hq, Hkv, D = cfg.batch, cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    bf = torch.bfloat16
    idx = torch.from_numpy(np.stack([p[0] for p in packs])).to(DEV)
    e = torch.from_numpy(np.stack([p[1] for p in packs])).to(DEV)
    out = {}
    for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv), ("do", Hq)):
        t = normal_tensor((B, N, H, D), seeds[name], cfg.value_scale, bf, DEV)
        out[name] = torch.stack([t[b, idx[b]] for b in range(B)]).contiguous()
    return traces, packs, e, out


def test_reprefill_4k_full_parity():
    cfg = TRAIN_4K
    traces, packs, e, x = _packed_inputs(cfg)
    assert len(reprefill_segments(traces[0])) >= 2
    o, lse = ks.ks_evict_attn_fwd(x["q"], x["k"], x["v"], e)
    dq, dk, dv = ks.ks_evict_attn_bwd(x["q"], x["k"], x["v"], e, o, lse, x["do"])
    torch.cuda.synchronize()
    G = cfg.Hq // cfg.Hkv
    en = e.cpu().numpy().astype(np.int64)
    for g in range(cfg.Hkv):
        hs = slice(g * G, (g + 1) * G)
        q, k, v, do = (f64(x[n][:, :, s]) for n, s in
                       (("q", hs), ("k", slice(g, g + 1)), ("v", slice(g, g + 1)), ("do", hs)))
        ro, rl = O.attn_fwd(q, k, v, en)
        rdq, rdk, rdv = O.attn_bwd(q, k, v, en, do)
        gate(o[:, :, hs], ro, "bf16", f"O kv{g}")
        gate(lse[:, hs], rl, "bf16", f"LSE kv{g}")
        gate(dq[:, :, hs], rdq, "bf16grad", f"dQ kv{g}")
        gate(dk[:, :, g:g + 1], rdk, "bf16grad", f"dK kv{g}")
        gate(dv[:, :, g:g + 1], rdv, "bf16grad", f"dV kv{g}")


def test_reprefill_32k_sampled():
    """The bench's packed launch (4 traces padded to a common length)."""
    cfg = SUMMARY_32K
    traces, packs, e, x = _packed_inputs(cfg)
    o, lse = ks.ks_evict_attn_fwd(x["q"], x["k"], x["v"], e)
    dq, dk, dv = ks.ks_evict_attn_bwd(x["q"], x["k"], x["v"], e, o, lse, x["do"])
    torch.cuda.synchronize()
    B, Hq, Hkv, D = cfg.batch, cfg.Hq, cfg.Hkv, cfg.D
    G = Hq // Hkv
    sdv = dv.float().sum(1)
    sdo = x["do"].float().sum(1).view(B, Hkv, G, D).sum(2)
    assert torch.allclose(sdv, sdo, atol=0.05 * sdo.abs().max().item())
    b, g = 2, 5
    L = e.shape[1]
    hs = slice(g * G, (g + 1) * G)
    q, k, v, do = (f64(x[n][b:b + 1, :, s]) for n, s in
                   (("q", hs), ("k", slice(g, g + 1)), ("v", slice(g, g + 1)), ("do", hs)))
    en = e[b:b + 1].cpu().numpy().astype(np.int64)
    n = sum(len(s) for s in reprefill_segments(traces[b]))
    rng = np.random.default_rng(9)
    rows = {0, 1, n - 1, L - 1}
    p = 0
    for s in reprefill_segments(traces[b]):      # first and last rows of segments
        rows.update({p, p + 1, p + len(s) - 1})
        p += len(s)
    rows.update(int(r) for r in rng.integers(0, L, 24))
    rows = np.array(sorted(rows))
    for hh in range(G):
        ro, rl = O.attn_fwd_rows(q, k, v, en, 0, hh, rows)
        gate(o[b, rows, g * G + hh], ro, "bf16", f"O rows h{hh}")
        gate(lse[b, g * G + hh, rows], rl, "bf16", f"LSE rows h{hh}")
        rdq = O.attn_bwd_rows(q, k, v, en, do, 0, hh, rows)
        mdq = RM.dq_rows(q, k, v, en, do, 0, hh, rows)
        gate_rows_model(dq[b, rows, g * G + hh], rdq, mdq, f"dQ rows h{hh}")
    for keys in (np.arange(0, 64), np.arange(n - 64, n)):
        rdk, rdv = O.attn_bwd_keys(q, k, v, en, do, 0, 0, keys)
        gate(dk[b, keys, g], rdk, "bf16grad", f"dK keys {keys[0]}..")
        gate(dv[b, keys, g], rdv, "bf16grad", f"dV keys {keys[0]}..")
