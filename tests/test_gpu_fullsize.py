"""GPU parity at full configuration sizes, in the launch configuration the
bench times: sampled outputs the oracle computes one by one, plus
properties that hold at any size."""
import numpy as np
import pytest
import torch

import kv_cache_compaction_amd as ks
import oracle as O
from parity_util import announce, f64, gate
from workloads import (SUMMARY_32K, build_trace, check_trace, config_trace_batch,
                       normal_tensor, stacked_e)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


def _sample_rows(tr, rng, n=40):
    N = tr.N
    rows = {0, 1, 63, 64, 127, 128, N - 1, N - 2, N - 64, N - 65}
    for t in tr.events:
        rows.update({t - 1, t, t + 1})
    rows.update(int(x) for x in rng.integers(0, N, n))
    return np.array(sorted(r for r in rows if 0 <= r < N))


def run_training_config(cfg, b, hkv, key_blocks):
    traces, seeds = config_trace_batch(cfg)
    e = stacked_e(traces)
    B, N, Hq, Hkv, D = cfg.batch, cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    G = Hq // Hkv
    bf = torch.bfloat16
    q = normal_tensor((B, N, Hq, D), seeds["q"], cfg.value_scale, bf, DEV)
    k = normal_tensor((B, N, Hkv, D), seeds["k"], cfg.value_scale, bf, DEV)
    v = normal_tensor((B, N, Hkv, D), seeds["v"], cfg.value_scale, bf, DEV)
    do = normal_tensor((B, N, Hq, D), seeds["do"], cfg.value_scale, bf, DEV)
    heads = slice(hkv * G, (hkv + 1) * G)
    # raw projections of the sampled (trace, kv group) for the oracle
    q_raw = f64(q[b:b + 1, :, heads])
    k_raw = f64(k[b:b + 1, :, hkv:hkv + 1])
    v_h = f64(v[b:b + 1, :, hkv:hkv + 1])
    do_h = f64(do[b:b + 1, :, heads])
    pos = torch.arange(N, dtype=torch.int32, device=DEV)[None].repeat(B, 1).contiguous()
    ks.ks_rope_logical(q, k, pos)
    eg = torch.from_numpy(e).to(DEV)
    o, lse = ks.ks_evict_attn_fwd(q, k, v, eg)
    dq, dk, dv = ks.ks_evict_attn_bwd(q, k, v, eg, o, lse, do)
    torch.cuda.synchronize()

    # properties over every trace and head: softmax rows sum to one, so the
    # dV of a kv group sums to the dO of its query heads; S is bilinear in
    # (q, k), so sum q.dq = sum k.dk
    sdv = dv.float().sum(1)                                   # [B, Hkv, D]
    sdo = do.float().sum(1).view(B, Hkv, G, D).sum(2)
    assert torch.allclose(sdv, sdo, atol=0.05 * sdo.abs().max().item()), \
        (sdv - sdo).abs().max().item()
    a, c = q.float() * dq.float(), k.float() * dk.float()
    lhs, rhs = a.sum().item(), c.sum().item()
    # the exact sums are equal; bf16 rounding of each dq, dk element (2^-9
    # relative) moves them by about 2^-9 * sqrt(sum of squared terms)
    noise = 2.0**-9 * (a.square().sum().sqrt().item() + c.square().sum().sqrt().item())
    assert abs(lhs - rhs) <= 8 * noise, (lhs, rhs, noise)

    tr = traces[b]
    rows = _sample_rows(tr, np.random.default_rng(5))
    qs = O.rope(q_raw, np.arange(N)[None])
    kk = O.rope(k_raw, np.arange(N)[None])
    eb = e[b:b + 1]
    for hh in range(G):
        ro, rl = O.attn_fwd_rows(qs, kk, v_h, eb, 0, hh, rows)
        gate(o[b, rows, hkv * G + hh], ro, "bf16", f"O rows h{hh}")
        gate(lse[b, hkv * G + hh, rows], rl, "bf16", f"LSE rows h{hh}")
        rdq = O.attn_bwd_rows(qs, kk, v_h, eb, do_h, 0, hh, rows)
        gate(dq[b, rows, hkv * G + hh], rdq, "bf16grad", f"dQ rows h{hh}")
    for keys in key_blocks(tr):
        rdk, rdv = O.attn_bwd_keys(qs, kk, v_h, eb, do_h, 0, 0, keys)
        gate(dk[b, keys, hkv], rdk, "bf16grad", f"dK keys {keys[0]}..")
        gate(dv[b, keys, hkv], rdv, "bf16grad", f"dV keys {keys[0]}..")


def test_summary_32k_sampled():
    def key_blocks(tr):
        t1 = tr.events[0]
        return [np.arange(tr.N - 64, tr.N),                      # queries [j, N)
                np.arange(t1 - 1536 - 64, t1 - 1536)]            # evicted at t1
    run_training_config(SUMMARY_32K, b=1, hkv=3, key_blocks=key_blocks)


def test_trace_past_one_live_window():
    """A 132,096-token trace: the forward and dQ kernels list live key tiles
    in windows of 2,048 tiles (131,072 tokens), so query tiles past that
    point gather theirs from two windows (the pinned prompt and older recent
    turns in the first, the newest turns in the second).  Sampled rows there
    and key blocks on both sides of the boundary against the oracle."""
    N, Hq, Hkv, D = 132096, 8, 2, 128
    G = Hq // Hkv
    tr = build_trace(np.random.default_rng(77), N, 512, 8192, "recent")
    check_trace(tr)
    e = tr.e[None].astype(np.int32)
    bf = torch.bfloat16
    q = normal_tensor((1, N, Hq, D), 7701, 0.5, bf, DEV)
    k = normal_tensor((1, N, Hkv, D), 7702, 0.5, bf, DEV)
    v = normal_tensor((1, N, Hkv, D), 7703, 0.5, bf, DEV)
    do = normal_tensor((1, N, Hq, D), 7704, 0.5, bf, DEV)
    eg = torch.from_numpy(e).to(DEV)
    o, lse = ks.ks_evict_attn_fwd(q, k, v, eg)
    dq, dk, dv = ks.ks_evict_attn_bwd(q, k, v, eg, o, lse, do)
    torch.cuda.synchronize()
    hkv = 1
    heads = slice(hkv * G, (hkv + 1) * G)
    qh, kh, vh, doh = (f64(q[:, :, heads]), f64(k[:, :, hkv:hkv + 1]),
                       f64(v[:, :, hkv:hkv + 1]), f64(do[:, :, heads]))
    w = 2048 * 64
    rng = np.random.default_rng(78)
    rows = {w - 1, w, w + 1, w + 63, w + 64, N - 65, N - 64, N - 2, N - 1}
    rows.update(t for t in tr.events if t < N)
    rows.update(int(x) for x in rng.integers(w, N, 12))
    rows.update(int(x) for x in rng.integers(0, w, 6))
    rows = np.array(sorted(r for r in rows if 0 <= r < N))
    e64 = e.astype(np.int64)
    for hh in range(G):
        ro, rl = O.attn_fwd_rows(qh, kh, vh, e64, 0, hh, rows)
        gate(o[0, rows, hkv * G + hh], ro, "bf16", f"O rows h{hh}")
        gate(lse[0, hkv * G + hh, rows], rl, "bf16", f"LSE rows h{hh}")
        rdq = O.attn_bwd_rows(qh, kh, vh, e64, doh, 0, hh, rows)
        gate(dq[0, rows, hkv * G + hh], rdq, "bf16grad", f"dQ rows h{hh}")
    for keys in (np.arange(N - 64, N), np.arange(w - 32, w + 32)):
        rdk, rdv = O.attn_bwd_keys(qh, kh, vh, e64, doh, 0, 0, keys)
        gate(dk[0, keys, hkv], rdk, "bf16grad", f"dK keys {keys[0]}..")
        gate(dv[0, keys, hkv], rdv, "bf16grad", f"dV keys {keys[0]}..")
