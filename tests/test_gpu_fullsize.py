"""GPU parity at full configuration sizes, in the launch configuration the
bench times: sampled outputs the oracle computes one by one, plus
properties that hold at any size."""
import numpy as np
import pytest
import torch

import kv_cache_compaction_amd as ks
import oracle as O
import rounding_model as RM
from parity_util import announce, f64, gate, gate_rows_model, oracle_bwd_keys
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


def check_rows(o, lse, dq, q_raw, k_raw, v_h, do_h, e, b, hkv, rows, tag="", unrotated=False):
    """Forward and dQ rows of one (trace, kv group) against the oracle; the
    dQ gate is tied to the rounding model (parity_util.gate_rows_model).
    ``unrotated``: dq holds gradients of the unrotated queries (the RoPE-
    fused backward), so the oracle's rows are rotated back at their
    positions (0..N-1 here)."""
    N = q_raw.shape[1]
    G = q_raw.shape[2]
    qs = O.rope(q_raw, np.arange(N)[None])
    kk = O.rope(k_raw, np.arange(N)[None])
    eb = e[b:b + 1]
    for hh in range(G):
        h = hkv * G + hh
        ro, rl = O.attn_fwd_rows(qs, kk, v_h, eb, 0, hh, rows)
        gate(o[b, rows, h], ro, "bf16", f"O rows{tag} h{h}")
        gate(lse[b, h, rows], rl, "bf16", f"LSE rows{tag} h{h}")
        rdq = O.attn_bwd_rows(qs, kk, v_h, eb, do_h, 0, hh, rows)
        if unrotated:
            rdq = RM.unrotate_rows(rdq, rows)
        mdq = RM.dq_rows(qs, kk, v_h, eb, do_h, 0, hh, rows, pos=rows if unrotated else None)
        gate_rows_model(dq[b, rows, h], rdq, mdq, f"dQ rows{tag} h{h}")
    return qs, kk


def run_training_config(cfg, b, hkv, key_blocks):
    """The bench's launch on the full configuration (RoPE fused into the
    forward and backward; q and k are the unrotated projections at
    positions 0..N-1, and the gradients are theirs); rows of every (trace,
    kv group) unit and key blocks of unit (b, hkv) against the oracle."""
    traces, seeds = config_trace_batch(cfg)
    e = stacked_e(traces)
    B, N, Hq, Hkv, D = cfg.batch, cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    G = Hq // Hkv
    bf = torch.bfloat16
    q = normal_tensor((B, N, Hq, D), seeds["q"], cfg.value_scale, bf, DEV)
    k = normal_tensor((B, N, Hkv, D), seeds["k"], cfg.value_scale, bf, DEV)
    v = normal_tensor((B, N, Hkv, D), seeds["v"], cfg.value_scale, bf, DEV)
    do = normal_tensor((B, N, Hq, D), seeds["do"], cfg.value_scale, bf, DEV)
    q_raw, k_raw = q.cpu(), k.cpu()
    pos = torch.arange(N, dtype=torch.int32, device=DEV)[None].repeat(B, 1).contiguous()
    eg = torch.from_numpy(e).to(DEV)
    o, lse, q_rot, k_rot = ks.ks_evict_attn_fwd_rope(q, k, v, eg, pos)
    dq, dk, dv = ks.ks_evict_attn_bwd_rope(q_rot, k_rot, v, eg, pos, o, lse, do)
    del q_rot, k_rot
    torch.cuda.synchronize()

    # properties over every trace and head: softmax rows sum to one, so the
    # dV of a kv group sums to the dO of its query heads; S is bilinear in
    # (q, k), so sum q.dq = sum k.dk (also for the unrotated projections
    # and their gradients: the rotation is orthogonal)
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

    o, lse, dq, dk, dv, v_c, do_c = (t.cpu() for t in (o, lse, dq, dk, dv, v, do))
    # rows of every (trace, kv group) unit: the structural rows plus random
    # ones (40 for the unit whose keys are checked, 8 elsewhere)
    for bb in range(B):
        for gg in range(Hkv):
            heads = slice(gg * G, (gg + 1) * G)
            main = (bb, gg) == (b, hkv)
            rows = _sample_rows(traces[bb], np.random.default_rng(5 + 100 * bb + gg),
                                n=40 if main else 8)
            qs, kk = check_rows(o, lse, dq, f64(q_raw[bb:bb + 1, :, heads]),
                                f64(k_raw[bb:bb + 1, :, gg:gg + 1]),
                                f64(v_c[bb:bb + 1, :, gg:gg + 1]),
                                f64(do_c[bb:bb + 1, :, heads]), e, bb, gg, rows,
                                tag=f" t{bb}", unrotated=True)
            if not main:
                continue
            v_h = f64(v_c[bb:bb + 1, :, gg:gg + 1])
            do_h = f64(do_c[bb:bb + 1, :, heads])
            blocks = key_blocks(traces[bb])
            allk = np.concatenate(blocks)
            rdk, rdv = oracle_bwd_keys(qs, kk, v_h, e[bb:bb + 1], do_h, allk)
            rdk = RM.unrotate_rows(rdk, allk)               # keys at positions 0..N-1
            at = 0
            for keys in blocks:
                sl = slice(at, at + len(keys))
                at += len(keys)
                gate(dk[bb, keys, gg], rdk[sl], "bf16grad", f"dK t{bb} keys {keys[0]}..")
                gate(dv[bb, keys, gg], rdv[sl], "bf16grad", f"dV t{bb} keys {keys[0]}..")


def summary_key_blocks(tr):
    """Key blocks whose dK/dV sum over the longest and the event-crossing
    query ranges: the never-evicted prompt (every row of the trace), the
    block retained at the first event and evicted at the second (its queries
    span the first event), the trace's last keys, and a block evicted at
    the first event."""
    t1 = tr.events[0]
    keep = tr.overlap + tr.summary
    return [np.arange(0, 64),                                   # prompt: rows [0, N)
            np.arange(tr.P - 64, tr.P),                         # prompt, last block
            np.arange(t1 - 64, t1),                             # kept at t1, evicted later
            np.arange(tr.N - 64, tr.N),                         # queries [j, N)
            np.arange(t1 - keep - 64, t1 - keep)]               # evicted at t1


def test_summary_32k_sampled():
    run_training_config(SUMMARY_32K, b=1, hkv=3, key_blocks=summary_key_blocks)


def test_trace_past_one_live_window():
    """A 132,096-token trace: the forward and dQ kernels list live key tiles
    in windows of 2,048 tiles (131,072 tokens), so query tiles past that
    point gather theirs from two windows (the pinned prompt and older recent
    turns in the first, the newest turns in the second).  Sampled rows there
    and key blocks on both sides of the boundary against the oracle, through
    the fused RoPE entry points (positions 0..N-1; gradients of the raw
    projections)."""
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
    pos = torch.arange(N, dtype=torch.int32, device=DEV)[None].contiguous()
    o, lse, q_rot, k_rot = ks.ks_evict_attn_fwd_rope(q, k, v, eg, pos)
    dq, dk, dv = ks.ks_evict_attn_bwd_rope(q_rot, k_rot, v, eg, pos, o, lse, do)
    del q_rot, k_rot
    torch.cuda.synchronize()
    hkv = 1
    heads = slice(hkv * G, (hkv + 1) * G)
    pn = np.arange(N)[None]
    qh, kh, vh, doh = (O.rope(f64(q[:, :, heads]), pn), O.rope(f64(k[:, :, hkv:hkv + 1]), pn),
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
        rdq = RM.unrotate_rows(O.attn_bwd_rows(qh, kh, vh, e64, doh, 0, hh, rows), rows)
        mdq = RM.dq_rows(qh, kh, vh, e64, doh, 0, hh, rows, pos=rows)
        gate_rows_model(dq[0, rows, hkv * G + hh], rdq, mdq, f"dQ rows h{hh}")
    for keys in (np.arange(N - 64, N), np.arange(w - 32, w + 32)):
        rdk, rdv = O.attn_bwd_keys(qh, kh, vh, e64, doh, 0, 0, keys)
        rdk = RM.unrotate_rows(rdk, keys)
        gate(dk[0, keys, hkv], rdk, "bf16grad", f"dK keys {keys[0]}..")
        gate(dv[0, keys, hkv], rdv, "bf16grad", f"dV keys {keys[0]}..")
