"""GPU parity of the long mixed workload: 8 traces of 65,536 tokens with
window / prompt+recent / summary compaction, 64 q / 8 kv heads; masked
forward + backward with RoPE fused in (the bench's launch: q and k are the
raw projections, dq and dk their gradients), then 256 decode steps per trace
with a forced compaction after the 128th new token.  Sampled outputs are checked against the oracle
(rows and key blocks of one kv group per trace); properties over all."""
import numpy as np
import pytest
import torch

import kv_cache_compaction_amd as ks
import oracle as O
import rounding_model as RM
from parity_util import announce, f64, gate, gate_rows_model, oracle_bwd_keys
from workloads import (BLOCK, KS_NEVER, LONG_MIXED_64K, config_trace_batch,
                       continuation_layout, normal_tensor, stacked_e)

pytestmark = pytest.mark.gpu
DEV = "cuda"
CFG = LONG_MIXED_64K
NDEC = 256
EVENT_AFTER = 128


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


@pytest.fixture(scope="module")
def run():
    traces, seeds = config_trace_batch(CFG)
    e = stacked_e(traces)
    B, N, Hq, Hkv, D = CFG.batch, CFG.N, CFG.Hq, CFG.Hkv, CFG.D
    G = Hq // Hkv
    bf = torch.bfloat16
    q = normal_tensor((B, N, Hq, D), seeds["q"], CFG.value_scale, bf, DEV)
    k = normal_tensor((B, N, Hkv, D), seeds["k"], CFG.value_scale, bf, DEV)
    v = normal_tensor((B, N, Hkv, D), seeds["v"], CFG.value_scale, bf, DEV)
    do = normal_tensor((B, N, Hq, D), seeds["do"], CFG.value_scale, bf, DEV)
    # raw projections of kv group (b % Hkv) of every trace, for the oracle
    raw = []
    for b in range(B):
        g = b % Hkv
        d = dict(k=f64(k[b:b + 1, :, g:g + 1]), v=f64(v[b:b + 1, :, g:g + 1]))
        if b < 3:   # the row/key samples use one trace per strategy
            d.update(q=f64(q[b:b + 1, :, g * G:(g + 1) * G]),
                     do=f64(do[b:b + 1, :, g * G:(g + 1) * G]))
        raw.append(d)
    pos = torch.arange(N, dtype=torch.int32, device=DEV)[None].repeat(B, 1).contiguous()
    eg = torch.from_numpy(e).to(DEV)
    o, lse, q_rot, k_rot = ks.ks_evict_attn_fwd_rope(q, k, v, eg, pos)
    dq, dk, dv = ks.ks_evict_attn_bwd_rope(q_rot, k_rot, v, eg, pos, o, lse, do)
    del q_rot
    torch.cuda.synchronize()
    return dict(traces=traces, e=e, q=q, k=k, k_rot=k_rot, v=v, do=do, o=o, lse=lse, dq=dq,
                dk=dk, dv=dv, raw=raw)


def test_mixed64k_properties(run):
    B, Hq, Hkv, D = CFG.batch, CFG.Hq, CFG.Hkv, CFG.D
    G = Hq // Hkv
    for b in range(B):
        sdv = run["dv"][b].float().sum(0)
        sdo = run["do"][b].float().sum(0).view(Hkv, G, D).sum(1)
        assert torch.allclose(sdv, sdo, atol=0.05 * sdo.abs().max().item()), b
        a = run["q"][b].float() * run["dq"][b].float()
        c = run["k"][b].float() * run["dk"][b].float()
        lhs, rhs = a.sum().item(), c.sum().item()
        # the exact sums are equal; bf16 rounding of each dq, dk element (2^-9
        # relative) moves them by about 2^-9 * sqrt(sum of squared terms)
        noise = 2.0**-9 * (a.square().sum().sqrt().item() + c.square().sum().sqrt().item())
        assert abs(lhs - rhs) <= 8 * noise, (b, lhs, rhs, noise)
        assert torch.isfinite(run["o"][b].float()).all()


@pytest.mark.parametrize("b", [0, 1, 2])      # one trace per strategy
def test_mixed64k_sampled_rows_and_keys(run, b):
    tr = run["traces"][b]
    N, G, Hkv = CFG.N, CFG.Hq // CFG.Hkv, CFG.Hkv
    g = b % Hkv
    r = run["raw"][b]
    pos = np.arange(N)[None]
    qs, kk = O.rope(r["q"], pos), O.rope(r["k"], pos)
    eb = run["e"][b:b + 1]
    rng = np.random.default_rng(50 + b)
    rows = {0, 1, N - 1, N - 2, N // 2}
    for t in tr.events:
        rows.update({t - 1, t, t + 1})
    rows.update(int(x) for x in rng.integers(0, N, 12))
    rows = np.array(sorted(x for x in rows if 0 <= x < N))
    for hh in range(G):
        h = g * G + hh
        ro, rl = O.attn_fwd_rows(qs, kk, r["v"], eb, 0, hh, rows)
        gate(run["o"][b, rows, h], ro, "bf16", f"O rows t{b} h{h}")
        gate(run["lse"][b, h, rows], rl, "bf16", f"LSE rows t{b} h{h}")
        # gradients of the raw projections: the oracle's rows rotated back
        rdq = RM.unrotate_rows(O.attn_bwd_rows(qs, kk, r["v"], eb, r["do"], 0, hh, rows), rows)
        mdq = RM.dq_rows(qs, kk, r["v"], eb, r["do"], 0, hh, rows, pos=rows)
        gate_rows_model(run["dq"][b, rows, h], rdq, mdq, f"dQ rows t{b} h{h}")
    blocks = key_blocks(tr)
    allk = np.concatenate(blocks)
    rdk, rdv = oracle_bwd_keys(qs, kk, r["v"], eb, r["do"], allk)
    rdk = RM.unrotate_rows(rdk, allk)
    at = 0
    for keys in blocks:
        sl = slice(at, at + len(keys))
        at += len(keys)
        gate(run["dk"][b, keys, g], rdk[sl], "bf16grad", f"dK t{b} keys {keys[0]}..")
        gate(run["dv"][b, keys, g], rdv[sl], "bf16grad", f"dV t{b} keys {keys[0]}..")


def key_blocks(tr):
    """Key blocks of one trace whose dK/dV sum over the longest and the
    event-crossing query ranges: the prompt's first and last blocks (every
    row of the trace where the prompt is pinned; up to the event that pops
    it in the sliding window), a block alive across the first event and
    evicted later, the trace's last keys, and for the summary strategy a
    block evicted at the first event."""
    N, P = tr.N, tr.P
    t1 = tr.events[0]
    blocks = [np.arange(0, 64), np.arange(P - 64, P)]
    for j0 in range(t1 - 64, P - 1, -64):         # alive across t1, evicted later
        ej = tr.e[j0:j0 + 64].astype(np.int64)
        if ej.min() > t1 and ej.max() < N:
            blocks.append(np.arange(j0, j0 + 64))
            break
    else:
        raise AssertionError("no block alive across the first event")
    blocks.append(np.arange(N - 64, N))
    if tr.strategy == "summary":
        lo = t1 - (tr.overlap + tr.summary)
        blocks.append(np.arange(lo - 64, lo))       # evicted at the first event
    return blocks


def test_mixed64k_decode_with_forced_compaction(run):
    """Lay each trace's final live set into a paged pool (keys as the training
    path rotated them), then decode 256 tokens per trace: RoPE of q and k at
    positions N + s, append, paged decode; after token 128 a forced event
    applies the trace's strategy and the tables are compacted.  Sampled steps
    are compared with the oracle's masked attention over the extended trace."""
    traces = run["traces"]
    B, N, Hq, Hkv, D = CFG.batch, CFG.N, CFG.Hq, CFG.Hkv, CFG.D
    G = Hq // Hkv
    bf = torch.bfloat16
    # --- pool and tables: live tokens of the trace, then NDEC/16 fresh blocks;
    # the forced event after token EVENT_AFTER
    lay = continuation_layout(traces, N, NDEC, EVENT_AFTER, np.random.default_rng(5005))
    table0, nblk0, L0, NB = lay.table0, lay.nblk0, lay.live_len, lay.num_pool_blocks
    kp = torch.full((NB, Hkv, BLOCK, D), float("nan"), dtype=bf, device=DEV)
    vp = torch.full((NB, Hkv, BLOCK, D), float("nan"), dtype=bf, device=DEV)
    for b in range(B):
        blk = torch.from_numpy(np.repeat(table0[b, :L0[b] // BLOCK], BLOCK).astype(np.int64)).to(DEV)
        slot = torch.arange(L0[b], device=DEV) % BLOCK
        tok = torch.from_numpy(lay.live_tok[b].astype(np.int64)).to(DEV)
        kp[blk, :, slot] = run["k_rot"][b, tok]
        vp[blk, :, slot] = run["v"][b, tok]
    keep, ev_tokens, ev_spans, t_ev = lay.keep, lay.ev_tokens, lay.ev_spans, lay.t_ev
    # --- decode inputs (raw), seeded
    qn = normal_tensor((NDEC, B, Hq, D), 7001, 0.5, bf, DEV)
    kn = normal_tensor((NDEC, B, Hkv, D), 7002, 0.5, bf, DEV)
    vn = normal_tensor((NDEC, B, Hkv, D), 7003, 0.5, bf, DEV)
    qn_raw, kn_raw, vn_raw = f64(qn), f64(kn), f64(vn)
    table = torch.from_numpy(table0).to(DEV)
    nblk = torch.from_numpy(nblk0.astype(np.int32)).to(DEV)
    keep_g = torch.from_numpy(keep).to(DEV)
    length = L0.copy()
    check_steps = [0, 1, EVENT_AFTER - 1, EVENT_AFTER, 200, NDEC - 1]
    got = {}
    for s in range(NDEC):
        if s == EVENT_AFTER:
            table, nblk, _ = ks.ks_compact_block_table(table, nblk, keep_g)
            length = length - ev_tokens
        length = length + 1
        seq = torch.from_numpy(length.astype(np.int32)).to(DEV)
        posn = torch.full((B,), N + s, dtype=torch.int32, device=DEV)
        qs = qn[s][:, None].contiguous()
        ks.ks_rope_logical(qs, None, posn[:, None].contiguous())
        ks.ks_append_kv(kn[s].contiguous(), vn[s].contiguous(), posn, table, seq, kp, vp)
        out, lse = ks.ks_paged_decode(qs[:, 0].contiguous(), kp, vp, table, seq)
        if s in check_steps:
            got[s] = (out.clone(), lse.clone())
    torch.cuda.synchronize()
    for s, (out, _) in got.items():
        assert torch.isfinite(out.float()).all(), s
    # --- oracle: rows N + s of the masked attention over the extended trace
    Next = N + NDEC
    for b in range(B):
        g = b % Hkv
        r = run["raw"][b]
        e_ext = np.full(Next, KS_NEVER, np.int64)
        e_ext[:N] = run["e"][b]
        for (x, y) in ev_spans[b]:
            e_ext[x:y] = t_ev
        k_ext = np.concatenate([r["k"][0, :, 0], kn_raw[:, b, g]], axis=0)[None, :, None]
        v_ext = np.concatenate([r["v"][0, :, 0], vn_raw[:, b, g]], axis=0)[None, :, None]
        k_ext = O.rope(k_ext, np.arange(Next)[None])
        q_ext = np.zeros((1, Next, G, D))
        rows = np.array([N + s for s in check_steps])
        q_ext[0, rows] = O.rope(qn_raw[check_steps, b, g * G:(g + 1) * G][None], rows[None])[0]
        for hh in range(G):
            ro, rl = O.attn_fwd_rows(q_ext, k_ext, v_ext, e_ext[None], 0, hh, rows)
            h = g * G + hh
            out_h = torch.stack([got[s][0][b, h] for s in check_steps])
            lse_h = torch.stack([got[s][1][b, h] for s in check_steps])
            gate(out_h, ro, "bf16", f"decode t{b} h{h}")
            gate(lse_h, rl, "bf16", f"decode lse t{b} h{h}")
