"""GPU parity of the single-token-block variant (the SGLang setup: no
padding to 16, token-granular compaction and gather) against the fp64
oracle: token-table compaction bit-exact (long rows split over workgroups),
decode and append over [slots, Hkv, D] pools, the token-granular decode
batch at full size, and masked training attention on an unpadded trace."""
import math

import numpy as np
import pytest
import torch

import kv_cache_compaction_amd as ks
import oracle as O
from parity_util import announce, f64, gate
from workloads import (KS_NEVER, PAGED_DECODE, TRAIN_4K, build_decode_batch, build_trace,
                       check_trace, normal_tensor, workload_rng)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


def _gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


# ---------------------------------------------------------------------------
# token-table compaction
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,MB,seed,with_pos,in_place_n", [
    (1, 4097, 1, False, False), (3, 10000, 2, True, False), (5, 12288, 3, False, True),
    (64, 65537, 4, True, False), (2, 8193, 5, True, True)])
def test_compact_long_token_tables(B, MB, seed, with_pos, in_place_n):
    rng = np.random.default_rng(seed)
    tin = rng.integers(0, 2**31 - 1, size=(B, MB), dtype=np.int32)
    n = rng.integers(0, MB + 1, size=B).astype(np.int32)
    n[0] = MB
    if B > 2:
        n[1], n[2] = 0, MB - 1
    keep = (rng.random((B, MB)) < rng.random((B, 1))).astype(np.uint8)
    keep[keep == 1] = rng.integers(1, 256, size=int(keep.sum()), dtype=np.uint8)  # any nonzero
    if B > 3:
        keep[3] = 0
    pin = rng.integers(0, 10**6, size=(B, MB), dtype=np.int32) if with_pos else None
    rt, rn = O.compact_block_table(tin, n, keep)
    tg, ng, kg = _gpu(tin), _gpu(n), _gpu(keep)
    tout = torch.full((B, MB), 7, dtype=torch.int32, device=DEV)
    nout = ng if in_place_n else torch.empty(B, dtype=torch.int32, device=DEV)
    pin_g = _gpu(pin) if with_pos else None
    pout = torch.full((B, MB), 7, dtype=torch.int32, device=DEV) if with_pos else None
    ks.ks_compact_block_table(tg, ng, kg, tout, nout, pin_g, pout)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(tout.cpu().numpy(), rt)
    np.testing.assert_array_equal(nout.cpu().numpy(), rn)
    if with_pos:
        rp, _ = O.compact_block_table(pin, n, keep)
        np.testing.assert_array_equal(pout.cpu().numpy(), rp)


def _oracle_rounds(table, nblk, keeps, pos=None):
    """Events applied one by one with the oracle's single-event splice (an
    all-keep splice when there is no event)."""
    if keeps.shape[0] == 0:
        keeps = np.ones((1,) + table.shape, np.uint8)
    t, n, p = table, np.clip(nblk, 0, table.shape[1]), pos
    for r in range(keeps.shape[0]):
        t2, n2 = O.compact_block_table(t, n, keeps[r])
        if p is not None:
            p, _ = O.compact_block_table(p, n, keeps[r])
        t, n = t2, n2
    return t, n, p


@pytest.mark.parametrize("B,MB,R,seed,with_pos", [
    (1, 4097, 1, 0, True), (3, 65536, 3, 1, False), (4, 20000, 0, 2, True),
    (5, 9999, 9, 3, True), (2, 30001, 64, 4, False)])
def test_compact_rounds_long_rows(B, MB, R, seed, with_pos):
    """Several events in one launch on rows above 4096 entries (survival
    bits on chip) vs the oracle's event-by-event splice."""
    rng = np.random.default_rng(600 + seed)
    table = rng.integers(0, 2**31 - 1, size=(B, MB)).astype(np.int32)
    pos = rng.integers(0, 2**31 - 1, size=(B, MB)).astype(np.int32) if with_pos else None
    nblk = rng.integers(-5, MB + 20, size=B).astype(np.int32)      # clamped on both sides
    nblk[0] = MB
    if B > 1:
        nblk[1] = 0 if seed % 2 else MB - 1
    p_keep = 1.0 - 0.5 / max(R, 1)
    keeps = (rng.random((R, B, MB)) < p_keep).astype(np.uint8)
    keeps[keeps == 1] = rng.integers(1, 256, size=int(keeps.sum()), dtype=np.uint8)
    rt, rn, rp = _oracle_rounds(table, nblk, keeps, pos)
    out = torch.full((B, MB), 7, dtype=torch.int32, device=DEV)
    po = torch.full((B, MB), 7, dtype=torch.int32, device=DEV) if with_pos else None
    n_in = _gpu(nblk)
    kg = _gpu(keeps) if R else torch.zeros((0, B, MB), dtype=torch.uint8, device=DEV)
    ks.ks_compact_block_table_rounds(_gpu(table), n_in, kg, out, n_in,
                                     _gpu(pos) if with_pos else None, po)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), rt)
    np.testing.assert_array_equal(n_in.cpu().numpy(), rn)         # lengths in place
    if with_pos:
        np.testing.assert_array_equal(po.cpu().numpy(), rp)


@pytest.mark.parametrize("MB,seed", [(40001, 0), (65536, 1), (4103, 2)])
def test_compact_rounds_runs_of_flags(MB, seed):
    """Flags in runs, as eviction writes them (whole 64-flag windows of one
    value, with run ends at any offset), with keep runs of 1, of other nonzero
    bytes and of mixed nonzero bytes, on rows that start at every alignment
    (odd row lengths), vs the oracle's event-by-event splice."""
    rng = np.random.default_rng(900 + seed)
    B, R = 7, 5
    table = rng.integers(0, 2**31 - 1, size=(B, MB)).astype(np.int32)
    pos = rng.integers(0, 2**31 - 1, size=(B, MB)).astype(np.int32)
    nblk = rng.integers(MB // 2, MB + 1, size=B).astype(np.int32)
    nblk[0] = MB
    keeps = np.ones((R, B, MB), np.uint8)
    for r in range(R):
        for b in range(B):
            row = keeps[r, b]
            for _ in range(int(rng.integers(0, 6))):       # evicted runs
                a = int(rng.integers(0, MB))
                row[a:a + int(rng.integers(1, 3000))] = 0
            kind = (r + b) % 4
            if kind == 1:                                  # keep written as 0xff
                row[row == 1] = 255
            elif kind == 2:                                # a run of another value
                a = int(rng.integers(0, MB))
                seg = row[a:a + int(rng.integers(1, 5000))]
                seg[seg == 1] = int(rng.integers(2, 256))
            elif kind == 3:                                # single odd bytes among ones
                idx = rng.integers(0, MB, size=8)
                row[idx] = np.where(row[idx] == 1, 7, row[idx])
    keeps[:, 6] = 0                                        # a row evicted whole
    rt, rn, rp = _oracle_rounds(table, nblk, keeps, pos)
    out = torch.full((B, MB), 7, dtype=torch.int32, device=DEV)
    po = torch.full((B, MB), 7, dtype=torch.int32, device=DEV)
    n_out = torch.empty(B, dtype=torch.int32, device=DEV)
    ks.ks_compact_block_table_rounds(_gpu(table), _gpu(nblk), _gpu(keeps), out, n_out,
                                     _gpu(pos), po)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), rt)
    np.testing.assert_array_equal(n_out.cpu().numpy(), rn)
    np.testing.assert_array_equal(po.cpu().numpy(), rp)


def test_compact_rounds_token_batch():
    db = build_decode_batch(workload_rng(PAGED_DECODE), 64, block=1)
    out, n, _ = ks.ks_compact_block_table_rounds(_gpu(db.table0), _gpu(db.nblk0),
                                                 _gpu(db.keeps))
    torch.cuda.synchronize()
    rt, rn, _ = _oracle_rounds(db.table0, db.nblk0, db.keeps)
    np.testing.assert_array_equal(out.cpu().numpy(), rt)
    np.testing.assert_array_equal(n.cpu().numpy(), rn)
    np.testing.assert_array_equal(rn, db.live_len + 1)


# ---------------------------------------------------------------------------
# decode and append over single-token blocks
# ---------------------------------------------------------------------------
def _direct_bs1(B, Hq, Hkv, lens, seed, extra=7):
    D = 128
    MT = max(int(max(lens)), 1)
    NT = int(sum(lens)) + extra
    perm = np.random.default_rng(seed).permutation(NT).astype(np.int32)
    table = np.full((B, MT), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :lens[b]] = perm[off:off + lens[b]]
        off += int(lens[b])
    kp = normal_tensor((NT, Hkv, D), seed + 1, 0.5, torch.bfloat16, DEV)
    vp = normal_tensor((NT, Hkv, D), seed + 2, 0.5, torch.bfloat16, DEV)
    q = normal_tensor((B, Hq, D), seed + 3, 0.5, torch.bfloat16, DEV)
    used = np.zeros(NT, bool)
    used[perm[:off]] = True
    if (~used).any():            # slots no sequence lists hold NaN
        idx = torch.from_numpy(np.nonzero(~used)[0]).to(DEV)
        kp[idx] = float("nan")
        vp[idx] = float("nan")
    return q, kp, vp, table


@pytest.mark.parametrize("Hq,Hkv,seed", [(32, 8, 1), (8, 4, 2), (4, 4, 3), (12, 4, 4),
                                         (12, 2, 5)])
def test_decode_bs1_ragged_lengths(Hq, Hkv, seed):
    # 256 and 768: one split of 16 or of 48 groups of 16 tokens (this small
    # grid takes 16-group splits)
    lens = np.array([0, 1, 15, 16, 17, 255, 256, 257, 767, 768, 769, 1537, 3001], np.int32)
    B = len(lens)
    q, kp, vp, table = _direct_bs1(B, Hq, Hkv, lens, 100 + seed)
    out, lse = ks.ks_paged_decode_bs1(q, kp, vp, _gpu(table), _gpu(lens))
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and math.isinf(lse[0, 0].item()) and lse[0, 0].item() < 0
    kh = kp.float().cpu().numpy()[:, :, None]
    vh = vp.float().cpu().numpy()[:, :, None]
    ro, rl = O.paged_decode(f64(q[1:]), kh, vh, table[1:], lens[1:])
    gate(out[1:], ro, "bf16", "decode bs1 out")
    gate(lse[1:], rl, "bf16", "decode bs1 lse")


# 8 kv heads (the workload's) with 1, 2 or 4 query heads per kv head, with
# and without the in-kernel rotation of the query: lengths of a few tokens,
# around the 16-token groups and 768-token splits, and a length past the
# table's capacity (clamped to the row)
@pytest.mark.parametrize("Hq,seed", [(8, 11), (16, 12), (32, 13)])
@pytest.mark.parametrize("rotate", [False, True])
def test_decode_bs1_eight_kv_heads(Hq, seed, rotate):
    Hkv, D = 8, 128
    lens = np.array([0, 1, 2, 3, 15, 16, 17, 255, 767, 768, 769, 1537, 2500], np.int32)
    B = len(lens)
    q, kp, vp, table = _direct_bs1(B, Hq, Hkv, lens, 500 + seed)
    lg = lens.copy()
    lg[-1] = table.shape[1] + 40                  # beyond the row: clamped to MT
    pos = (np.arange(B, dtype=np.int32) * 977 + 13) if rotate else None
    if rotate:
        out, lse = ks.ks_paged_decode_rope(q, _gpu(pos), kp, vp, _gpu(table), _gpu(lg))
    else:
        out, lse = ks.ks_paged_decode_bs1(q, kp, vp, _gpu(table), _gpu(lg))
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    qh = f64(q[1:])
    if rotate:
        qh = O.rope(qh[:, None], pos[1:, None])[:, 0]
    lens_ref = lens[1:].copy()
    lens_ref[-1] = table.shape[1]
    kh = kp.float().cpu().numpy()[:, :, None]
    vh = vp.float().cpu().numpy()[:, :, None]
    ro, rl = O.paged_decode(qh, kh, vh, table[1:], lens_ref)
    gate(out[1:], ro, "bf16", f"decode bs1 out Hq={Hq} rotate={rotate}")
    gate(lse[1:], rl, "bf16", f"decode bs1 lse Hq={Hq} rotate={rotate}")


def test_decode_bs1_rope_matches_separate_rotation():
    """The in-kernel rotation of the query gives the same bits as rotating it
    first with ks_rope_logical."""
    lens = np.array([300, 1, 700], np.int32)
    q, kp, vp, table = _direct_bs1(3, 32, 8, lens, 600)
    pos = torch.tensor([12345, 7, 99999], dtype=torch.int32, device=DEV)
    o1, l1 = ks.ks_paged_decode_rope(q, pos, kp, vp, _gpu(table), _gpu(lens))
    qr = q.clone()
    ks.ks_rope_logical(qr[:, None], None, pos[:, None].contiguous())
    o2, l2 = ks.ks_paged_decode_bs1(qr, kp, vp, _gpu(table), _gpu(lens))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_bs1_invalid_slot_in_a_later_split():
    lens = np.array([40, 40, 1600], np.int32)
    q, kp, vp, table = _direct_bs1(3, 32, 8, lens, 700)
    table[1, 33] = kp.shape[0] + 5          # out of range
    table[2, 1500] = -3                     # past the first split (256 or 768 tokens)
    out, _ = ks.ks_paged_decode_bs1(q, kp, vp, _gpu(table), _gpu(lens))
    torch.cuda.synchronize()
    assert torch.isfinite(out[0].float()).all()
    assert torch.isnan(out[1].float()).all() and torch.isnan(out[2].float()).all()


def test_decode_bs1_invalid_slot_gives_nan_not_fault():
    lens = np.array([40, 40, 40], np.int32)
    q, kp, vp, table = _direct_bs1(3, 4, 1, lens, 200)
    table[1, 33] = kp.shape[0] + 5          # out of range, one lane's slot
    table[2, 39] = -3
    out, _ = ks.ks_paged_decode_bs1(q, kp, vp, _gpu(table), _gpu(lens))
    torch.cuda.synchronize()
    assert torch.isfinite(out[0].float()).all()
    assert torch.isnan(out[1].float()).all() and torch.isnan(out[2].float()).all()


def test_append_kv_bs1_rotates_and_places():
    lens = np.array([1, 16, 17, 40, 0], np.int32)      # counting the new token
    B, Hkv, D = len(lens), 4, 128
    _, kp, vp, table = _direct_bs1(B, 8, Hkv, lens, 300)
    kp = torch.nan_to_num(kp)
    vp = torch.nan_to_num(vp)
    k0, v0 = kp.clone(), vp.clone()
    k_new = normal_tensor((B, Hkv, D), 301, 0.5, torch.bfloat16, DEV)
    v_new = normal_tensor((B, Hkv, D), 302, 0.5, torch.bfloat16, DEV)
    pos = np.array([0, 17, 4099, 65791, 5], np.int32)
    ks.ks_append_kv_bs1(k_new, v_new, _gpu(pos), _gpu(table), _gpu(lens), kp, vp)
    torch.cuda.synchronize()
    ref = O.rope(f64(k_new)[:, None], pos[:, None])[:, 0]
    touched = torch.zeros(kp.shape[:2], dtype=torch.bool, device=DEV)
    for b in range(B):
        if lens[b] < 1:
            continue
        p = int(table[b, lens[b] - 1])
        got = f64(kp[p])
        assert np.all(np.abs(got - ref[b]) <= np.abs(ref[b]) * 2.0**-8 + 1e-6), b
        assert torch.equal(vp[p], v_new[b])
        touched[p] = True
    assert torch.equal(kp[~touched], k0[~touched]) and torch.equal(vp[~touched], v0[~touched])


def test_token_granular_batch_full_size():
    """The 64-sequence decode batch with single-token blocks: 4k-16k live
    tokens at any length, 1-6 token-run events compacted one call per event
    (rows of up to 65k entries), RoPE of q, append of the new token, decode.
    Tables bit-exact; outputs of 8 sampled sequences against the oracle."""
    cfg = PAGED_DECODE
    db = build_decode_batch(workload_rng(PAGED_DECODE), cfg.batch, block=1)
    B, MT = db.table0.shape
    NT = db.num_pool_blocks
    Hq, Hkv, D = cfg.Hq, cfg.Hkv, cfg.D
    kp = normal_tensor((NT, Hkv, D), 8001, 0.5, torch.bfloat16, DEV)
    vp = normal_tensor((NT, Hkv, D), 8002, 0.5, torch.bfloat16, DEV)
    # evicted tokens hold NaN: any read of them would show
    dead = np.concatenate([db.table0[b, x0:x1] for b in range(B) for (x0, x1) in db.runs[b]])
    kp[_gpu(dead.astype(np.int64))] = float("nan")
    vp[_gpu(dead.astype(np.int64))] = float("nan")
    q_raw = normal_tensor((B, Hq, D), 8003, 0.5, torch.bfloat16, "cpu")
    k_new = normal_tensor((B, Hkv, D), 8004, 0.5, torch.bfloat16, DEV)
    v_new = normal_tensor((B, Hkv, D), 8005, 0.5, torch.bfloat16, DEV)
    ta, tb = _gpu(db.table0), torch.empty((B, MT), dtype=torch.int32, device=DEV)
    na, nb = _gpu(db.nblk0), torch.empty(B, dtype=torch.int32, device=DEV)
    for r in range(db.keeps.shape[0]):
        ks.ks_compact_block_table(ta, na, _gpu(db.keeps[r]), tb, nb)
        ta, tb, na, nb = tb, ta, nb, na
    seq_lens = _gpu((db.live_len + 1).astype(np.int32))
    pos = _gpu(db.pos.astype(np.int32))
    q = q_raw.to(DEV)[:, None].contiguous()
    ks.ks_rope_logical(q, None, pos[:, None].contiguous())
    ks.ks_append_kv_bs1(k_new, v_new, pos, ta, seq_lens, kp, vp)
    out, lse = ks.ks_paged_decode_bs1(q[:, 0].contiguous(), kp, vp, ta, seq_lens)
    torch.cuda.synchronize()
    rt, rn = db.table0, db.nblk0
    for r in range(db.keeps.shape[0]):
        rt, rn = O.compact_block_table(rt, rn, db.keeps[r])
    np.testing.assert_array_equal(ta.cpu().numpy(), rt)
    np.testing.assert_array_equal(na.cpu().numpy(), rn)
    assert torch.isfinite(out.float()).all()
    L = db.live_len + 1
    qr = O.rope(f64(q_raw)[:, None], db.pos[:, None])[:, 0]
    knr = O.rope(f64(k_new)[:, None], db.pos[:, None])[:, 0]
    for b in (0, 1, 7, 19, 31, 42, 55, 63):
        slots = rt[b, :L[b]]
        kh = kp[_gpu(slots[:-1].astype(np.int64))].float().cpu().numpy()
        vh = vp[_gpu(slots[:-1].astype(np.int64))].float().cpu().numpy()
        kh = np.concatenate([kh, knr[b][None]], 0)[:, :, None]      # new token: oracle's rope
        vh = np.concatenate([vh, f64(v_new[b])[None]], 0)[:, :, None]
        ro, rl = O.paged_decode(qr[b:b + 1], kh, vh, np.arange(L[b])[None], L[b:b + 1])
        gate(out[b:b + 1], ro, "bf16", f"token decode seq {b}")
        gate(lse[b:b + 1], rl, "bf16", f"token decode lse seq {b}")


# ---------------------------------------------------------------------------
# training on an unpadded (token-granular) trace
# ---------------------------------------------------------------------------
def test_masked_attention_on_token_granular_trace():
    cfg = TRAIN_4K
    rng = np.random.default_rng(2222)
    tr = build_trace(rng, cfg.N, cfg.P + 5, cfg.budget, "recent", turn_len=(37, 301),
                     granule=1)
    check_trace(tr)
    assert any(t % 16 for t in tr.events)
    e = tr.e[None].astype(np.int64)
    N, Hq, Hkv, D = cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    bf = torch.bfloat16
    q, k, v, do = (normal_tensor((1, N, h, D), s, 0.5, bf, DEV)
                   for h, s in ((Hq, 11), (Hkv, 12), (Hkv, 13), (Hq, 14)))
    eg = _gpu(tr.e[None].astype(np.int32))
    o, lse = ks.ks_evict_attn_fwd(q, k, v, eg)
    dq, dk, dv = ks.ks_evict_attn_bwd(q, k, v, eg, o, lse, do)
    torch.cuda.synchronize()
    ro, rl = O.attn_fwd(f64(q), f64(k), f64(v), e)
    rdq, rdk, rdv = O.attn_bwd(f64(q), f64(k), f64(v), e, f64(do))
    gate(o, ro, "bf16", "O")
    gate(lse, rl, "bf16", "LSE")
    gate(dq, rdq, "bf16grad", "dQ")
    gate(dk, rdk, "bf16grad", "dK")
    gate(dv, rdv, "bf16grad", "dV")


# ---------------------------------------------------------------------------
# input checks
# ---------------------------------------------------------------------------
def test_input_checks_count_violations():
    rng = np.random.default_rng(900)
    B, N = 5, 3001
    e = np.full((B, N), KS_NEVER, np.int32)
    e[:, :N - 1] = np.arange(1, N)[None] + rng.integers(0, 50, size=(B, N - 1))
    for b in range(1, B):          # plant violations
        idx = rng.choice(N, size=b * 7, replace=False)
        e[b, idx] = idx - rng.integers(0, 3, size=idx.size)
    got = ks.ks_check_eviction_record(_gpu(e))
    for BS, NB, MB in ((16, 300, 190), (1, 5000, 3001)):
        table = rng.integers(0, NB, size=(B, MB)).astype(np.int32)
        table[1, 5] = NB
        table[2, 0] = -1
        table[3, MB - 1] = NB + 100
        seq = rng.integers(1, BS * MB + 1, size=B).astype(np.int32)
        seq[3] = BS * MB
        seq[4] = BS * MB + 3          # longer than the row
        bt = ks.ks_check_block_table(_gpu(table), _gpu(seq), NB, BS)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bt.cpu().numpy(), O.count_bad_table(table, seq, NB, BS))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), O.count_bad_e(e))
    assert got[0].item() == 0
