"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test checks the oracle against a closed form, a library routine, an
invariant the mathematics fixes, brute force, or a hand-derived worked
example, chosen so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from workloads import (KS_NEVER, PAGED_DECODE, SUMMARY_32K, TINY_F32, TRAINING_WORKLOADS,
                       build_decode_batch, build_trace, check_trace, config_trace_batch,
                       trace_blocks_keep, workload_rng)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def random_e(rng, N, p_never=0.3):
    """A random eviction record with e_j > j (some never evicted)."""
    e = np.empty(N, dtype=np.int64)
    for j in range(N):
        e[j] = KS_NEVER if rng.random() < p_never else rng.integers(j + 1, N + 1)
    return e


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def test_rope_pos0_identity():
    x = rnd((1, 5, 3, 8), 1)
    np.testing.assert_array_equal(O.rope(x, np.zeros((1, 5), int)), x)


def test_rope_complex_rotation_closed_form():
    """Rotate-half RoPE = multiplying (x_k + i x_{k+D/2}) by exp(i theta_k)."""
    D, base = 16, 10000.0
    x = rnd((2, 7, 2, D), 2)
    pos = np.random.default_rng(3).integers(0, 70000, size=(2, 7))
    y = O.rope(x, pos, base)
    for b, n, h in itertools.product(range(2), range(7), range(2)):
        for kk in range(D // 2):
            theta = pos[b, n] * base ** (-2.0 * kk / D)
            z = complex(x[b, n, h, kk], x[b, n, h, kk + D // 2]) * complex(
                math.cos(theta), math.sin(theta))
            assert abs(y[b, n, h, kk] - z.real) < 1e-12
            assert abs(y[b, n, h, kk + D // 2] - z.imag) < 1e-12


def test_rope_norm_relative_composition_inverse():
    D = 64
    x = rnd((1, 6, 1, D), 4)
    k = rnd((1, 6, 1, D), 5)
    m = np.array([[0, 5, 17, 1000, 40000, 65791]])
    n = np.array([[3, 1, 17, 12, 39999, 65536]])
    xm, kn = O.rope(x, m), O.rope(k, n)
    # norm preserved
    np.testing.assert_allclose(np.linalg.norm(xm, axis=-1),
                               np.linalg.norm(x, axis=-1), rtol=1e-13)
    # <R(m)q, R(n)k> = <R(m-n)q, k>
    lhs = (xm * kn).sum(-1)
    rhs = (O.rope(x, m - n) * k).sum(-1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-9)
    # R(a) R(b) = R(a+b)
    np.testing.assert_allclose(O.rope(O.rope(x, m), n), O.rope(x, m + n),
                               rtol=1e-9, atol=1e-9)
    # inverse o forward = id
    np.testing.assert_allclose(O.rope(xm, m, inverse=True), x, atol=1e-12)


# ---------------------------------------------------------------------------
# Masked attention forward
# ---------------------------------------------------------------------------
def _sdpa(q, k, v, mask=None, causal=False):
    """torch SDPA in fp64 on the CPU for one (b, h): q,k,v [N, D]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v),
        attn_mask=None if mask is None else torch.from_numpy(mask)[None, None],
        is_causal=causal)
    return out[0, 0].numpy()


def test_fwd_no_evictions_is_causal_sdpa():
    B, N, Hq, Hkv, D = 2, 77, 4, 2, 16
    q, k, v = rnd((B, N, Hq, D), 6), rnd((B, N, Hkv, D), 7), rnd((B, N, Hkv, D), 8)
    e = np.full((B, N), KS_NEVER)
    o, lse = O.attn_fwd(q, k, v, e)
    for b in range(B):
        for h in range(Hq):
            ref = _sdpa(q[b, :, h], k[b, :, h // 2], v[b, :, h // 2], causal=True)
            np.testing.assert_allclose(o[b, :, h], ref, atol=1e-12)


def test_fwd_band_is_local_attention():
    N, D, w = 64, 8, 9
    q, k, v = rnd((1, N, 1, D), 9), rnd((1, N, 1, D), 10), rnd((1, N, 1, D), 11)
    e = (np.arange(N) + w)[None]
    o, _ = O.attn_fwd(q, k, v, e)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    band = (j <= i) & (j > i - w)          # written independently of e
    ref = _sdpa(q[0, :, 0], k[0, :, 0], v[0, :, 0], mask=band)
    np.testing.assert_allclose(o[0, :, 0], ref, atol=1e-12)


def test_fwd_diagonal_only():
    N, D = 40, 16
    q, k, v = rnd((1, N, 2, D), 12), rnd((1, N, 1, D), 13), rnd((1, N, 1, D), 14)
    e = (np.arange(N) + 1)[None]
    o, lse = O.attn_fwd(q, k, v, e)
    for h in range(2):
        np.testing.assert_allclose(o[0, :, h], v[0, :, 0], atol=1e-13)
        sii = (q[0, :, h] * k[0, :, 0]).sum(-1) / math.sqrt(D)
        np.testing.assert_allclose(lse[0, h], sii, atol=1e-12)


def test_fwd_zero_keys_counts_live_set():
    """K = 0 gives uniform weights: LSE_i = log|live(i)| and, with one-hot
    values, O_i[j] = 1/|live(i)| exactly on the live set."""
    N = 48
    rng = np.random.default_rng(15)
    e = random_e(rng, N)[None]
    q = rnd((1, N, 1, N), 16)
    k = np.zeros((1, N, 1, N))
    v = np.eye(N)[None, :, None, :]
    o, lse = O.attn_fwd(q, k, v, e)
    for i in range(N):
        live = [j for j in range(i + 1) if e[0, j] > i]
        assert abs(lse[0, 0, i] - math.log(len(live))) < 1e-13
        expect = np.zeros(N)
        expect[live] = 1.0 / len(live)
        np.testing.assert_allclose(o[0, i, 0], expect, atol=1e-15)


def _brute_fwd(q, k, v, e, scale):
    N, D = q.shape
    o = np.zeros((N, D))
    lse = np.zeros(N)
    for i in range(N):
        s = {}
        for j in range(N):
            if j <= i and i < e[j]:
                s[j] = scale * sum(q[i, d] * k[j, d] for d in range(D))
        mx = max(s.values())
        z = sum(math.exp(x - mx) for x in s.values())
        lse[i] = mx + math.log(z)
        for j, x in s.items():
            o[i] += math.exp(x - lse[i]) * v[j]
    return o, lse


def test_fwd_brute_force_tiny_and_exhaustive():
    D = 4
    for N in range(1, 6):
        q, k, v = rnd((1, N, 1, D), 20 + N), rnd((1, N, 1, D), 30 + N), rnd((1, N, 1, D), 40 + N)
        choices = [list(range(j + 1, N + 1)) + [KS_NEVER] for j in range(N)]
        for ecomb in itertools.product(*choices):
            e = np.array(ecomb)[None]
            o, lse = O.attn_fwd(q, k, v, e)
            ob, lb = _brute_fwd(q[0, :, 0], k[0, :, 0], v[0, :, 0], e[0], 1 / math.sqrt(D))
            np.testing.assert_allclose(o[0, :, 0], ob, atol=1e-12)
            np.testing.assert_allclose(lse[0, 0], lb, atol=1e-12)
    N = 32
    rng = np.random.default_rng(50)
    e = random_e(rng, N)[None]
    q, k, v = rnd((1, N, 1, D), 51), rnd((1, N, 1, D), 52), rnd((1, N, 1, D), 53)
    o, lse = O.attn_fwd(q, k, v, e, row_chunk=7)
    ob, lb = _brute_fwd(q[0, :, 0], k[0, :, 0], v[0, :, 0], e[0], 1 / math.sqrt(D))
    np.testing.assert_allclose(o[0, :, 0], ob, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], lb, atol=1e-12)


def test_broken_records_give_empty_rows():
    """Records that break e_j > j (outside the method's preconditions): a
    token with e_j <= j is seen by no query, and a row that sees no key is an
    empty softmax (O = 0, LSE = -inf).  Brute force over every record with
    e_j in {0..N} and never, for N <= 4."""
    D = 3
    for N in range(1, 5):
        q, k, v = rnd((1, N, 1, D), 60 + N), rnd((1, N, 1, D), 70 + N), rnd((1, N, 1, D), 80 + N)
        for ecomb in itertools.product(*([list(range(0, N + 1)) + [KS_NEVER]] * N)):
            e = np.array(ecomb)[None]
            o, lse = O.attn_fwd(q, k, v, e)
            for i in range(N):
                vis = [j for j in range(i + 1) if i < e[0, j]]
                if not vis:
                    assert np.all(o[0, i, 0] == 0) and lse[0, 0, i] == -np.inf
                    continue
                qs = q[0, vis, 0].copy()
                qs[-1] = q[0, i, 0]          # the last causal row of the subset is query i
                ob, lb = _brute_fwd(qs, k[0, vis, 0], v[0, vis, 0],
                                    np.full(len(vis), KS_NEVER), 1 / math.sqrt(D))
                np.testing.assert_allclose(o[0, i, 0], ob[-1], atol=1e-12)
                np.testing.assert_allclose(lse[0, 0, i], lb[-1], atol=1e-12)


def test_broken_record_gradients_by_finite_differences():
    B, N, Hq, Hkv, D = 1, 16, 2, 1, 5
    rng = np.random.default_rng(86)
    e = random_e(rng, N)[None]
    e[0, [0, 1, 5, 6, 9]] = [0, 1, 2, 6, 3]        # e_j <= j: rows 0 and 1 see nothing
    q, k, v = rnd((B, N, Hq, D), 87), rnd((B, N, Hkv, D), 88), rnd((B, N, Hkv, D), 89)
    do = rnd((B, N, Hq, D), 90)
    o, _ = O.attn_fwd(q, k, v, e)
    assert np.all(o[0, :2] == 0)
    dq, dk, dv = O.attn_bwd(q, k, v, e, do)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    assert np.all(dq[0, :2] == 0)
    h = 1e-6
    pick = np.random.default_rng(91)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(20):
            idx = tuple(int(pick.integers(0, sz)) for sz in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            fp = _loss(*(xp if n == name else args[n] for n in "qkv"), e, do)
            fm = _loss(*(xm if n == name else args[n] for n in "qkv"), e, do)
            assert abs((fp - fm) / (2 * h) - g[idx]) < 1e-6, (name, idx)


def test_fwd_equals_reassembled_sequence_at_logical_positions():
    """The method's core claim: every row of the masked trace attention equals
    plain attention of that query over the re-assembled live keys, each
    rotated at its logical (original) position.  Rotating at physical slots
    instead must give a different answer."""
    rng = np.random.default_rng(60)
    tr = build_trace(rng, 512, 64, 256, "recent", turn_len=(64, 64))
    N, D = tr.N, 32
    e = tr.e[None].astype(np.int64)
    qr, kr, v = rnd((1, N, 1, D), 61), rnd((1, N, 1, D), 62), rnd((1, N, 1, D), 63)
    pos = np.arange(N)[None]
    q, k = O.rope(qr, pos), O.rope(kr, pos)
    o, _ = O.attn_fwd(q, k, v, e)
    worst_phys = 0.0
    for i in range(0, N, 7):
        live = O.live_keys(e[0], i)
        lk = O.rope(kr[:, live], live[None])            # logical positions
        s = (lk[0, :, 0] @ q[0, i, 0]) / math.sqrt(D)
        w = np.exp(s - s.max())
        ref = (w / w.sum()) @ v[0, live, 0]
        np.testing.assert_allclose(o[0, i, 0], ref, atol=1e-12)
        # negative control: physical slots 0..|live|-1, query at slot |live|-1
        pk = O.rope(kr[:, live], np.arange(len(live))[None])
        pq = O.rope(qr[:, i:i + 1], np.array([[len(live) - 1]]))
        s2 = (pk[0, :, 0] @ pq[0, 0, 0]) / math.sqrt(D)
        w2 = np.exp(s2 - s2.max())
        worst_phys = max(worst_phys, np.abs((w2 / w2.sum()) @ v[0, live, 0] - ref).max())
    assert worst_phys > 1e-3


def test_fwd_rows_matches_full():
    B, N, Hq, Hkv, D = 1, 100, 4, 2, 8
    rng = np.random.default_rng(70)
    e = random_e(rng, N)[None]
    q, k, v = rnd((B, N, Hq, D), 71), rnd((B, N, Hkv, D), 72), rnd((B, N, Hkv, D), 73)
    o, lse = O.attn_fwd(q, k, v, e, row_chunk=33)
    rows = np.array([0, 5, 50, 99])
    orr, lrr = O.attn_fwd_rows(q, k, v, e, 0, 3, rows)
    np.testing.assert_allclose(orr, o[0, rows, 3], atol=1e-13)
    np.testing.assert_allclose(lrr, lse[0, 3, rows], atol=1e-13)


# ---------------------------------------------------------------------------
# Masked attention backward
# ---------------------------------------------------------------------------
def _loss(q, k, v, e, do):
    o, _ = O.attn_fwd(q, k, v, e)
    return float((o * do).sum())


def test_bwd_central_finite_differences():
    B, N, Hq, Hkv, D = 1, 20, 2, 1, 6
    rng = np.random.default_rng(80)
    e = random_e(rng, N)[None]
    q, k, v = rnd((B, N, Hq, D), 81), rnd((B, N, Hkv, D), 82), rnd((B, N, Hkv, D), 83)
    do = rnd((B, N, Hq, D), 84)
    dq, dk, dv = O.attn_bwd(q, k, v, e, do)
    h = 1e-6
    pick = np.random.default_rng(85)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(25):
            idx = tuple(int(pick.integers(0, s)) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            fp = _loss(*(xp if n == name else args[n] for n in "qkv"), e, do)
            fm = _loss(*(xm if n == name else args[n] for n in "qkv"), e, do)
            assert abs((fp - fm) / (2 * h) - g[idx]) < 1e-6, (name, idx)


def test_bwd_matches_torch_autograd_sdpa():
    B, N, Hq, Hkv, D = 1, 96, 4, 2, 16
    rng = np.random.default_rng(90)
    e = random_e(rng, N, p_never=0.5)[None]
    q, k, v = rnd((B, N, Hq, D), 91), rnd((B, N, Hkv, D), 92), rnd((B, N, Hkv, D), 93)
    do = rnd((B, N, Hq, D), 94)
    dq, dk, dv = O.attn_bwd(q, k, v, e, do, row_chunk=40)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    mask = (j <= i) & (i < torch.from_numpy(e[0])[None, :])
    G = Hq // Hkv
    kk = tk.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vv = tv.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), kk, vv, attn_mask=mask)
    out.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


def test_raw_projection_gradients_are_inverse_rotations():
    """Gradients with respect to the raw (unrotated) q and k are the inverse
    rotation of the gradients with respect to the rotated ones: checked by
    torch autograd through a complex-number RoPE and masked SDPA in fp64."""
    B, N, Hq, Hkv, D = 1, 80, 4, 2, 16
    rng = np.random.default_rng(95)
    e = random_e(rng, N, p_never=0.4)[None]
    qr, kr, v = rnd((B, N, Hq, D), 96), rnd((B, N, Hkv, D), 97), rnd((B, N, Hkv, D), 98)
    do = rnd((B, N, Hq, D), 99)
    pos = (np.arange(N) + 1000)[None]
    dq, dk, _ = O.attn_bwd(O.rope(qr, pos), O.rope(kr, pos), v, e, do)
    gq, gk = O.rope(dq, pos, inverse=True), O.rope(dk, pos, inverse=True)
    tq = torch.tensor(qr, requires_grad=True)
    tk = torch.tensor(kr, requires_grad=True)
    inv = 10000.0 ** (-2.0 * torch.arange(D // 2, dtype=torch.float64) / D)
    rot = torch.polar(torch.ones(N, D // 2, dtype=torch.float64),
                      torch.from_numpy(pos[0]).double()[:, None] * inv[None])

    def rope(t):
        c = torch.complex(t[..., :D // 2], t[..., D // 2:]) * rot[None, :, None]
        return torch.cat([c.real, c.imag], -1)
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    mask = (j <= i) & (i < torch.from_numpy(e[0])[None, :])
    G = Hq // Hkv
    kk = rope(tk).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vv = torch.tensor(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    out = torch.nn.functional.scaled_dot_product_attention(
        rope(tq).permute(0, 2, 1, 3), kk, vv, attn_mask=mask)
    out.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    np.testing.assert_allclose(gq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(gk, tk.grad.numpy(), atol=1e-11)


def test_bwd_invariants_and_sampled_variants():
    B, N, Hq, Hkv, D = 2, 120, 4, 2, 8
    rng = np.random.default_rng(100)
    e = np.stack([random_e(rng, N), random_e(rng, N)])
    q, k, v = rnd((B, N, Hq, D), 101), rnd((B, N, Hkv, D), 102), rnd((B, N, Hkv, D), 103)
    do = rnd((B, N, Hq, D), 104)
    dq, dk, dv = O.attn_bwd(q, k, v, e, do, row_chunk=50)
    G = Hq // Hkv
    for b in range(B):
        for kv in range(Hkv):
            # softmax rows sum to 1: sum_j dV_j = sum_i sum_{h in group} dO_i
            np.testing.assert_allclose(dv[b, :, kv].sum(0),
                                       do[b, :, kv * G:(kv + 1) * G].sum((0, 1)), atol=1e-11)
    # bilinearity of S in (q, k): sum_i q_i.dq_i = sum_j k_j.dk_j
    np.testing.assert_allclose((q * dq).sum(), (k * dk).sum(), rtol=1e-10)
    rows = np.array([3, 64, 119])
    np.testing.assert_allclose(O.attn_bwd_rows(q, k, v, e, do, 1, 2, rows),
                               dq[1, rows, 2], atol=1e-12)
    keys = np.array([0, 7, 8, 60, 119])
    skd, svd = O.attn_bwd_keys(q, k, v, e, do, 1, 1, keys, row_chunk=31)
    np.testing.assert_allclose(skd, dk[1, keys, 1], atol=1e-12)
    np.testing.assert_allclose(svd, dv[1, keys, 1], atol=1e-12)


# ---------------------------------------------------------------------------
# Block-table compaction
# ---------------------------------------------------------------------------
def test_compaction_basic_properties():
    rng = np.random.default_rng(110)
    B, MB = 9, 50
    table = rng.integers(0, 10**6, size=(B, MB)).astype(np.int32)
    nblk = rng.integers(0, MB + 1, size=B).astype(np.int32)
    keep = (rng.random((B, MB)) < 0.6).astype(np.uint8)
    out, n = O.compact_block_table(table, nblk, keep)
    for b in range(B):
        kept_idx = np.nonzero(keep[b, :nblk[b]])[0]      # boolean-index form
        assert n[b] == len(kept_idx)
        np.testing.assert_array_equal(out[b, :n[b]], table[b, kept_idx])
        assert np.all(out[b, n[b]:] == -1)
    out1, n1 = O.compact_block_table(table, nblk, np.ones_like(keep))
    for b in range(B):
        np.testing.assert_array_equal(out1[b, :nblk[b]], table[b, :nblk[b]])
    out0, n0 = O.compact_block_table(table, nblk, np.zeros_like(keep))
    assert np.all(n0 == 0) and np.all(out0 == -1)


def test_compaction_rounds_equal_union_and_conserve_tokens():
    db = build_decode_batch(np.random.default_rng(120), 6, live_range=(256, 1024),
                            max_pos=4096)
    table, n = db.table0, db.nblk0
    for r in range(db.keeps.shape[0]):
        table, n = O.compact_block_table(table, n, db.keeps[r])
    for b in range(6):
        # union of all evicted runs, applied in one go on logical ids
        gone = set()
        for (x0, x1) in db.runs[b]:
            gone.update(range(x0, x1))
        logical = [x for x in range(int(db.nblk0[b])) if x not in gone]
        np.testing.assert_array_equal(table[b, :n[b]], db.table0[b, logical])
        # retained tokens conserved: live blocks + the fresh block
        assert 16 * (int(n[b]) - 1) == int(db.live_len[b])
        # logical order strictly increasing
        assert all(a < c for a, c in zip(logical, logical[1:]))


def test_tiny512_worked_example():
    with open(os.path.join(GOLDEN, "tiny512_trace.json")) as f:
        g = json.load(f)
    (tr,), _ = config_trace_batch(TINY_F32)
    assert tr.events == g["events"]
    e = tr.e.astype(np.int64)
    for t, spans in g["evicted"].items():
        for (a, b) in spans:
            assert np.all(e[a:b] == int(t))
    n_evicted = sum(b - a for spans in g["evicted"].values() for (a, b) in spans)
    assert int((e != KS_NEVER).sum()) == n_evicted
    pairs = int(sum(len(O.live_keys(e, i)) for i in range(tr.N)))
    assert pairs == g["live_pairs"]
    m = O.eviction_mask(e, np.arange(tr.N), tr.N)
    assert int(m.sum()) == g["live_pairs"]
    # block compaction of the 32-block table keeps exactly the final live blocks
    perm = np.random.default_rng(7).permutation(32).astype(np.int32)[None]
    keep = trace_blocks_keep(tr)[None]
    out, n = O.compact_block_table(perm, np.array([32]), keep)
    assert int(n[0]) == len(g["final_live_blocks"]) == 16
    np.testing.assert_array_equal(out[0, :16], perm[0, g["final_live_blocks"]])


# ---------------------------------------------------------------------------
# Paged decode
# ---------------------------------------------------------------------------
def _pool_from_trace(kr, v, live_tokens, rng, extra_blocks=3):
    """Lay the given token rows (trace order) into a permuted block pool."""
    Hkv, D = kr.shape[1], kr.shape[2]
    nb = (len(live_tokens) + 15) // 16
    NB = nb + extra_blocks
    perm = rng.permutation(NB)
    kp = np.full((NB, Hkv, 16, D), np.nan)
    vp = np.full((NB, Hkv, 16, D), np.nan)
    for s, tok in enumerate(live_tokens):
        kp[perm[s // 16], :, s % 16] = kr[tok]
        vp[perm[s // 16], :, s % 16] = v[tok]
    return kp, vp, perm[:nb]


def test_decode_equals_masked_trace_row():
    """Decode of token T over the compacted cache = row T of the masked trace
    attention (trainer replay equals generation)."""
    rng = np.random.default_rng(130)
    tr = build_trace(rng, 900, 64, 512, "recent", turn_len=(64, 160))
    check_trace(tr)
    N, Hq, Hkv, D = tr.N, 4, 2, 16
    T = N - 1                                   # the decoded token
    qr, kr, v = rnd((1, N, Hq, D), 131), rnd((1, N, Hkv, D), 132), rnd((1, N, Hkv, D), 133)
    pos = np.arange(N)[None]
    q, k = O.rope(qr, pos), O.rope(kr, pos)
    e = tr.e[None].astype(np.int64)
    o, lse = O.attn_fwd_rows(q, k, v, e, 0, 0, np.array([T]))
    live = O.live_keys(e[0], T)                 # includes T itself
    kp, vp, blocks = _pool_from_trace(k[0], v[0], live, rng)
    table = np.full((1, len(blocks) + 4), -1)
    table[0, :len(blocks)] = blocks
    out, dl = O.paged_decode(q[:, T], kp, vp, table, np.array([len(live)]))
    np.testing.assert_allclose(out[0, 0], o[0], atol=1e-12)
    np.testing.assert_allclose(dl[0, 0], lse[0], atol=1e-12)
    for h in range(Hq):
        oh, lh = O.attn_fwd_rows(q, k, v, e, 0, h, np.array([T]))
        np.testing.assert_allclose(out[0, h], oh[0], atol=1e-12)
    assert np.isfinite(out).all()               # NaN tail slots never read


def test_decode_no_evictions_is_last_causal_row():
    rng = np.random.default_rng(140)
    N, D = 53, 16
    q, k, v = rnd((N, D), 141), rnd((N, D), 142), rnd((N, D), 143)
    kp, vp, blocks = _pool_from_trace(k[:, None], v[:, None], list(range(N)), rng)
    table = np.array([list(blocks)])
    out, _ = O.paged_decode(q[None, N - 1:N], kp, vp, table, np.array([N]))
    ref = _sdpa(q, k, v, causal=True)[N - 1]
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-12)


# ---------------------------------------------------------------------------
# Generator invariants (inputs shared by both sides)
# ---------------------------------------------------------------------------
def test_generator_invariants_all_configs():
    for cfg in TRAINING_WORKLOADS:
        traces, _ = config_trace_batch(cfg)      # runs check_trace on each
        assert len(traces) == cfg.batch
    (t3, *_), _ = config_trace_batch(SUMMARY_32K)
    # re-prefill factor N/(B-(o+s)) of the paper's Fig. 3: 32768/6656 = 4.92
    assert abs(32768 / (8192 - 1536) - 4.92) < 0.01
    assert len(t3.events) == 5


def test_decode_batch_structure():
    db = build_decode_batch(workload_rng(PAGED_DECODE), 64)
    assert np.all(db.live_len % 16 == 0) and np.all(db.pos % 16 == 0)
    assert db.live_len.min() >= 4096 and db.live_len.max() <= 16384
    assert db.pos.max() <= 65536
    ids = np.concatenate([db.table0[b, :db.nblk0[b]] for b in range(64)])
    assert len(np.unique(ids)) == len(ids) == db.num_pool_blocks
    for b in range(64):
        assert 1 <= len(db.runs[b]) <= 6
        for (x0, x1) in db.runs[b]:
            assert x0 >= 1 and x1 <= db.nblk0[b] - 2


def test_continuation_layout_structure():
    """The long mixed traces continued by 256 decoded tokens: every live
    token sits in a listed block in trace order, block ids are unique, the
    fresh blocks follow at N, N + 16, ..., and the forced event's flags drop
    exactly the listed blocks its spans cover (whole blocks only)."""
    from workloads import LONG_MIXED_64K, continuation_layout
    traces, _ = config_trace_batch(LONG_MIXED_64K)
    N = LONG_MIXED_64K.N
    lay = continuation_layout(traces, N, 256, 128, np.random.default_rng(5005))
    B = len(traces)
    ids = np.concatenate([lay.table0[b, :lay.nblk0[b]] for b in range(B)])
    assert len(np.unique(ids)) == len(ids) == lay.num_pool_blocks
    assert np.all(lay.table0[np.arange(lay.table0.shape[1])[None] >= lay.nblk0[:, None]] == -1)
    assert lay.t_ev == N + 128
    for b, tr in enumerate(traces):
        live = lay.live_tok[b]
        assert len(live) == lay.live_len[b] == sum(y - x for x, y in tr.live_units)
        assert np.all(np.diff(live) > 0) and live.max() < N
        lg = lay.logical[b]
        assert len(lg) == lay.nblk0[b] and np.all(lg % 16 == 0)
        assert np.array_equal(lg[-16:], N + 16 * np.arange(16))
        assert np.array_equal(live.reshape(-1, 16), lg[:-16, None] + np.arange(16))
        gone = np.zeros(N + 256, bool)
        for x, y in lay.ev_spans[b]:
            assert x % 16 == 0 and y % 16 == 0 and y <= lay.t_ev
            gone[x:y] = True
        assert lay.ev_tokens[b] == gone.sum() > 0
        assert np.array_equal(lay.keep[b, :lay.nblk0[b]], ~gone[lg])
        assert not lay.keep[b, lay.nblk0[b]:].any()


# ---------------------------------------------------------------------------
# Single-token blocks (token-granular traces, tables and decode)
# ---------------------------------------------------------------------------
def test_token_granular_trace_decode_and_compaction():
    """With single-token blocks nothing is padded: turns end anywhere, the
    token table of the final live set is the splice of the per-token keep
    flags, and decode over it equals row T of the masked trace attention."""
    rng = np.random.default_rng(150)
    tr = build_trace(rng, 777, 37, 400, "recent", turn_len=(23, 97), granule=1)
    check_trace(tr)
    assert any(x % 16 for (x, _) in tr.turns)          # really unpadded
    N, Hq, Hkv, D = tr.N, 4, 2, 16
    T = N - 1
    qr, kr, v = rnd((1, N, Hq, D), 151), rnd((1, N, Hkv, D), 152), rnd((1, N, Hkv, D), 153)
    pos = np.arange(N)[None]
    q, k = O.rope(qr, pos), O.rope(kr, pos)
    e = tr.e[None].astype(np.int64)
    # token table before compaction: a permutation of pool slots
    NT = N + 5
    slots = rng.permutation(NT)[:N]
    kp = np.full((NT, Hkv, 1, D), np.nan)
    vp = np.full((NT, Hkv, 1, D), np.nan)
    kp[slots, :, 0], vp[slots, :, 0] = k[0], v[0]
    keep = (tr.e == KS_NEVER).astype(np.uint8)[None]
    table, n = O.compact_block_table(slots[None].astype(np.int32), np.array([N]), keep)
    live = O.live_keys(e[0], T)
    assert int(n[0]) == len(live)
    np.testing.assert_array_equal(table[0, :n[0]], slots[live])
    out, lse = O.paged_decode(q[:, T], kp, vp, table, n)
    for h in range(Hq):
        oh, lh = O.attn_fwd_rows(q, k, v, e, 0, h, np.array([T]))
        np.testing.assert_allclose(out[0, h], oh[0], atol=1e-12)
        np.testing.assert_allclose(lse[0, h], lh[0], atol=1e-12)


def test_decode_single_token_blocks_equal_16_token_blocks():
    """The same live tokens reached through 16-token blocks or through one
    slot per token give the same decode (the layout is not the math)."""
    rng = np.random.default_rng(160)
    L, Hq, Hkv, D = 83, 4, 1, 16
    kr, v = rnd((L, Hkv, D), 161), rnd((L, Hkv, D), 162)
    q = rnd((1, Hq, D), 163)
    kp16, vp16, blocks = _pool_from_trace(kr, v, list(range(L)), rng)
    slots = rng.permutation(L + 9)[:L]
    kp1 = np.full((L + 9, Hkv, 1, D), np.nan)
    vp1 = np.full((L + 9, Hkv, 1, D), np.nan)
    kp1[slots, :, 0], vp1[slots, :, 0] = kr, v
    o16, l16 = O.paged_decode(q, kp16, vp16, np.array([list(blocks)]), np.array([L]))
    o1, l1 = O.paged_decode(q, kp1, vp1, slots[None], np.array([L]))
    np.testing.assert_allclose(o1, o16, atol=1e-13)
    np.testing.assert_allclose(l1, l16, atol=1e-13)
    ref = _sdpa(q[0], kr[:, 0], v[:, 0])          # every head sees all L keys
    np.testing.assert_allclose(o1[0], ref, atol=1e-12)


def test_token_decode_batch_structure():
    db = build_decode_batch(workload_rng(PAGED_DECODE), 64, block=1)
    assert db.block == 1 and np.any(db.live_len % 16) and np.any(db.pos % 16)
    assert db.live_len.min() >= 4096 and db.live_len.max() <= 16384
    ids = np.concatenate([db.table0[b, :db.nblk0[b]] for b in range(64)])
    assert len(np.unique(ids)) == len(ids) == db.num_pool_blocks
    # replaying the rounds leaves exactly L_b + 1 slots (live tokens + the
    # decoded token's slot)
    out, n = db.table0, db.nblk0
    for r in range(db.keeps.shape[0]):
        out, n = O.compact_block_table(out, n, db.keeps[r])
    np.testing.assert_array_equal(n, db.live_len + 1)


# ---------------------------------------------------------------------------
# Input checks
# ---------------------------------------------------------------------------
def test_input_check_counts_hand_examples():
    # e_j <= j at j = 0 (e = 0), j = 3 (e = 3), j = 4 (e = -7); e_j = j + 1 is fine
    e = np.array([[0, 5, 9, 3, -7, 6], [1, 2, 3, 4, 5, KS_NEVER]])
    np.testing.assert_array_equal(O.count_bad_e(e), [3, 0])
    # 16-token blocks, pool of 10: row 0 reaches 2 entries (L = 17), one bad;
    # row 1 L = 0 reaches none; row 2 L = 65 > 16 * 4: the 4 entries, two bad,
    # plus one for the length; row 3 negative length
    t = np.array([[3, -1, 7, 7], [11, 12, 13, 14], [0, 10, 9, -2], [1, 1, 1, 1]])
    np.testing.assert_array_equal(O.count_bad_table(t, [17, 0, 65, -3], 10, 16), [1, 0, 3, 1])
    # single-token blocks: L = 3 reaches 3 entries
    np.testing.assert_array_equal(O.count_bad_table(t[:1], [3], 10, 1), [1])
