"""GPU parity: block-table compaction (bit-exact) and RoPE at logical
positions, through the C ABI, against the fp64 oracle."""
import numpy as np
import pytest
import torch

import kv_cache_compaction_amd as ks
import oracle as O
from parity_util import announce, f64
from workloads import (PAGED_DECODE, TINY_F32, build_decode_batch, config_trace_batch,
                       normal_tensor, trace_blocks_keep, workload_rng)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


def _gpu(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t if dtype is None else t.to(dtype)


def test_compact_tiny512_table():
    (tr,), _ = config_trace_batch(TINY_F32)
    perm = np.random.default_rng(7).permutation(32).astype(np.int32)[None]
    keep = trace_blocks_keep(tr)[None]
    nblk = np.array([32], np.int32)
    out, n, _ = ks.ks_compact_block_table(_gpu(perm), _gpu(nblk), _gpu(keep))
    ref, rn = O.compact_block_table(perm, nblk, keep)
    torch.cuda.synchronize()
    assert int(n.cpu()[0]) == int(rn[0]) == 16
    np.testing.assert_array_equal(out.cpu().numpy(), ref)


def test_compact_decode64_rounds_pingpong():
    db = build_decode_batch(workload_rng(PAGED_DECODE), 64)
    B, MB = db.table0.shape
    ta, tb = _gpu(db.table0), torch.empty((B, MB), dtype=torch.int32, device=DEV)
    na, nb = _gpu(db.nblk0), torch.empty(B, dtype=torch.int32, device=DEV)
    pos0 = np.tile(np.arange(MB, dtype=np.int32), (B, 1))
    pa, pb = _gpu(pos0), torch.empty((B, MB), dtype=torch.int32, device=DEV)
    rt, rn, rp = db.table0, db.nblk0, pos0
    for r in range(db.keeps.shape[0]):
        keep = _gpu(db.keeps[r])
        ks.ks_compact_block_table(ta, na, keep, tb, nb, pa, pb)
        ta, tb, na, nb, pa, pb = tb, ta, nb, na, pb, pa
        rt2, rn2 = O.compact_block_table(rt, rn, db.keeps[r])
        rp2, _ = O.compact_block_table(rp, rn, db.keeps[r])
        rt, rn, rp = rt2, rn2, rp2
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ta.cpu().numpy(), rt)
        np.testing.assert_array_equal(na.cpu().numpy(), rn)
        np.testing.assert_array_equal(pa.cpu().numpy(), rp)
    # retained tokens conserved: live blocks plus the decode block
    assert np.array_equal(16 * (rn.astype(np.int64) - 1), db.live_len.astype(np.int64))


def _oracle_rounds(table, nblk, keeps, pos=None):
    """Events applied one by one with the oracle's single-event splice; with no
    event the table is only normalised (-1 past its length), i.e. an all-keep
    splice."""
    if keeps.shape[0] == 0:
        keeps = np.ones((1,) + table.shape, np.uint8)
    t, n, p = table, nblk, pos
    for r in range(keeps.shape[0]):
        t2, n2 = O.compact_block_table(t, n, keeps[r])
        if p is not None:
            p, _ = O.compact_block_table(p, n, keeps[r])
        t, n = t2, n2
    return t, n, p


def test_compact_rounds_decode64_one_launch():
    """All events of the decode workload in one launch equal the event-by-event oracle."""
    db = build_decode_batch(workload_rng(PAGED_DECODE), 64)
    B, MB = db.table0.shape
    pos0 = np.tile(np.arange(MB, dtype=np.int32), (B, 1))
    out, n, pos = ks.ks_compact_block_table_rounds(_gpu(db.table0), _gpu(db.nblk0),
                                                   _gpu(db.keeps), pos_in=_gpu(pos0))
    rt, rn, rp = _oracle_rounds(db.table0, db.nblk0, db.keeps, pos0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), rt)
    np.testing.assert_array_equal(n.cpu().numpy(), rn)
    np.testing.assert_array_equal(pos.cpu().numpy(), rp)


@pytest.mark.parametrize("B,MB,R,seed", [(1, 1, 1, 0), (3, 5, 0, 1), (4, 4096, 3, 2),
                                         (5, 1001, 12, 3), (2, 64, 64, 4), (6, 333, 8, 5)])
def test_compact_rounds_random_and_edges(B, MB, R, seed):
    """R events in one launch vs the oracle: ragged widths, zero events, more
    events than are preloaded, the widest row, empty and clamped lengths."""
    rng = np.random.default_rng(100 + seed)
    table = rng.integers(0, 2**31 - 1, size=(B, MB)).astype(np.int32)
    pos = rng.integers(0, 2**31 - 1, size=(B, MB)).astype(np.int32)
    nblk = rng.integers(0, MB + 1, size=B).astype(np.int32)
    nblk[0] = MB
    if B > 1:
        nblk[1] = 0
    if B > 4:
        nblk[4] = MB + 7     # clamped to MB
    keeps = (rng.random((R, B, MB)) < 0.85).astype(np.uint8)
    if B > 2 and R > 0:
        keeps[:, 2] = 1
    if B > 3 and R > 1:
        keeps[1, 3] = 0
    out, n, po = ks.ks_compact_block_table_rounds(_gpu(table), _gpu(nblk), _gpu(keeps),
                                                  pos_in=_gpu(pos))
    rt, rn, rp = _oracle_rounds(table, np.clip(nblk, 0, MB), keeps, pos)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), rt)
    np.testing.assert_array_equal(n.cpu().numpy(), rn)
    np.testing.assert_array_equal(po.cpu().numpy(), rp)


# widths that are a multiple of 16 (64, 2048, 4096) take the whole-row
# vector kernel, the others the entry-by-entry one; rows past 4096 entries
# are split over several workgroups
@pytest.mark.parametrize("B,MB,seed,with_pos", [
    (1, 1, 0, False), (3, 5, 1, False), (7, 4096, 2, False), (2, 10000, 3, False),
    (5, 4097, 4, False), (6, 64, 5, True), (5, 2048, 6, True), (4, 4096, 7, True),
    (6, 4088, 8, True)])
def test_compact_random_and_edges(B, MB, seed, with_pos):
    rng = np.random.default_rng(seed)
    table = rng.integers(0, 2**31 - 1, size=(B, MB)).astype(np.int32)
    pos = rng.integers(0, 2**31 - 1, size=(B, MB)).astype(np.int32)
    nblk = rng.integers(0, MB + 1, size=B).astype(np.int32)
    nblk[0] = MB
    if B > 1:
        nblk[1] = 0
    if B > 4:
        nblk[4] = MB + 7     # clamped to MB
    keep = (rng.random((B, MB)) < 0.7).astype(np.uint8)
    if B > 2:
        keep[2] = 1
    if B > 3:
        keep[3] = 0
    out, n, po = ks.ks_compact_block_table(_gpu(table), _gpu(nblk), _gpu(keep),
                                           pos_in=_gpu(pos) if with_pos else None)
    nb = np.clip(nblk, 0, MB)
    ref, rn = O.compact_block_table(table, nb, keep)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), ref)
    np.testing.assert_array_equal(n.cpu().numpy(), rn)
    if with_pos:
        rp, _ = O.compact_block_table(pos, nb, keep)
        np.testing.assert_array_equal(po.cpu().numpy(), rp)


def test_compact_rejects_aliasing_on_device():
    t = torch.zeros((2, 8), dtype=torch.int32, device=DEV)
    n = torch.full((2,), 8, dtype=torch.int32, device=DEV)
    k = torch.ones((2, 8), dtype=torch.uint8, device=DEV)
    with pytest.raises(ks.KSError):
        ks.ks_compact_block_table(t, n, k, t, n)


@pytest.mark.parametrize("D", [64, 48, 256])
def test_rope_f32_tiny512_positions(D):
    B, N, Hq, Hkv = 1, 512, 1, 1
    q = normal_tensor((B, N, Hq, D), 11)
    k = normal_tensor((B, N, Hkv, D), 12)
    pos = np.arange(N, dtype=np.int32)[None]
    qg, kg = q.to(DEV), k.to(DEV)
    ks.ks_rope_logical(qg, kg, _gpu(pos))
    torch.cuda.synchronize()
    np.testing.assert_allclose(f64(qg), O.rope(f64(q), pos), atol=1e-5, rtol=0)
    np.testing.assert_allclose(f64(kg), O.rope(f64(k), pos), atol=1e-5, rtol=0)


@pytest.mark.parametrize("D", [16, 32, 64, 96, 128, 256])
def test_rope_bf16_large_logical_positions(D):
    B, N, Hq, Hkv = 3, 37, 8, 2
    q = normal_tensor((B, N, Hq, D), 21, 0.5, torch.bfloat16)
    k = normal_tensor((B, N, Hkv, D), 22, 0.5, torch.bfloat16)
    pos = np.random.default_rng(23).integers(0, 65792, size=(B, N)).astype(np.int32)
    pos[0, :4] = [0, 1, 65535, 65791]
    qg, kg = q.to(DEV), k.to(DEV)
    ks.ks_rope_logical(qg, kg, _gpu(pos))
    torch.cuda.synchronize()
    for got, raw in ((qg, q), (kg, k)):
        ref = O.rope(f64(raw), pos)
        err = np.abs(f64(got) - ref)
        # one rounding to bf16 (2^-9 relative) plus fp32 arithmetic
        assert np.all(err <= np.abs(ref) * 2.0**-8 + 1e-6), err.max()
    # inverse undoes forward up to the two roundings
    ks.ks_rope_logical(qg, None, _gpu(pos), inverse=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(f64(qg), f64(q), atol=2e-2, rtol=0)


def test_rope_physical_positions_differ():
    """Negative control: rotating at physical slots is not the logical RoPE."""
    q = normal_tensor((1, 64, 2, 128), 31, 0.5, torch.bfloat16).to(DEV)
    logical = torch.arange(1000, 1064, dtype=torch.int32, device=DEV)[None]
    physical = torch.arange(0, 64, dtype=torch.int32, device=DEV)[None]
    a, b = q.clone(), q.clone()
    ks.ks_rope_logical(a, None, logical)
    ks.ks_rope_logical(b, None, physical)
    torch.cuda.synchronize()
    assert (a.float() - b.float()).abs().max().item() > 0.1
