"""The allocation-free decode entry point (ks_paged_decode_noalloc) against
ks_paged_decode: same kernels, so the outputs must agree bit for bit, on two
calls in a row (the second with fewer sequences and a narrower table), and a
call that needs more than the library's scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import kv_cache_compaction_amd as ks
from parity_util import announce
from workloads import PAGED_DECODE, build_decode_batch, normal_tensor, workload_rng

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc_raw(q, kp, vp, table, lens, out, lse):
    """the C ABI call itself (no binding in between)"""
    lib = ks.load_library()
    B, Hq, D = q.shape
    NB, Hkv = kp.shape[0], kp.shape[1]
    st = lib.ks_paged_decode_noalloc(_p(q), _p(kp), _p(vp), _p(table), _p(lens), _p(out),
                                     _p(lse), B, Hq, Hkv, D, table.shape[1], NB, ks.KS_BF16,
                                     1.0 / np.sqrt(D),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, lib.ks_last_error().decode()


def test_noalloc_decode_matches_the_workspace_entry_point():
    db = build_decode_batch(workload_rng(PAGED_DECODE), PAGED_DECODE.batch)
    B, MB = db.table0.shape
    Hq, Hkv, D = PAGED_DECODE.Hq, PAGED_DECODE.Hkv, PAGED_DECODE.D
    NB = db.num_pool_blocks
    bf = torch.bfloat16
    kp = normal_tensor((NB, Hkv, 16, D), 4101, 0.5, bf, DEV)
    vp = normal_tensor((NB, Hkv, 16, D), 4102, 0.5, bf, DEV)
    q = normal_tensor((B, Hq, D), 4103, 0.5, bf, DEV)
    table = torch.from_numpy(db.table0).to(DEV)
    nblk = torch.from_numpy(db.nblk0).to(DEV)
    keeps = torch.from_numpy(np.ascontiguousarray(db.keeps)).to(DEV)
    table, _, _ = ks.ks_compact_block_table_rounds(table, nblk, keeps)
    lens = torch.from_numpy((db.live_len + 1).astype(np.int32)).to(DEV)
    assert ks.ks_paged_decode_workspace(B, Hq, D, MB) <= ks.ks_paged_decode_noalloc_max_scratch()

    # call 1: the full 64-sequence batch
    ref, ref_lse = ks.ks_paged_decode(q, kp, vp, table, lens)
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    st, msg = _noalloc_raw(q, kp, vp, table, lens, out, lse)
    assert st == 0, msg
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)

    # call 2: fewer sequences over a narrower table (the scratch keeps call 1's
    # contents; the split partials this call reads are all its own)
    B2 = 9
    width = int(((db.live_len[:B2] + 1 + 15) // 16).max()) + 3
    t2 = table[:B2, :width].contiguous()
    l2 = lens[:B2].contiguous()
    q2 = q[:B2].contiguous()
    ref2, ref2_lse = ks.ks_paged_decode(q2, kp, vp, t2, l2)
    out2 = torch.full_like(ref2, float("nan"))
    lse2 = torch.full_like(ref2_lse, float("nan"))
    st, msg = _noalloc_raw(q2, kp, vp, t2, l2, out2, lse2)
    assert st == 0, msg
    torch.cuda.synchronize()
    assert torch.equal(out2, ref2) and torch.equal(lse2, ref2_lse)

    # the binding of the same entry point, with its outputs supplied
    out3, lse3 = ks.ks_paged_decode_noalloc(q2, kp, vp, t2, l2, out=torch.empty_like(ref2),
                                            lse=torch.empty_like(ref2_lse))
    torch.cuda.synchronize()
    assert torch.equal(out3, ref2) and torch.equal(lse3, ref2_lse)


def test_noalloc_decode_refuses_calls_beyond_its_scratch():
    Hq, Hkv, D = 32, 8, 128
    bf = torch.bfloat16
    MBw = 500_000                      # 2 x 32 x ceil(500000 / 48) split slots: > 96 MiB
    table = torch.full((2, MBw), -1, dtype=torch.int32, device=DEV)
    lens = torch.zeros(2, dtype=torch.int32, device=DEV)
    pool = torch.zeros(1, Hkv, 16, D, dtype=bf, device=DEV)
    q = torch.zeros(2, Hq, D, dtype=bf, device=DEV)
    out = torch.zeros_like(q)
    lse = torch.zeros(2, Hq, dtype=torch.float32, device=DEV)
    st, msg = _noalloc_raw(q, pool, pool, table, lens, out, lse)
    assert st == 4 and "scratch" in msg, (st, msg)      # KS_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == 0)  # nothing was written
