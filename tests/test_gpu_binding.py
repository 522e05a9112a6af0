"""The Python binding refuses caller-supplied buffers that the library would
write past or read wrongly (wrong shape, dtype, strides) before anything is
launched: the C ABI takes plain pointers and cannot check sizes itself."""
import pytest
import torch

import kv_cache_compaction_amd as ks
from parity_util import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"
bf = torch.bfloat16


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


def _qkv(B=1, N=64, Hq=4, Hkv=2, D=128):
    q = torch.zeros(B, N, Hq, D, dtype=bf, device=DEV)
    k = torch.zeros(B, N, Hkv, D, dtype=bf, device=DEV)
    v = torch.zeros(B, N, Hkv, D, dtype=bf, device=DEV)
    e = torch.full((B, N), ks.KS_NEVER, dtype=torch.int32, device=DEV)
    return q, k, v, e


def test_attention_outputs_are_checked():
    q, k, v, e = _qkv()
    with pytest.raises(ValueError, match="out"):
        ks.ks_evict_attn_fwd(q, k, v, e, out=torch.empty(1, 32, 4, 128, dtype=bf, device=DEV))
    with pytest.raises(ValueError, match="lse"):
        ks.ks_evict_attn_fwd(q, k, v, e, lse=torch.empty(1, 4, 63, device=DEV))
    o, lse = ks.ks_evict_attn_fwd(q, k, v, e)
    with pytest.raises(ValueError, match="dq"):
        ks.ks_evict_attn_bwd(q, k, v, e, o, lse, o, dq=torch.empty_like(q, dtype=torch.float32))
    with pytest.raises(ValueError, match="dk"):
        ks.ks_evict_attn_bwd(q, k, v, e, o, lse, o, dk=torch.empty_like(q))
    with pytest.raises(ValueError, match="contiguous"):
        ks.ks_evict_attn_bwd(q, k, v, e, o, lse, o, dv=torch.empty(1, 64, 128, 2, dtype=bf,
                                                                   device=DEV).transpose(2, 3))
    with pytest.raises(ValueError, match="k/v"):
        ks.ks_evict_attn_bwd(q, k[:, :32].contiguous(), v, e, o, lse, o)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)[::2]
    with pytest.raises(ValueError, match="ws"):
        ks.ks_evict_attn_fwd(q, k, v, e, ws=ws)
    torch.cuda.synchronize()


def test_decode_pools_and_outputs_are_checked():
    B, Hq, Hkv, D, NB = 2, 8, 2, 128, 4
    q = torch.zeros(B, Hq, D, dtype=bf, device=DEV)
    table = torch.zeros(B, 2, dtype=torch.int32, device=DEV)
    lens = torch.ones(B, dtype=torch.int32, device=DEV)
    bad_pool = torch.zeros(NB, Hkv, 16, 64, dtype=bf, device=DEV)     # head dim 64 != 128
    with pytest.raises(ValueError, match="D"):
        ks.ks_paged_decode(q, bad_pool, bad_pool, table, lens)
    pool = torch.zeros(NB, Hkv, 16, D, dtype=bf, device=DEV)
    with pytest.raises(ValueError, match="out"):
        ks.ks_paged_decode(q, pool, pool, table, lens, out=torch.empty(B, Hq - 1, D, dtype=bf,
                                                                       device=DEV))
    with pytest.raises(ValueError, match="lse"):
        ks.ks_paged_decode(q, pool, pool, table, lens, lse=torch.empty(B, device=DEV))
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="head dim"):
        ks.ks_paged_decode_rope(q, pos, bad_pool, bad_pool, table, lens)
    slots = torch.zeros(16, Hkv, 64, dtype=bf, device=DEV)
    with pytest.raises(ValueError, match="D"):
        ks.ks_paged_decode_bs1(q, slots, slots, table, lens)
    torch.cuda.synchronize()


def test_compaction_outputs_are_checked():
    B, MB = 3, 10
    table = torch.arange(B * MB, dtype=torch.int32, device=DEV).view(B, MB)
    nblk = torch.full((B,), MB, dtype=torch.int32, device=DEV)
    keep = torch.ones(B, MB, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="table_out"):
        ks.ks_compact_block_table(table, nblk, keep, table_out=torch.empty(B, MB - 1,
                                                                           dtype=torch.int32,
                                                                           device=DEV))
    with pytest.raises(ValueError, match="nblk_out"):
        ks.ks_compact_block_table(table, nblk, keep, nblk_out=torch.empty(B, dtype=torch.int64,
                                                                          device=DEV))
    with pytest.raises(ValueError, match="pos_out"):
        ks.ks_compact_block_table(table, nblk, keep, pos_out=torch.empty_like(table))
    with pytest.raises(ValueError, match="pos_in"):
        ks.ks_compact_block_table(table, nblk, keep, pos_in=table[:, :5].contiguous())
    with pytest.raises(ValueError, match="pos_out"):
        ks.ks_compact_block_table_rounds(table, nblk, keep[None], pos_in=table,
                                         pos_out=torch.empty(B, MB + 1, dtype=torch.int32,
                                                             device=DEV))
    with pytest.raises(ValueError, match="bad"):
        ks.ks_check_block_table(table, nblk, 100, bad=torch.empty(B + 1, dtype=torch.int32,
                                                                  device=DEV))
    # the well-formed call still works
    t2, n2, _ = ks.ks_compact_block_table(table, nblk, keep)
    torch.cuda.synchronize()
    assert torch.equal(t2, table) and torch.equal(n2, nblk)


def test_empty_inputs_are_no_ops():
    """B = 0, N = 0 and empty table rows: nothing is read, outputs are empty or
    the documented zero rows (lse = -inf)."""
    for B, N in ((0, 64), (2, 0)):
        q, k, v, e = _qkv(B=B, N=N)
        pos = torch.zeros(B, N, dtype=torch.int32, device=DEV)
        ks.ks_rope_logical(q, k, pos)
        o, lse = ks.ks_evict_attn_fwd(q, k, v, e)
        dq, dk, dv = ks.ks_evict_attn_bwd(q, k, v, e, o, lse, o)
        assert o.shape == q.shape and lse.shape == (B, 4, N) and dk.shape == k.shape
    # compaction of zero rows and of zero-length rows
    t0 = torch.empty(0, 7, dtype=torch.int32, device=DEV)
    n0 = torch.empty(0, dtype=torch.int32, device=DEV)
    t1, n1, _ = ks.ks_compact_block_table(t0, n0, torch.empty(0, 7, dtype=torch.uint8,
                                                               device=DEV))
    assert t1.shape == (0, 7) and n1.numel() == 0
    tz = torch.empty(3, 0, dtype=torch.int32, device=DEV)
    nz = torch.tensor([0, 2, 5], dtype=torch.int32, device=DEV)
    _, nz_out, _ = ks.ks_compact_block_table(tz, nz, torch.empty(3, 0, dtype=torch.uint8,
                                                                  device=DEV))
    _, nz_out2, _ = ks.ks_compact_block_table_rounds(tz, nz, torch.empty(2, 3, 0,
                                                                          dtype=torch.uint8,
                                                                          device=DEV))
    # decode: no sequences, and sequences whose table has no entries
    Hq, Hkv, D = 8, 2, 128
    pool = torch.zeros(4, Hkv, 16, D, dtype=bf, device=DEV)
    q0 = torch.zeros(0, Hq, D, dtype=bf, device=DEV)
    out0, lse0 = ks.ks_paged_decode(q0, pool, pool, torch.empty(0, 3, dtype=torch.int32,
                                                                device=DEV),
                                    torch.empty(0, dtype=torch.int32, device=DEV))
    assert out0.shape == (0, Hq, D)
    q = torch.ones(3, Hq, D, dtype=bf, device=DEV)
    lens = torch.tensor([0, 5, 40], dtype=torch.int32, device=DEV)
    empty_pool = torch.empty(0, Hkv, 16, D, dtype=bf, device=DEV)
    out, lse = ks.ks_paged_decode(q, empty_pool, empty_pool, tz, lens)
    pos1 = torch.full((3,), 100, dtype=torch.int32, device=DEV)
    out_r, lse_r = ks.ks_paged_decode_rope(q, pos1, empty_pool, empty_pool, tz, lens)
    # the workspace the binding passes is exactly the C query's size for an
    # empty table (one split per sequence and head)
    empty_tok = torch.empty(0, Hkv, D, dtype=bf, device=DEV)
    out_1, lse_1 = ks.ks_paged_decode_bs1(q, empty_tok, empty_tok, tz, lens)
    torch.cuda.synchronize()
    assert torch.all(nz_out == 0) and torch.all(nz_out2 == 0)
    for o_, l_ in ((out, lse), (out_r, lse_r), (out_1, lse_1)):
        assert torch.all(o_ == 0)
        assert torch.all(torch.isinf(l_)) and torch.all(l_ < 0)
    # entries present but no pool blocks: refused before launching
    with pytest.raises(ks.KSError, match="no blocks"):
        ks.ks_paged_decode(q, empty_pool, empty_pool,
                           torch.zeros(3, 2, dtype=torch.int32, device=DEV), lens)
