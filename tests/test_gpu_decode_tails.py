"""GPU parity of paged decode on split tails: sequences whose last split has
an odd number of 16-token groups and ends in a full group (the final group
is processed after the paired main loop, with no masking), beside even and
partial tails, for every heads-per-wave variant (1, 2 and 4 heads per wave),
both block sizes and both split lengths (16 groups for these small grids;
48 when the table is widened so that the grid counts as large).  Checked
against the fp64 oracle."""
import numpy as np
import pytest
import torch

import kv_cache_compaction_amd as ks
import oracle as O
from parity_util import announce, f64, gate
from workloads import normal_tensor

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 128
# 16-token groups per sequence: odd tails of a split (1, 3, 47 mod 48 and
# 1, 3, 15 mod 16), even tails, and exactly full splits of either length
GROUPS = [1, 3, 47, 49, 51, 95, 97, 2, 50, 48]
# table width (groups) at which 10 sequences of up to 4 query heads make a
# grid of at least 4096 waves of 48-group splits: the long split length
WIDE = 48 * 410


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


def _gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _lengths(partial):
    g = np.array(GROUPS, np.int64)
    # full final group, or 5 tokens short of it
    return (16 * g - (5 if partial else 0)).astype(np.int32)


@pytest.mark.parametrize("G", [1, 2, 3, 4])          # 1, 2, 1, 4 heads per wave
@pytest.mark.parametrize("partial", [False, True])
@pytest.mark.parametrize("wide", [False, True])
def test_decode_split_tails(G, partial, wide):
    Hkv = 2
    Hq = G * Hkv
    lens = _lengths(partial)
    B = len(lens)
    nblk = (lens + 15) // 16
    MB = WIDE if wide else int(nblk.max())
    NB = int(nblk.sum()) + 7
    rng = np.random.default_rng(900 + 10 * G + partial)
    perm = rng.permutation(NB).astype(np.int32)
    table = np.full((B, MB), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    seed = 9100 + 10 * G + partial
    kp = normal_tensor((NB, Hkv, 16, D), seed, 0.5, torch.bfloat16, DEV)
    vp = normal_tensor((NB, Hkv, 16, D), seed + 1, 0.5, torch.bfloat16, DEV)
    q = normal_tensor((B, Hq, D), seed + 2, 0.5, torch.bfloat16, DEV)
    out, lse = ks.ks_paged_decode(q, kp, vp, _gpu(table), _gpu(lens))
    torch.cuda.synchronize()
    ro, rl = O.paged_decode(f64(q), f64(kp), f64(vp), table, lens)
    gate(out, ro, "bf16", f"decode tails G{G} partial={partial} wide={wide}")
    gate(lse, rl, "bf16", f"decode tails lse G{G} partial={partial} wide={wide}")


@pytest.mark.parametrize("G", [1, 2, 3, 4])
@pytest.mark.parametrize("wide", [False, True])
def test_decode_bs1_split_tails(G, wide):
    Hkv = 2
    Hq = G * Hkv
    lens = _lengths(False)
    B = len(lens)
    NT = int(lens.sum()) + 33
    rng = np.random.default_rng(950 + G)
    perm = rng.permutation(NT).astype(np.int32)
    table = np.full((B, 16 * WIDE if wide else int(lens.max())), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :lens[b]] = perm[off:off + lens[b]]
        off += lens[b]
    seed = 9500 + 10 * G
    kp = normal_tensor((NT, Hkv, D), seed, 0.5, torch.bfloat16, DEV)
    vp = normal_tensor((NT, Hkv, D), seed + 1, 0.5, torch.bfloat16, DEV)
    q = normal_tensor((B, Hq, D), seed + 2, 0.5, torch.bfloat16, DEV)
    out, lse = ks.ks_paged_decode_bs1(q, kp, vp, _gpu(table), _gpu(lens))
    torch.cuda.synchronize()
    ro, rl = O.paged_decode(f64(q), f64(kp)[:, :, None], f64(vp)[:, :, None], table, lens)
    gate(out, ro, "bf16", f"decode bs1 tails G{G} wide={wide}")
    gate(lse, rl, "bf16", f"decode bs1 tails lse G{G} wide={wide}")
