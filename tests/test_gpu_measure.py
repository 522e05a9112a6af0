"""The measurement aids of include/ks_measure.h do the work the bench credits
them with: the MFMA rate loop performs every MFMA it counts, and the dQ
atomics probe adds once per (256-key workgroup, covered row, head)."""
import numpy as np
import pytest
import torch

import kv_cache_compaction_amd as ks
from parity_util import announce
from workloads import build_trace

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


def test_mfma_rate_loop_runs_every_counted_mfma():
    wg, iters = 16, 5
    seed = torch.full((1024,), 0.01, dtype=torch.bfloat16, device=DEV)
    sink = torch.zeros(wg * 512, dtype=torch.float32, device=DEV)
    ks.ks_measure_mfma_bf16(seed, sink, wg, iters)
    torch.cuda.synchronize()
    a = float(seed[0].float())
    # per lane: 4 chains x 16 accumulators, each the sum of 8 * iters MFMAs of
    # 16 products a * a; the flop count credits 2*32*32*16 flop per MFMA
    want = 4 * 16 * 8 * iters * 16 * a * a
    got = sink.cpu().numpy()
    assert np.allclose(got, want, rtol=1e-3), (got[:4], want)
    assert ks.ks_measure_mfma_flops(wg, iters) == 2 * 32 * 32 * 16 * 32 * iters * 8 * wg


def test_dq_atomics_probe_adds_once_per_covering_workgroup():
    N, Hq, Hkv = 1000, 4, 2
    tr = build_trace(np.random.default_rng(11), N, 64, 320, "recent", turn_len=(64, 128))
    e = tr.e.astype(np.int64)
    nkt = (N + 255) // 256
    cend = np.zeros((1, nkt), np.int32)
    for t in range(nkt):
        cend[0, t] = (min(N, int(e[256 * t:256 * (t + 1)].max())) + 31) // 32
    acc = torch.zeros((1, N, Hq, 128), dtype=torch.float32, device=DEV)
    ks.ks_measure_dq_atomics(acc, torch.from_numpy(cend).to(DEV), Hkv)
    torch.cuda.synchronize()
    want = np.zeros(N)
    for t in range(nkt):
        want[256 * t:min(N, 32 * int(cend[0, t]))] += 1      # rows of chunks [8t, cend)
    got = acc.cpu().numpy()
    assert np.array_equal(got, np.broadcast_to(want[None, :, None, None], got.shape))
