"""GPU parity of the RoPE-fused training entry points: the forward against
the separate RoPE pass plus the plain forward (bit for bit), and the
backward's gradients of the unrotated projections against the oracle (the
RoPE backward is the inverse rotation: explainer, RoPE paragraph, for the
logical positions; the softmax backward is the calculus of the forward)."""
import numpy as np
import pytest
import torch

import kv_cache_compaction_amd as ks
import oracle as O
from parity_util import announce, f64, gate
from workloads import TRAIN_4K, config_trace_batch, normal_tensor, stacked_e

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


def _random_e(rng, B, N):
    e = np.empty((B, N), dtype=np.int64)
    for b in range(B):
        j = np.arange(N)
        e[b] = j + 1 + (rng.random(N) * (N - j)).astype(np.int64)
        e[b][rng.random(N) < 0.3] = ks.KS_NEVER
    return e


def _positions(rng, B, N):
    """Logical positions: increasing, with gaps (retained tokens keep their
    original positions after compaction), offset per trace."""
    steps = 1 + (rng.random((B, N)) < 0.1) * rng.integers(1, 400, (B, N))
    pos = np.cumsum(steps, axis=1) - 1 + rng.integers(0, 5000, (B, 1))
    return pos.astype(np.int32)


def _case(B, N, Hq, Hkv, seed, e=None):
    D = 128
    rng = np.random.default_rng(seed)
    if e is None:
        e = _random_e(rng, B, N)
    pos = _positions(rng, B, N)
    bf = torch.bfloat16
    q = normal_tensor((B, N, Hq, D), 900 + seed, 0.5, bf)
    k = normal_tensor((B, N, Hkv, D), 901 + seed, 0.5, bf)
    v = normal_tensor((B, N, Hkv, D), 902 + seed, 0.5, bf)
    do = normal_tensor((B, N, Hq, D), 903 + seed, 0.5, bf)
    return e, pos, q, k, v, do


def _gpu(*ts):
    return [t.to(DEV) for t in ts]


CASES = [  # (B, N, Hq, Hkv, seed): ragged tails, group sizes 1, 2, 3, 4, 8
    (1, 1, 4, 1, 1), (2, 70, 4, 4, 2), (2, 300, 8, 2, 3), (1, 517, 8, 1, 4),
    (1, 150, 6, 2, 5), (2, 129, 16, 2, 6), (1, 4000, 8, 2, 7)]


@pytest.mark.parametrize("B,N,Hq,Hkv,seed", CASES)
def test_fused_forward_matches_separate_pass(B, N, Hq, Hkv, seed):
    """q_rot, k_rot, O and LSE equal ks_rope_logical then ks_evict_attn_fwd,
    bit for bit, and q, k are left unrotated."""
    e, pos, q, k, v, _ = _case(B, N, Hq, Hkv, seed)
    qg, kg, vg, eg, pg = _gpu(q, k, v, torch.from_numpy(e.astype(np.int32)),
                              torch.from_numpy(pos))
    q0, k0 = qg.clone(), kg.clone()
    o, lse, q_rot, k_rot = ks.ks_evict_attn_fwd_rope(qg, kg, vg, eg, pg)
    qs, kss = qg.clone(), kg.clone()
    ks.ks_rope_logical(qs, kss, pg)
    ro, rl = ks.ks_evict_attn_fwd(qs, kss, vg, eg)
    torch.cuda.synchronize()
    assert torch.equal(qg, q0) and torch.equal(kg, k0), "inputs modified"
    assert torch.equal(q_rot, qs), "q_rot"
    assert torch.equal(k_rot, kss), "k_rot"
    assert torch.equal(o, ro), "O"
    assert torch.equal(lse, rl), "LSE"


@pytest.mark.parametrize("B,N,Hq,Hkv,seed", CASES)
def test_fused_backward_against_oracle(B, N, Hq, Hkv, seed):
    """dQ and dK of the unrotated projections against the oracle (the fp64
    gradients of the rotated operands rotated back by -theta), dV against
    the oracle and bit for bit against the plain backward; dQ and dK within
    the bound of one extra rounding of the separate path (plain backward,
    then the inverse RoPE pass)."""
    e, pos, q, k, v, do = _case(B, N, Hq, Hkv, seed)
    qg, kg, vg, dog, eg, pg = _gpu(q, k, v, do, torch.from_numpy(e.astype(np.int32)),
                                   torch.from_numpy(pos))
    o, lse, q_rot, k_rot = ks.ks_evict_attn_fwd_rope(qg, kg, vg, eg, pg)
    dq, dk, dv = ks.ks_evict_attn_bwd_rope(q_rot, k_rot, vg, eg, pg, o, lse, dog)
    sq, sk, sv = ks.ks_evict_attn_bwd(q_rot, k_rot, vg, eg, o, lse, dog)
    ks.ks_rope_logical(sq, sk, pg, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(dv, sv), "dV differs from the plain backward"
    # one extra bf16 rounding before an orthogonal rotation moves a pair
    # (x_k, x_{k+D/2}) by at most 2^-9 of its norm; with the two final
    # roundings the two results differ by less than 2^-7 (|x_k| + |x_{k+D/2}|)
    for name, a, b in (("dQ", dq, sq), ("dK", dk, sk)):
        a, b = a.float(), b.float()
        h = b.shape[-1] // 2
        pair = b[..., :h].abs() + b[..., h:].abs()
        lim = 2.0**-7 * torch.cat([pair, pair], -1) + 1e-30
        assert bool(((a - b).abs() <= lim).all()), f"{name}: fused vs separate"
    qr, kr = O.rope(f64(q), pos), O.rope(f64(k), pos)
    rdq, rdk, rdv = O.attn_bwd(qr, kr, f64(v), e, f64(do))
    gate(dq, O.rope(rdq, pos, inverse=True), "bf16grad", "dQ (unrotated)")
    gate(dk, O.rope(rdk, pos, inverse=True), "bf16grad", "dK (unrotated)")
    gate(dv, rdv, "bf16grad", "dV")


def test_fused_train4k_end_to_end():
    """The 4k training configuration through the fused entry points, from
    the raw projections at positions 0..N-1, against the oracle."""
    cfg = TRAIN_4K
    traces, seeds = config_trace_batch(cfg)
    e = stacked_e(traces)
    B, N = cfg.batch, cfg.N
    bf = torch.bfloat16
    q = normal_tensor((B, N, cfg.Hq, cfg.D), seeds["q"], cfg.value_scale, bf)
    k = normal_tensor((B, N, cfg.Hkv, cfg.D), seeds["k"], cfg.value_scale, bf)
    v = normal_tensor((B, N, cfg.Hkv, cfg.D), seeds["v"], cfg.value_scale, bf)
    do = normal_tensor((B, N, cfg.Hq, cfg.D), seeds["do"], cfg.value_scale, bf)
    pos = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    qg, kg, vg, dog, eg, pg = _gpu(q, k, v, do, torch.from_numpy(e), torch.from_numpy(pos))
    o, lse, q_rot, k_rot = ks.ks_evict_attn_fwd_rope(qg, kg, vg, eg, pg)
    dq, dk, dv = ks.ks_evict_attn_bwd_rope(q_rot, k_rot, vg, eg, pg, o, lse, dog)
    torch.cuda.synchronize()
    qr, kr = O.rope(f64(q), pos), O.rope(f64(k), pos)
    ro, rl = O.attn_fwd(qr, kr, f64(v), e)
    gate(o, ro, "bf16", "O")
    gate(lse, rl, "bf16", "LSE")
    rdq, rdk, rdv = O.attn_bwd(qr, kr, f64(v), e, f64(do))
    gate(dq, O.rope(rdq, pos, inverse=True), "bf16grad", "dQ (unrotated)")
    gate(dk, O.rope(rdk, pos, inverse=True), "bf16grad", "dK (unrotated)")
    gate(dv, rdv, "bf16grad", "dV")


def test_fused_rejections():
    """Unsupported dtypes and sizes, aliasing outputs and short workspaces
    are refused before any launch."""
    B, N, H, D = 1, 64, 2, 128
    q = torch.zeros((B, N, H, D), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, N, H, D), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    e = torch.full((B, N), ks.KS_NEVER, dtype=torch.int32, device=DEV)
    pos = torch.arange(N, dtype=torch.int32, device=DEV)[None].contiguous()
    with pytest.raises(ks.KSError):   # q_rot aliasing q
        ks.ks_evict_attn_fwd_rope(q, k, v, e, pos, q_rot=q)
    with pytest.raises(ks.KSError):   # k_rot aliasing k
        ks.ks_evict_attn_fwd_rope(q, k, v, e, pos, k_rot=k)
    with pytest.raises(ks.KSError):   # fp32 is not supported by the fused path
        ks.ks_evict_attn_fwd_rope(q.float(), k.float(), v.float(), e, pos)
    with pytest.raises(ks.KSError):   # base must exceed one
        ks.ks_evict_attn_fwd_rope(q, k, v, e, pos, base=1.0)
    # a workspace short of the RoPE table is refused by the library itself
    # (status KS_ERR_WORKSPACE = 4), before anything is written
    lib = ks.load_library()
    need = lib.ks_evict_attn_bwd_rope_workspace(B, N, H, H, D, ks.KS_BF16)
    assert need > lib.ks_evict_attn_bwd_workspace(B, N, H, H, D, ks.KS_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    lse = torch.zeros((B, H, N), dtype=torch.float32, device=DEV)
    dq, dk, dv = (torch.zeros_like(q) for _ in range(3))
    p = lambda t: t.data_ptr()
    st = lib.ks_evict_attn_bwd_rope(p(q), p(k), p(v), p(e), p(pos), p(q), p(lse), p(q), p(dq),
                                    p(dk), p(dv), B, N, H, H, D, ks.KS_BF16, 0.125, 10000.0,
                                    p(ws), need - 256, None)
    assert st == 4, st
    torch.cuda.synchronize()
    assert not dq.any() and not dk.any() and not dv.any()


def test_fused_training_pass_replays_from_a_graph():
    """The fused forward and backward are capture-safe (no memsets, no
    allocation): a captured pass replays to the eager results every time,
    with its outputs and workspaces overwritten in between."""
    B, N, Hq, Hkv = 2, 700, 8, 2
    e, pos, q, k, v, do = _case(B, N, Hq, Hkv, 61)
    qg, kg, vg, dog, eg, pg = _gpu(q, k, v, do, torch.from_numpy(e.astype(np.int32)),
                                   torch.from_numpy(pos))
    D = qg.shape[-1]
    q_rot, k_rot = torch.empty_like(qg), torch.empty_like(kg)
    o = torch.empty_like(qg)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    lib = ks.load_library()
    wsf = torch.empty(lib.ks_evict_attn_fwd_rope_workspace(B, N, Hq, Hkv, D, ks.KS_BF16),
                      dtype=torch.uint8, device=DEV)
    wsb = torch.empty(lib.ks_evict_attn_bwd_rope_workspace(B, N, Hq, Hkv, D, ks.KS_BF16),
                      dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()

    def step():
        ks.ks_evict_attn_fwd_rope(qg, kg, vg, eg, pg, q_rot=q_rot, k_rot=k_rot, out=o, lse=lse,
                                  ws=wsf, stream=s)
        ks.ks_evict_attn_bwd_rope(q_rot, k_rot, vg, eg, pg, o, lse, dog, dq=dq, dk=dk, dv=dv,
                                  ws=wsb, stream=s)
    outs = (q_rot, k_rot, o, lse, dq, dk, dv)
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        ref = [t.clone() for t in outs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
        torch.cuda.synchronize()
        for _ in range(4):
            for t in (q_rot, k_rot, o, dq, dk, dv):
                t.fill_(7)
            lse.zero_()
            wsf.fill_(255)
            wsb.fill_(255)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for got, want in zip(outs, ref):
                assert torch.equal(got, want)
