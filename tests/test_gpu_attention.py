"""GPU parity of the eviction-masked attention (forward and backward) against
the fp64 oracle, on full small configurations and edge cases."""
import math

import numpy as np
import pytest
import torch

import kv_cache_compaction_amd as ks
import oracle as O
from parity_util import announce, errors, f64, gate, passes
from workloads import KS_NEVER, TINY_F32, TRAIN_4K, config_trace_batch, normal_tensor, stacked_e

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


def _e_gpu(e):
    return torch.from_numpy(np.ascontiguousarray(e.astype(np.int32))).to(DEV)


def _random_e(rng, B, N, p_never=0.3):
    e = np.empty((B, N), dtype=np.int64)
    for b in range(B):
        j = np.arange(N)
        e[b] = j + 1 + (rng.random(N) * (N - j)).astype(np.int64)
        e[b][rng.random(N) < p_never] = KS_NEVER
    return e


def _inputs(B, N, Hq, Hkv, D, seed, dtype, scale=0.5):
    q = normal_tensor((B, N, Hq, D), seed, scale, dtype)
    k = normal_tensor((B, N, Hkv, D), seed + 1, scale, dtype)
    v = normal_tensor((B, N, Hkv, D), seed + 2, scale, dtype)
    do = normal_tensor((B, N, Hq, D), seed + 3, scale, dtype)
    return q, k, v, do


# ---------------------------------------------------------------------------
def test_tiny512_f32_rope_then_forward():
    cfg = TINY_F32
    (tr,), seeds = config_trace_batch(cfg)
    B, N, D = 1, cfg.N, cfg.D
    q = normal_tensor((B, N, 1, D), seeds["q"])
    k = normal_tensor((B, N, 1, D), seeds["k"])
    v = normal_tensor((B, N, 1, D), seeds["v"])
    pos = np.arange(N, dtype=np.int32)[None]
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    ks.ks_rope_logical(qg, kg, torch.from_numpy(pos).to(DEV))
    e = stacked_e([tr])
    o, lse = ks.ks_evict_attn_fwd(qg, kg, vg, _e_gpu(e))
    torch.cuda.synchronize()
    qr, kr = O.rope(f64(q), pos), O.rope(f64(k), pos)
    ro, rl = O.attn_fwd(qr, kr, f64(v), e)
    gate(o, ro, "f32", "O")
    gate(lse, rl, "f32", "LSE")


@pytest.mark.parametrize("N,G,D,seed", [(1, 1, 64, 1), (63, 1, 64, 2), (200, 2, 64, 3),
                                        (333, 4, 64, 4), (150, 3, 128, 5), (97, 1, 128, 6)])
def test_f32_forward_random_masks(N, G, D, seed):
    B, Hkv = 2, 2
    rng = np.random.default_rng(seed)
    e = _random_e(rng, B, N)
    q, k, v, _ = _inputs(B, N, Hkv * G, Hkv, D, 100 + seed, torch.float32, 1.0)
    o, lse = ks.ks_evict_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), _e_gpu(e))
    torch.cuda.synchronize()
    ro, rl = O.attn_fwd(f64(q), f64(k), f64(v), e)
    gate(o, ro, "f32", "O")
    gate(lse, rl, "f32", "LSE")


# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def train4k():
    cfg = TRAIN_4K
    traces, seeds = config_trace_batch(cfg)
    e = stacked_e(traces)
    B, N = cfg.batch, cfg.N
    q, k, v, do = _inputs(B, N, cfg.Hq, cfg.Hkv, cfg.D, seeds["q"], torch.bfloat16)
    qg, kg, vg, dog = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    eg = _e_gpu(e)
    o, lse = ks.ks_evict_attn_fwd(qg, kg, vg, eg)
    dq, dk, dv = ks.ks_evict_attn_bwd(qg, kg, vg, eg, o, lse, dog)
    torch.cuda.synchronize()
    ro, rl = O.attn_fwd(f64(q), f64(k), f64(v), e)
    rdq, rdk, rdv = O.attn_bwd(f64(q), f64(k), f64(v), e, f64(do))
    return dict(e=e, q=q, k=k, v=v, do=do, got=(o, lse, dq, dk, dv),
                ref=(ro, rl, rdq, rdk, rdv))


def test_train4k_forward(train4k):
    o, lse = train4k["got"][:2]
    ro, rl = train4k["ref"][:2]
    gate(o, ro, "bf16", "O")
    gate(lse, rl, "bf16", "LSE")


def test_train4k_backward(train4k):
    for name, got, ref in zip(("dQ", "dK", "dV"), train4k["got"][2:], train4k["ref"][2:]):
        gate(got, ref, "bf16grad", name)


def test_train4k_negative_controls(train4k):
    """The gate must reject outputs compared against a wrong mask."""
    o = train4k["got"][0]
    q, k, v, e = f64(train4k["q"]), f64(train4k["k"]), f64(train4k["v"]), train4k["e"]
    N = e.shape[1]
    never = np.full_like(e, KS_NEVER)
    wrong_causal, _ = O.attn_fwd(q, k, v, never)
    ok, er = passes(o, wrong_causal, "bf16")
    assert not ok, f"mask dropped not detected: {er}"
    ep1 = np.where(e < N, e + 1, e)    # off by one: i <= e_j
    wrong_off, _ = O.attn_fwd(q, k, v, ep1)
    ok, er = passes(o, wrong_off, "bf16")
    assert not ok, f"off-by-one e not detected: {er}"


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,Hq,Hkv,D,seed", [
    (1, 4, 1, 128, 1), (65, 4, 4, 128, 2), (300, 8, 2, 128, 3), (517, 8, 1, 128, 4),
    (700, 2, 1, 128, 5), (450, 4, 2, 64, 6), (129, 16, 2, 128, 7),
    # group sizes 3 and 6: one and two query heads per wave
    (150, 6, 2, 128, 8), (140, 12, 2, 128, 9), (90, 3, 1, 64, 10), (77, 12, 2, 64, 11),
    # D = 64 with four query heads per wave
    (180, 8, 2, 64, 12), (65, 8, 1, 64, 13)])
def test_bf16_forward_random_masks(N, Hq, Hkv, D, seed):
    B = 2
    rng = np.random.default_rng(seed)
    e = _random_e(rng, B, N)
    q, k, v, _ = _inputs(B, N, Hq, Hkv, D, 200 + seed, torch.bfloat16)
    o, lse = ks.ks_evict_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), _e_gpu(e))
    torch.cuda.synchronize()
    ro, rl = O.attn_fwd(f64(q), f64(k), f64(v), e)
    gate(o, ro, "bf16", "O")
    gate(lse, rl, "bf16", "LSE")


@pytest.mark.parametrize("N,Hq,Hkv,seed", [
    (1, 4, 1, 1), (70, 4, 4, 2), (300, 8, 2, 3), (517, 8, 1, 4), (260, 2, 1, 5),
    (129, 16, 2, 6), (150, 6, 2, 7), (140, 12, 2, 8)])
def test_bf16_backward_random_masks(N, Hq, Hkv, seed):
    B, D = 2, 128
    rng = np.random.default_rng(seed)
    e = _random_e(rng, B, N)
    q, k, v, do = _inputs(B, N, Hq, Hkv, D, 300 + seed, torch.bfloat16)
    qg, kg, vg, dog, eg = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), _e_gpu(e)
    o, lse = ks.ks_evict_attn_fwd(qg, kg, vg, eg)
    dq, dk, dv = ks.ks_evict_attn_bwd(qg, kg, vg, eg, o, lse, dog)
    torch.cuda.synchronize()
    rdq, rdk, rdv = O.attn_bwd(f64(q), f64(k), f64(v), e, f64(do))
    gate(dq, rdq, "bf16grad", "dQ")
    gate(dk, rdk, "bf16grad", "dK")
    gate(dv, rdv, "bf16grad", "dV")


def test_bf16_diagonal_only_and_causal():
    B, N, Hq, Hkv, D = 1, 257, 4, 2, 128
    q, k, v, do = _inputs(B, N, Hq, Hkv, D, 400, torch.bfloat16)
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    diag = (np.arange(N) + 1)[None]
    o, lse = ks.ks_evict_attn_fwd(qg, kg, vg, _e_gpu(diag))
    torch.cuda.synchronize()
    # O = V exactly up to the bf16 round trip of P = 1
    for h in range(Hq):
        np.testing.assert_allclose(f64(o)[0, :, h], f64(v)[0, :, h // 2], atol=1e-6)
    never = np.full((B, N), KS_NEVER)
    o2, _ = ks.ks_evict_attn_fwd(qg, kg, vg, _e_gpu(never))
    torch.cuda.synchronize()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.double().permute(0, 2, 1, 3),
        k.double().repeat_interleave(2, 2).permute(0, 2, 1, 3).contiguous(),
        v.double().repeat_interleave(2, 2).permute(0, 2, 1, 3).contiguous(),
        is_causal=True).permute(0, 2, 1, 3)
    gate(o2, ref, "bf16", "causal O")


def test_bf16_end_to_end_rope_train4k():
    """RoPE at logical positions then the masked forward, against the oracle
    doing both in fp64 from the same raw projections."""
    cfg = TRAIN_4K
    traces, seeds = config_trace_batch(cfg)
    e = stacked_e(traces)
    B, N = cfg.batch, cfg.N
    q, k, v, _ = _inputs(B, N, cfg.Hq, cfg.Hkv, cfg.D, seeds["q"] + 7, torch.bfloat16)
    pos = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    ks.ks_rope_logical(qg, kg, torch.from_numpy(pos).to(DEV))
    o, lse = ks.ks_evict_attn_fwd(qg, kg, vg, _e_gpu(e))
    torch.cuda.synchronize()
    ro, rl = O.attn_fwd(O.rope(f64(q), pos), O.rope(f64(k), pos), f64(v), e)
    gate(o, ro, "bf16", "O")
    gate(lse, rl, "bf16", "LSE")


def test_bf16_raw_projection_gradients_train4k():
    """Gradients with respect to the raw q, k of the 4k workload: RoPE, masked
    forward and backward on the GPU, then the inverse rotation of dQ, dK
    (ks_rope_logical with inverse), against the oracle's gradients through
    its own RoPE."""
    cfg = TRAIN_4K
    traces, seeds = config_trace_batch(cfg)
    e = stacked_e(traces)
    B, N = cfg.batch, cfg.N
    q, k, v, do = _inputs(B, N, cfg.Hq, cfg.Hkv, cfg.D, seeds["q"] + 11, torch.bfloat16)
    pos = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    pg = torch.from_numpy(pos).to(DEV)
    qg, kg, vg, dog = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    ks.ks_rope_logical(qg, kg, pg)
    o, lse = ks.ks_evict_attn_fwd(qg, kg, vg, _e_gpu(e))
    dq, dk, dv = ks.ks_evict_attn_bwd(qg, kg, vg, _e_gpu(e), o, lse, dog)
    ks.ks_rope_logical(dq, dk, pg, inverse=True)
    torch.cuda.synchronize()
    qr, kr = O.rope(f64(q), pos), O.rope(f64(k), pos)
    rdq, rdk, rdv = O.attn_bwd(qr, kr, f64(v), e, f64(do))
    gate(dq, O.rope(rdq, pos, inverse=True), "bf16grad", "dQ raw")
    gate(dk, O.rope(rdk, pos, inverse=True), "bf16grad", "dK raw")
    gate(dv, rdv, "bf16grad", "dV")



def _broken_e(rng, B, N):
    """Records that break e_j > j: a fifth of the tokens get e_j <= j (seen by
    no query), and the first three tokens too, so rows 0..2 see no key."""
    e = _random_e(rng, B, N)
    j = np.arange(N)[None].repeat(B, 0)
    bad = rng.random((B, N)) < 0.2
    e[bad] = (j - rng.integers(0, 5, (B, N)))[bad]
    e[:, :3] = [0, 1, 2]
    return e


def _empty_rows(e, N):
    """rows that see no key under j <= i < e_j"""
    out = []
    for b in range(e.shape[0]):
        vis = np.zeros(N, bool)
        for jj in range(N):
            vis[jj:max(jj, min(N, int(e[b, jj])))] = True
        out.append(~vis)
    return np.stack(out)


@pytest.mark.parametrize("N,Hq,Hkv,D,seed", [(300, 8, 2, 128, 1), (129, 4, 4, 128, 2),
                                            (200, 4, 2, 64, 3)])
def test_bf16_broken_records(N, Hq, Hkv, D, seed):
    """Outside the preconditions the kernels still follow the oracle's
    reading: invisible tokens contribute nothing, rows that see no key give
    O = 0 and LSE = -inf, and the gradients stay finite."""
    B = 2
    e = _broken_e(np.random.default_rng(700 + seed), B, N)
    empty = _empty_rows(e, N)
    assert empty[:, :3].all() and not empty.all()
    q, k, v, do = _inputs(B, N, Hq, Hkv, D, 710 + seed, torch.bfloat16)
    qg, kg, vg, dog, eg = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), _e_gpu(e)
    o, lse = ks.ks_evict_attn_fwd(qg, kg, vg, eg)
    torch.cuda.synchronize()
    ro, rl = O.attn_fwd(f64(q), f64(k), f64(v), e)
    gate(o, ro, "bf16", "O")
    lg = lse.cpu().numpy()
    for b in range(B):
        assert np.all(np.isneginf(lg[b][:, empty[b]]))
        assert torch.all(o[b][torch.from_numpy(empty[b]).to(DEV)] == 0)
        gate(lse[b][:, torch.from_numpy(~empty[b]).to(DEV)], rl[b][:, ~empty[b]], "bf16", "LSE")
    ks.ks_check_eviction_record(eg)       # counts only; exercised beside the kernels
    if D != 128:
        return
    dq, dk, dv = ks.ks_evict_attn_bwd(qg, kg, vg, eg, o, lse, dog)
    torch.cuda.synchronize()
    rdq, rdk, rdv = O.attn_bwd(f64(q), f64(k), f64(v), e, f64(do))
    gate(dq, rdq, "bf16grad", "dQ")
    gate(dk, rdk, "bf16grad", "dK")
    gate(dv, rdv, "bf16grad", "dV")


def test_f32_broken_records():
    B, N, Hq, Hkv, D = 2, 150, 2, 1, 64
    e = _broken_e(np.random.default_rng(720), B, N)
    empty = _empty_rows(e, N)
    q, k, v, _ = _inputs(B, N, Hq, Hkv, D, 721, torch.float32, scale=1.0)
    o, lse = ks.ks_evict_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), _e_gpu(e))
    torch.cuda.synchronize()
    ro, rl = O.attn_fwd(f64(q), f64(k), f64(v), e)
    gate(o, ro, "f32", "O")
    lg = lse.cpu().numpy()
    for b in range(B):
        assert np.all(np.isneginf(lg[b][:, empty[b]]))
        gate(lg[b][:, ~empty[b]], rl[b][:, ~empty[b]], "f32", "LSE")


def test_training_pass_replays_from_a_graph():
    """RoPE, masked forward and backward are capture-safe (the library records
    no memsets and allocates nothing): a captured graph, which first restores
    the unrotated q and k, replays to the eager results every time, with
    eager work on the same tensors in between."""
    rng = np.random.default_rng(61)
    B, N, Hq, Hkv, D = 2, 700, 8, 2, 128
    e = _random_e(rng, B, N)
    q0, k0, v, do = (t.to(DEV) for t in _inputs(B, N, Hq, Hkv, D, 610, torch.bfloat16))
    eg = _e_gpu(e)
    pos = torch.arange(N, dtype=torch.int32, device=DEV)[None].repeat(B, 1).contiguous()
    q, k = torch.empty_like(q0), torch.empty_like(k0)
    o = torch.empty_like(q0)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q0), torch.empty_like(k0), torch.empty_like(v)
    wsf = torch.empty(ks.ks_evict_attn_fwd_workspace(B, N, Hq, Hkv, D, ks.KS_BF16),
                      dtype=torch.uint8, device=DEV)
    wsb = torch.empty(ks.ks_evict_attn_bwd_workspace(B, N, Hq, Hkv, D, ks.KS_BF16),
                      dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()

    def step():
        q.copy_(q0)
        k.copy_(k0)
        ks.ks_rope_logical(q, k, pos, stream=s)
        ks.ks_evict_attn_fwd(q, k, v, eg, out=o, lse=lse, ws=wsf, stream=s)
        ks.ks_evict_attn_bwd(q, k, v, eg, o, lse, do, dq=dq, dk=dk, dv=dv, ws=wsb, stream=s)
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        ref = [t.clone() for t in (q, o, lse, dq, dk, dv)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
        torch.cuda.synchronize()
        for _ in range(4):
            for t in (q, k, o, dq, dk, dv):
                t.fill_(7)
            lse.zero_()
            wsb.fill_(255)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for got, want in zip((q, o, lse, dq, dk, dv), ref):
                assert torch.equal(got, want)
