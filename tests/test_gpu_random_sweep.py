"""Seeded random sweep of shapes through the attention and decode entry
points against the oracle: batch, length (ragged against every tile size),
group size, head dim, eviction records and cache lengths drawn at random,
so that combinations the fixed cases do not list are exercised as well."""
import numpy as np
import pytest
import torch

import kv_cache_compaction_amd as ks
import oracle as O
from parity_util import announce, f64, gate
from workloads import KS_NEVER, normal_tensor

pytestmark = pytest.mark.gpu
DEV = "cuda"
bf = torch.bfloat16


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


def _record(rng, B, N):
    """e_j > j: never-evicted tokens, short and long lifetimes, and runs of
    tokens evicted together at one event (as compaction produces)."""
    e = np.empty((B, N), np.int64)
    j = np.arange(N)
    for b in range(B):
        kind = rng.integers(0, 3, N)
        short = j + 1 + rng.integers(0, 64, N)
        long_ = j + 1 + (rng.random(N) * (N - j)).astype(np.int64)
        e[b] = np.where(kind == 0, KS_NEVER, np.where(kind == 1, short, long_))
        for _ in range(int(rng.integers(0, 4))):
            a = int(rng.integers(0, N))
            z = min(N, a + int(rng.integers(1, 200)))
            e[b, a:z] = z + int(rng.integers(0, 100))
    return e


@pytest.mark.parametrize("seed", range(12))
def test_attention_random_shapes(seed):
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.integers(1, 4))
    N = int(rng.integers(1, 600))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8]))
    D = int(rng.choice([64, 128]))
    Hq = Hkv * G
    e = _record(rng, B, N)
    s0 = 9100 + 10 * seed
    q = normal_tensor((B, N, Hq, D), s0, 0.5, bf)
    k = normal_tensor((B, N, Hkv, D), s0 + 1, 0.5, bf)
    v = normal_tensor((B, N, Hkv, D), s0 + 2, 0.5, bf)
    do = normal_tensor((B, N, Hq, D), s0 + 3, 0.5, bf)
    eg = torch.from_numpy(e.astype(np.int32)).to(DEV)
    qg, kg, vg, dog = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = ks.ks_evict_attn_fwd(qg, kg, vg, eg)
    grads = ks.ks_evict_attn_bwd(qg, kg, vg, eg, o, lse, dog) if D == 128 else None
    torch.cuda.synchronize()
    tag = f"B={B} N={N} Hq={Hq} Hkv={Hkv} D={D}"
    ro, rl = O.attn_fwd(f64(q), f64(k), f64(v), e)
    gate(o, ro, "bf16", f"O {tag}")
    gate(lse, rl, "bf16", f"LSE {tag}")
    if grads is not None:
        rdq, rdk, rdv = O.attn_bwd(f64(q), f64(k), f64(v), e, f64(do))
        for name, got, ref in zip(("dQ", "dK", "dV"), grads, (rdq, rdk, rdv)):
            gate(got, ref, "bf16grad", f"{name} {tag}")


@pytest.mark.parametrize("seed", range(8))
def test_fused_rope_random_shapes(seed):
    """The training step's entry points (RoPE fused into the forward and the
    backward) on random shapes, records and logical positions with gaps,
    against the oracle's outputs and its gradients of the unrotated
    projections (the gradients of the rotated operands rotated back)."""
    rng = np.random.default_rng(9300 + seed)
    B = int(rng.integers(1, 4))
    N = int(rng.integers(1, 300)) if seed % 2 else int(rng.integers(300, 2500))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8]))
    Hq, D = Hkv * G, 128
    e = _record(rng, B, N)
    steps = 1 + (rng.random((B, N)) < 0.1) * rng.integers(1, 400, (B, N))
    pos = (np.cumsum(steps, axis=1) - 1 + rng.integers(0, 5000, (B, 1))).astype(np.int32)
    s0 = 9300 + 10 * seed
    q = normal_tensor((B, N, Hq, D), s0, 0.5, bf)
    k = normal_tensor((B, N, Hkv, D), s0 + 1, 0.5, bf)
    v = normal_tensor((B, N, Hkv, D), s0 + 2, 0.5, bf)
    do = normal_tensor((B, N, Hq, D), s0 + 3, 0.5, bf)
    eg = torch.from_numpy(e.astype(np.int32)).to(DEV)
    pg = torch.from_numpy(pos).to(DEV)
    qg, kg, vg, dog = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse, q_rot, k_rot = ks.ks_evict_attn_fwd_rope(qg, kg, vg, eg, pg)
    dq, dk, dv = ks.ks_evict_attn_bwd_rope(q_rot, k_rot, vg, eg, pg, o, lse, dog)
    torch.cuda.synchronize()
    tag = f"B={B} N={N} Hq={Hq} Hkv={Hkv}"
    qr, kr = O.rope(f64(q), pos), O.rope(f64(k), pos)
    ro, rl = O.attn_fwd(qr, kr, f64(v), e)
    gate(o, ro, "bf16", f"O {tag}")
    gate(lse, rl, "bf16", f"LSE {tag}")
    rdq, rdk, rdv = O.attn_bwd(qr, kr, f64(v), e, f64(do))
    gate(dq, O.rope(rdq, pos, inverse=True), "bf16grad", f"dQ (unrotated) {tag}")
    gate(dk, O.rope(rdk, pos, inverse=True), "bf16grad", f"dK (unrotated) {tag}")
    gate(dv, rdv, "bf16grad", f"dV {tag}")


@pytest.mark.parametrize("seed", range(8))
def test_decode_random_shapes(seed):
    rng = np.random.default_rng(9500 + seed)
    block = int(rng.choice([16, 1]))
    B = int(rng.integers(1, 10))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8]))
    Hq, D = Hkv * G, 128
    lens = rng.integers(0, 2000, B).astype(np.int32)
    lens[rng.random(B) < 0.2] = 0
    ents = [(int(x) + block - 1) // block for x in lens]
    ME = max(max(ents), 1)
    NP = sum(ents) + 5
    perm = rng.permutation(NP).astype(np.int32)
    table = np.full((B, ME), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :ents[b]] = perm[off:off + ents[b]]
        off += ents[b]
    shape = (NP, Hkv, 16, D) if block == 16 else (NP, Hkv, D)
    s0 = 9600 + 10 * seed
    kp = normal_tensor(shape, s0, 0.5, bf, DEV)
    vp = normal_tensor(shape, s0 + 1, 0.5, bf, DEV)
    q = normal_tensor((B, Hq, D), s0 + 2, 0.5, bf, DEV)
    tg = torch.from_numpy(table).to(DEV)
    lg = torch.from_numpy(lens).to(DEV)
    if block == 16:
        out, lse = ks.ks_paged_decode(q, kp, vp, tg, lg)
    else:
        out, lse = ks.ks_paged_decode_bs1(q, kp, vp, tg, lg)
    torch.cuda.synchronize()
    kh, vh = kp.float().cpu().numpy(), vp.float().cpu().numpy()
    if block == 1:
        kh, vh = kh[:, :, None], vh[:, :, None]
    live = lens > 0
    tag = f"block={block} B={B} Hq={Hq} Hkv={Hkv}"
    # zero-length sequences: a zero output and lse = -inf
    assert torch.all(out[torch.from_numpy(~live).to(DEV)] == 0), tag
    assert torch.all(torch.isinf(lse[torch.from_numpy(~live).to(DEV)])), tag
    if live.any():
        ro, rl = O.paged_decode(f64(q[torch.from_numpy(live).to(DEV)]), kh, vh, table[live],
                                lens[live])
        gate(out[torch.from_numpy(live).to(DEV)], ro, "bf16", f"decode out {tag}")
        gate(lse[torch.from_numpy(live).to(DEV)], rl, "bf16", f"decode lse {tag}")
