"""The toy decoder stack on the GPU: a 3-layer random-weight model whose
attention is the KV-streams path.  Its masked training pass and its
token-by-token generation over compacted paged caches are compared with the
oracle's stack (logits element by element, and the KL divergence of the
next-token distributions, the trainer/generator mismatch measure the pages
quote) and with each other."""
import numpy as np
import pytest
import torch

from kv_cache_compaction_amd.toy_stack import ToyStack
from oracle import toy_stack as T
from parity_util import announce, errors
from workloads import ToyShape, build_trace, check_trace, toy_tokens, toy_weights

pytestmark = pytest.mark.gpu
DEV = "cuda"
SHAPE = ToyShape(layers=3, vocab=512, d_model=512, Hq=4, Hkv=2, D=128, ffn=1024)
# bf16 bounds on KL(p || q) per token, nats.  GEMM operands and attention
# inputs are rounded to bf16 (relative 2^-9) at ~8 places per layer; over 3
# layers the logits move by ~1e-2 absolute at unit scale, i.e. a KL of order
# (1e-2)^2 / 2 = 5e-5 per token.  The bounds leave a factor of ~10.
KL_MEAN = 5e-4
KL_MAX = 5e-3
# element by element: the same ~24 bf16 roundings (2^-9 relative each) put an
# rms error of about 2^-9 sqrt(24) ~ 1e-2 of the logits' rms (~1) on each
# logit; measured 4.7e-3 (relative L2) and 6e-3 (max over max |ref|)
LOGIT_REL_L2 = 1e-2
LOGIT_REL_MAX = 1.5e-2


def check_logits(got, ref, what):
    er = errors(got, ref, "bf16")
    announce(f"{what} logits: rel_l2 {er['rel_l2']:.3g} rel_max {er['rel_max']:.3g} "
             f"max_abs {er['max_abs']:.3g}")
    assert er["finite"] and er["rel_l2"] <= LOGIT_REL_L2 and er["rel_max"] <= LOGIT_REL_MAX, \
        (what, er)


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)


@pytest.mark.parametrize("strategy,seed", [("recent", 21), ("summary", 22)])
def test_training_pass_matches_generation(strategy, seed):
    rng = np.random.default_rng(seed)
    kw = dict(overlap=64, summary=32) if strategy == "summary" else {}
    tr = build_trace(rng, 1024, 64, 512, strategy, turn_len=(48, 160), **kw)
    check_trace(tr)
    assert len(tr.events) >= 2
    w = toy_weights(SHAPE, seed)
    tok = toy_tokens(SHAPE, tr.N, seed)
    stack = ToyStack(w, SHAPE.Hq, SHAPE.Hkv, SHAPE.D)
    tg = torch.from_numpy(tok).to(DEV)
    eg = torch.from_numpy(tr.e.astype(np.int32)).to(DEV)
    lt = stack.train_logits(tg, eg)
    ld = stack.decode_logits(tg, tr.evicted)
    torch.cuda.synchronize()
    ref = T.train_logits(w, tok, tr.e, SHAPE.Hq, SHAPE.Hkv, SHAPE.D)
    lt, ld = lt.cpu().numpy(), ld.cpu().numpy()
    for name, got in (("train", lt), ("decode", ld)):
        check_logits(got, ref, f"{strategy} {name}")
        kl = T.kl_rows(ref, got)
        announce(f"{strategy} {name} vs oracle: KL mean {kl.mean():.3g} max {kl.max():.3g}")
        assert np.isfinite(got).all()
        assert kl.mean() <= KL_MEAN and kl.max() <= KL_MAX, (name, kl.mean(), kl.max())
    kl = T.kl_rows(lt, ld)
    announce(f"{strategy} train vs decode (mismatch): KL mean {kl.mean():.3g} max {kl.max():.3g}")
    assert kl.mean() <= KL_MEAN and kl.max() <= KL_MAX
    # generation that ignored the events would not match the training pass
    lk = stack.decode_logits(tg, {}).cpu().numpy()
    t1 = tr.events[0]
    assert T.kl_rows(lt[t1:], lk[t1:]).mean() > 10 * KL_MEAN


def test_single_token_blocks_generation_matches():
    """The SGLang setup: turns of any length (no padding to 16), token-run
    eviction, generation over single-token blocks; the training pass is the
    same masked call."""
    rng = np.random.default_rng(23)
    tr = build_trace(rng, 1024, 61, 512, "recent", turn_len=(37, 151), granule=1)
    check_trace(tr)
    assert len(tr.events) >= 2 and any(t % 16 for t in tr.events)
    w = toy_weights(SHAPE, 23)
    tok = toy_tokens(SHAPE, tr.N, 23)
    stack = ToyStack(w, SHAPE.Hq, SHAPE.Hkv, SHAPE.D)
    tg = torch.from_numpy(tok).to(DEV)
    lt = stack.train_logits(tg, torch.from_numpy(tr.e.astype(np.int32)).to(DEV))
    ld = stack.decode_logits(tg, tr.evicted, block_size=1)
    with pytest.raises(ValueError):
        stack.decode_logits(tg[:4], {1: [(0, 1)]}, block_size=16)   # span not block-aligned
    torch.cuda.synchronize()
    ref = T.train_logits(w, tok, tr.e, SHAPE.Hq, SHAPE.Hkv, SHAPE.D)
    lt, ld = lt.cpu().numpy(), ld.cpu().numpy()
    check_logits(lt, ref, "single-token train")
    check_logits(ld, ref, "single-token decode")
    for name, a, b in (("train vs oracle", ref, lt), ("decode vs oracle", ref, ld),
                       ("train vs decode (mismatch)", lt, ld)):
        kl = T.kl_rows(a, b)
        announce(f"single-token {name}: KL mean {kl.mean():.3g} max {kl.max():.3g}")
        assert kl.mean() <= KL_MEAN and kl.max() <= KL_MAX, (name, kl.mean(), kl.max())

