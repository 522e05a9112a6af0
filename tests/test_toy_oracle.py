"""Pins of the oracle's toy decoder stack (CPU): the masked training pass and
token-by-token generation with physical eviction agree at every layer, and
without events the stack is a plain causal transformer."""
import numpy as np
import torch

from oracle import toy_stack as T
from workloads import KS_NEVER, ToyShape, build_trace, check_trace, toy_tokens, toy_weights

SMALL = ToyShape(layers=2, vocab=64, d_model=64, Hq=4, Hkv=2, D=16, ffn=128)


def _trace(strategy, seed):
    rng = np.random.default_rng(seed)
    kw = dict(overlap=32, summary=16) if strategy == "summary" else {}
    tr = build_trace(rng, 320, 32, 160, strategy, turn_len=(32, 64), **kw)
    check_trace(tr)
    assert len(tr.events) >= 2
    return tr


def test_training_pass_equals_generation_with_eviction():
    w = toy_weights(SMALL, 1)
    s = SMALL
    for strategy, seed in (("recent", 2), ("summary", 3), ("window", 4)):
        tr = _trace(strategy, seed)
        tok = toy_tokens(s, tr.N, seed)
        a = T.train_logits(w, tok, tr.e, s.Hq, s.Hkv, s.D)
        b = T.decode_logits(w, tok, tr.evicted, s.Hq, s.Hkv, s.D)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-9)
        # the events matter: generation that keeps everything differs after
        # the first event, and only there
        c = T.decode_logits(w, tok, {}, s.Hq, s.Hkv, s.D)
        t1 = tr.events[0]
        np.testing.assert_allclose(c[:t1], a[:t1], atol=1e-9)
        assert np.abs(c[t1:] - a[t1:]).max() > 1e-3


def _torch_causal_stack(w, tok, s):
    """The same architecture written with torch ops and torch's causal SDPA
    (fp64), RoPE as complex rotation of (x_k, x_{k+D/2}) pairs."""
    f = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)
    N = len(tok)
    x = f(w["emb"])[torch.tensor(tok)]
    pos = torch.arange(N, dtype=torch.float64)
    inv = 10000.0 ** (-2.0 * torch.arange(s.D // 2, dtype=torch.float64) / s.D)
    ang = pos[:, None] * inv[None]
    rot = torch.polar(torch.ones_like(ang), ang)                     # [N, D/2]

    def rope(t):                                                     # [N, H, D]
        c = torch.complex(t[..., :s.D // 2], t[..., s.D // 2:]) * rot[:, None]
        return torch.cat([c.real, c.imag], -1)
    norm = lambda t: t / torch.sqrt((t * t).mean(-1, keepdim=True) + 1e-6)
    G = s.Hq // s.Hkv
    for L in w["layers"]:
        a = norm(x)
        q = rope((a @ f(L["wq"])).view(N, s.Hq, s.D))
        k = rope((a @ f(L["wk"])).view(N, s.Hkv, s.D)).repeat_interleave(G, 1)
        v = (a @ f(L["wv"])).view(N, s.Hkv, s.D).repeat_interleave(G, 1)
        o = torch.nn.functional.scaled_dot_product_attention(
            q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), is_causal=True)
        x = x + o.transpose(0, 1).reshape(N, -1) @ f(L["wo"])
        x = x + torch.nn.functional.silu(norm(x) @ f(L["w1"])) @ f(L["w2"])
    return (norm(x) @ f(w["unemb"])).numpy()


def test_no_events_is_a_causal_transformer():
    s = SMALL
    w = toy_weights(s, 5)
    N = 97
    tok = toy_tokens(s, N, 6)
    e = np.full(N, KS_NEVER)
    ref = _torch_causal_stack(w, tok, s)
    np.testing.assert_allclose(T.train_logits(w, tok, e, s.Hq, s.Hkv, s.D), ref, atol=1e-10)
    np.testing.assert_allclose(T.decode_logits(w, tok, {}, s.Hq, s.Hkv, s.D), ref, atol=1e-10)


def test_kl_rows():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((5, 7))
    assert np.allclose(T.kl_rows(a, a), 0.0, atol=1e-15)
    assert np.allclose(T.kl_rows(a, a + 3.0), 0.0, atol=1e-12)      # shift invariant
    b = rng.standard_normal((5, 7))
    p = np.exp(a) / np.exp(a).sum(-1, keepdims=True)
    q = np.exp(b) / np.exp(b).sum(-1, keepdims=True)
    np.testing.assert_allclose(T.kl_rows(a, b), (p * np.log(p / q)).sum(-1), rtol=1e-12)
