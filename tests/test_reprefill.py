"""The re-prefill counterfactual's separate traces (paper page, Fig. 2A and
Fig. 3): structure pinned on the CPU against what the pages state and the
trace rules imply."""
import numpy as np

from workloads import (KS_NEVER, SUMMARY_32K, TINY_F32, TRAINING_WORKLOADS, TRAIN_4K,
                       config_trace_batch, reprefill_segments)


def test_segments_cover_the_rollout_once_and_respect_the_budget():
    for cfg in TRAINING_WORKLOADS:
        traces, _ = config_trace_batch(cfg)
        for tr in traces:
            segs = reprefill_segments(tr)
            assert len(segs) == len(tr.events) + 1
            # new tokens of the segments tile [0, N) in order, exactly once
            bounds = [0] + list(tr.events) + [tr.N]
            for s, (a, b) in zip(segs, zip(bounds[:-1], bounds[1:])):
                new = s[s >= a]
                np.testing.assert_array_equal(new, np.arange(a, b))
                old = s[s < a]
                assert np.all(np.diff(s) > 0)         # order preserved
                # re-prefilled tokens are exactly the live ones at the event
                e = tr.e.astype(np.int64)
                np.testing.assert_array_equal(old, np.nonzero(e[:a] > a)[0] if a else old)
                # a segment is the live context between two events, which the
                # trigger keeps within the budget
                assert len(s) <= tr.budget


def test_summary_retains_prompt_plus_overlap_and_summary():
    traces, _ = config_trace_batch(SUMMARY_32K)
    for tr in traces:
        segs = reprefill_segments(tr)
        for s, t in zip(segs[1:], tr.events):
            kept = s[s < t]
            assert kept.size == tr.P + tr.overlap + tr.summary
            np.testing.assert_array_equal(kept[:tr.P], np.arange(tr.P))
            np.testing.assert_array_equal(kept[tr.P:], np.arange(t - tr.overlap - tr.summary, t))


def test_reprocessing_factor_matches_fig3():
    """Fig. 3: each kept token is re-processed about N / (B - (o+s)) times;
    the 32k summary traces give 5 events for a factor of 32768/6656 = 4.92,
    and the extra re-prefilled tokens are events x (P + o + s)."""
    traces, _ = config_trace_batch(SUMMARY_32K)
    for tr in traces:
        factor = tr.N / (tr.budget - (tr.overlap + tr.summary))
        assert abs(len(tr.events) - factor) < 1.0
        extra = sum(len(s) for s in reprefill_segments(tr)) - tr.N
        assert extra == len(tr.events) * (tr.P + tr.overlap + tr.summary)


def test_no_event_means_one_segment():
    traces, _ = config_trace_batch(TINY_F32)
    tr = traces[0]
    import dataclasses
    flat = dataclasses.replace(tr, events=[], e=np.full(tr.N, KS_NEVER, np.int32))
    segs = reprefill_segments(flat)
    assert len(segs) == 1
    np.testing.assert_array_equal(segs[0], np.arange(tr.N))


def _textbook_causal(q, k, v, do):
    """softmax(q k^T / sqrt(D) + causal mask) v and its gradients, written
    with torch autograd in fp64: [L, H, D] inputs, one segment."""
    import torch
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    L, H, D = q.shape
    s = torch.einsum("ihd,jhd->hij", q, k) / np.sqrt(D)
    s = s.masked_fill(~torch.ones(L, L, dtype=torch.bool).tril(), float("-inf"))
    o = torch.einsum("hij,jhd->ihd", torch.softmax(s, -1), v)
    o.backward(torch.tensor(do))
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def test_packed_sequence_is_the_separate_causal_passes():
    """One masked pass over the packed segments equals plain causal attention
    run on every segment on its own (forward and all three gradients); pads
    see only themselves."""
    import oracle as O
    from workloads import build_trace, check_trace, reprefill_pack
    rng = np.random.default_rng(77)
    tr = build_trace(rng, 1024, 64, 384, "summary", turn_len=(48, 112), overlap=64, summary=32)
    check_trace(tr)
    segs = reprefill_segments(tr)
    assert len(segs) >= 3
    n = sum(len(x) for x in segs)
    idx, e = reprefill_pack(tr, length=n + 37)
    H, D = 2, 32
    g = np.random.default_rng(5)
    q, k, v, do = (g.standard_normal((1, tr.N, H, D)) for _ in range(4))
    qp, kp, vp, dop = (x[:, idx] for x in (q, k, v, do))
    ep = e[None].astype(np.int64)
    o, lse = O.attn_fwd(qp, kp, vp, ep)
    dq, dk, dv = O.attn_bwd(qp, kp, vp, ep, dop)
    p = 0
    for x in segs:
        sl = slice(p, p + len(x))
        ro, rdq, rdk, rdv = _textbook_causal(q[0, x], k[0, x], v[0, x], do[0, x])
        for got, ref in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
            np.testing.assert_allclose(got[0, sl], ref, rtol=1e-10, atol=1e-10)
        p += len(x)
    # pads: the output is the pad's own value row, its key gets no gradient
    # from any real query
    np.testing.assert_allclose(o[0, n:], vp[0, n:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq[0, n:], 0.0, atol=1e-12)
    assert np.all(e[n:] == np.arange(n, n + 37) + 1)


def test_pack_rejects_short_length():
    import pytest as _pt
    from workloads import reprefill_pack
    traces, _ = config_trace_batch(TRAIN_4K)
    n = sum(len(x) for x in reprefill_segments(traces[0]))
    with _pt.raises(ValueError):
        reprefill_pack(traces[0], length=n - 1)
