"""Synthetic rollout traces, compaction-event records and paged block tables.

The rules below stand in for the rollouts of the KV-streams paper
("KV-streams for Efficient Compaction in Agentic Reinforcement Learning",
Penaloza et al.).  The pages fix only the qualitative structure:

* a rollout is a prompt followed by turns; when the live context reaches its
  budget a compaction event removes older turns and keeps the prompt, recent
  turns or a summary (wqu.guru explainer, opening paragraphs; paper page,
  Fig. 2B "P: prompt; S: summary");
* whole turns are removed, boundary tokens included (explainer, paragraph on
  token-level eviction);
* every completion is padded to a multiple of 16 tokens so that events fall on
  16-token block boundaries (explainer, paragraph on vLLM's 16-token blocks);
* the trainer replays the recorded events as a mask over one continuous trace
  (explainer, paragraph on the trainer; paper page, Fig. 2A).

Everything quantitative (turn-length law, trigger, how much is evicted) is a
reading stated in the docstrings here.  This module only *constructs inputs*:
it never computes attention, RoPE or a compacted table.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

KS_NEVER = 2**31 - 1      # e_j of a token that is never evicted
BLOCK = 16                # tokens per KV block


def _round_up(x: int, g: int) -> int:
    return (int(x) + g - 1) // g * g


@dataclass
class Trace:
    """One continuous rollout trace and its compaction history.

    ``e[j]`` is the trace index of the event that evicted token ``j``
    (``KS_NEVER`` if never evicted); query ``i`` may attend key ``j`` iff
    ``j <= i < e[j]``.  An event at index ``t`` fires after token ``t-1`` and
    before token ``t`` is generated, so token ``t-1`` still saw everything it
    evicts.
    """
    N: int
    P: int
    budget: int
    strategy: str
    turns: list                      # [(start, end)] of non-prompt turns
    events: list                     # sorted event indices
    evicted: dict                    # event index -> [(a, b)] evicted spans
    e: np.ndarray = field(repr=False)  # int32 [N]
    live_units: list = field(default_factory=list)  # live spans after the trace
    overlap: int = 0
    summary: int = 0
    granule: int = BLOCK             # turn lengths are multiples of this


def build_trace(rng: np.random.Generator, N: int, P: int, budget: int,
                strategy: str, turn_len=(64, 512), overlap: int = 0,
                summary: int = 0, granule: int = BLOCK) -> Trace:
    """Build one trace.

    Turn lengths are integers uniform on ``turn_len`` (inclusive), rounded up
    to a multiple of ``granule``; a fixed length is given as
    ``turn_len=(L, L)``.  The last turn is cut at ``N``.  ``granule`` 16 is
    the vLLM setup, whose completions are padded to whole 16-token blocks;
    ``granule`` 1 is the SGLang setup with single-token blocks and no padding
    (explainer, paragraph on turns ending inside a block).

    Trigger: at the end of a turn, if the live size plus the next turn's
    length would exceed ``budget``, an event fires at that turn end.

    Strategies:
      ``recent``  pop the oldest complete non-prompt turns until live <= B/2
                  (the prompt is pinned);
      ``window``  the same, but the prompt is the oldest turn and may be popped;
      ``summary`` keep the prompt and the last ``overlap + summary`` tokens
                  before the event; everything else that is live is evicted.
    """
    if strategy not in ("recent", "window", "summary"):
        raise ValueError(strategy)
    lo, hi = turn_len
    turns = []
    t = P
    while t < N:
        L = _round_up(rng.integers(lo, hi + 1), granule) if lo != hi else lo
        end = min(t + L, N)
        turns.append((t, end))
        t = end

    e = np.full(N, KS_NEVER, dtype=np.int64)
    units = [(0, P)] if P > 0 else []   # live spans, oldest first
    events, evicted = [], {}
    for idx, (a, b) in enumerate(turns):
        units.append((a, b))
        if idx + 1 == len(turns):
            break
        nxt = turns[idx + 1][1] - turns[idx + 1][0]
        live = sum(y - x for x, y in units)
        if live + nxt <= budget:
            continue
        t_ev = b
        units, out = evict_units(units, t_ev, strategy, budget, P, overlap, summary)
        for (x, y) in out:
            e[x:y] = t_ev
        events.append(t_ev)
        evicted[t_ev] = out
    return Trace(N=N, P=P, budget=budget, strategy=strategy, turns=turns,
                 events=events, evicted=evicted, e=e.astype(np.int32),
                 live_units=list(units), overlap=overlap, summary=summary,
                 granule=granule)


def evict_units(units, t_ev, strategy, budget, P, overlap=0, summary=0):
    """Apply one compaction event at trace index ``t_ev`` to the live spans
    ``units`` (oldest first; the prompt, if any, is ``units[0]``).

    Returns ``(kept_units, evicted_spans)`` following the strategy rules of
    ``build_trace``.
    """
    units = list(units)
    live = sum(y - x for x, y in units)
    out = []
    if strategy in ("recent", "window"):
        first = 0 if (strategy == "window" or P == 0) else 1
        target = budget // 2
        while live > target and len(units) > first + 1:
            u = units.pop(first)
            out.append(u)
            live -= u[1] - u[0]
        return units, out
    keep_lo = t_ev - (overlap + summary)
    kept = [units[0]] if P > 0 else []
    for (x, y) in (units[1:] if P > 0 else units):
        if y <= keep_lo:
            out.append((x, y))
        elif x >= keep_lo:
            kept.append((x, y))
        else:
            out.append((x, keep_lo))
            kept.append((keep_lo, y))
    return kept, out


def check_trace(tr: Trace) -> None:
    """Assert the structural invariants every generated trace must satisfy."""
    N, e = tr.N, tr.e.astype(np.int64)
    j = np.arange(N)
    assert np.all(e > j), "e_j > j violated"
    ev = set(tr.events)
    assert all(int(x) in ev or int(x) == KS_NEVER for x in np.unique(e))
    g = tr.granule
    assert all(t % g == 0 for t in tr.events), "events must be granule-aligned"
    assert all(x % g == 0 and (y % g == 0 or y == tr.N) for (x, y) in tr.turns)
    # live size at every query index is within budget:
    # |live(i)| = (i+1) - #{j <= i : e_j <= i}
    ev_hist = np.zeros(N + 1, dtype=np.int64)
    fin = e[e < N]
    np.add.at(ev_hist, fin, 1)
    gone = np.cumsum(ev_hist)[:N]
    live = (j + 1) - gone
    assert live.max() <= tr.budget, (live.max(), tr.budget)
    if tr.strategy in ("recent", "window"):
        for (x, y) in tr.turns:
            assert np.all(e[x:y] == e[x]), "window strategies evict whole turns"
    if tr.strategy != "window" and tr.P > 0:
        assert np.all(e[:tr.P] == KS_NEVER), "prompt pinned"


def trace_blocks_keep(tr: Trace) -> np.ndarray:
    """Keep flag per 16-token block of the trace after its last event.

    A block is kept iff none of its tokens was evicted.  (Derived from the
    per-token record; the oracle derives its expected table from the event
    list instead.)
    """
    nb = (tr.N + BLOCK - 1) // BLOCK
    pad = np.full(nb * BLOCK, KS_NEVER, dtype=np.int64)
    pad[:tr.N] = tr.e
    return (pad.reshape(nb, BLOCK) == KS_NEVER).all(axis=1).astype(np.uint8)


def reprefill_segments(tr: Trace) -> list:
    """The separate training traces of re-prefill compaction on the same
    rollout (paper page, Fig. 2A: retained tokens are recomputed and every
    compaction starts a new trace).  Segment 0 is tokens [0, t_1); segment k
    is the tokens kept at event t_k -- {j < t_k : e_j > t_k}, re-prefilled in
    order -- followed by the new tokens [t_k, t_(k+1)) (t_(K+1) = N).  Returns
    a list of int64 arrays of trace token indices, one per segment; each is a
    plain causal sequence of its own."""
    ev = list(tr.events)
    bounds = [0] + ev + [tr.N]
    segs = []
    e = tr.e.astype(np.int64)
    for k in range(len(bounds) - 1):
        t, t_next = bounds[k], bounds[k + 1]
        kept = np.nonzero(e[:t] > t)[0] if k > 0 else np.zeros(0, np.int64)
        segs.append(np.concatenate([kept, np.arange(t, t_next)]).astype(np.int64))
    return segs


def reprefill_pack(tr: Trace, length: int | None = None):
    """The re-prefill segments of ``tr`` laid end to end in one sequence.

    Key ``j`` of the packed sequence gets the end of its segment as its
    eviction index, so under the rule j <= i < e_j every query sees exactly
    the earlier keys of its own segment: one masked pass over the packed
    sequence is the separate causal passes of the segments.  ``length`` pads
    the sequence on the right; a pad token is seen by itself only
    (e_j = j + 1), so it adds no work beyond its own diagonal tile and no
    row is empty.

    Returns ``(index, e)``: ``index[p]`` is the rollout token at packed
    position ``p`` (0 for pads), ``e`` the int32 eviction indices.
    """
    segs = reprefill_segments(tr)
    n = sum(len(x) for x in segs)
    length = n if length is None else int(length)
    if length < n:
        raise ValueError(f"length {length} < packed size {n}")
    index = np.zeros(length, np.int64)
    e = np.arange(1, length + 1, dtype=np.int64)
    p = 0
    for x in segs:
        index[p:p + len(x)] = x
        e[p:p + len(x)] = p + len(x)
        p += len(x)
    return index, e.astype(np.int32)


@dataclass
class DecodeBatch:
    """Paged caches of several sequences before a run of compaction rounds.

    ``table0``      int32 [B, MB] physical block ids before any round (-1 pad);
                    logical block x of sequence b holds tokens
                    [block*x, block*x + block), and the last listed block is a
                    fresh block that receives the decoded token.
    ``nblk0``       int32 [B] listed blocks before any round.
    ``keeps``       uint8 [R, B, MB] keep flags for round r, relative to the
                    table as it stands before round r (zeros past the end).
    ``runs``        per sequence, the evicted logical-block ranges [x0, x1) in
                    the order of the events that evict them.
    ``event_pos``   per sequence, the trace index of each event.
    ``live_len``    int32 [B] live tokens before the decoded token (L_b).
    ``pos``         int32 [B] logical position of the decoded token (T_b).
    ``num_pool_blocks`` physical blocks in the pool.
    ``block``       tokens per block (16, or 1 for single-token blocks, where
                    the table lists token slots).
    """
    table0: np.ndarray
    nblk0: np.ndarray
    keeps: np.ndarray
    runs: list
    event_pos: list
    live_len: np.ndarray
    pos: np.ndarray
    num_pool_blocks: int
    block: int = BLOCK


def build_decode_batch(rng: np.random.Generator, n_seqs: int,
                       live_range=(4096, 16384), max_pos: int = 65536,
                       events_range=(1, 6), block: int = BLOCK) -> DecodeBatch:
    """Paged caches compacted by 1-6 events, then one decode step.

    Per sequence: live length ``L`` uniform on the ``block``-aligned values of
    ``live_range``; event count ``K`` uniform on ``events_range``; the
    pre-compaction length ``T`` uniform ``block``-aligned on
    ``[L + block*K, max_pos]``.  The ``(T-L)/block`` evicted blocks form ``K``
    runs of whole blocks that never touch block 0 (the prompt) or the last
    block; run ``r`` is removed by event ``r``.  Physical ids are a seeded
    permutation of the pool.  The decoded token sits at logical position
    ``T`` in a fresh block appended to the table, so ``seq_len = L + 1``.
    With ``block`` 1 every quantity is token-granular: turns and evicted runs
    end anywhere and the table lists one pool slot per token.
    """
    lo, hi = live_range
    bs = int(block)
    Ls, Ts, Ks, runs_all, evs_all = [], [], [], [], []
    for _ in range(n_seqs):
        L = bs * int(rng.integers(lo // bs, hi // bs + 1))
        K = int(rng.integers(events_range[0], events_range[1] + 1))
        T = bs * int(rng.integers((L + bs * K) // bs, max_pos // bs + 1))
        nb_ev = (T - L) // bs
        nb_keep = L // bs
        # sizes of the K evicted runs (each >= 1 block)
        cuts = np.sort(rng.choice(np.arange(1, nb_ev), K - 1, replace=False)) \
            if K > 1 else np.array([], dtype=np.int64)
        sizes = np.diff(np.concatenate([[0], cuts, [nb_ev]])).astype(np.int64)
        # K+1 gaps of kept blocks, each >= 1, summing to nb_keep
        gcuts = np.sort(rng.choice(np.arange(1, nb_keep), K, replace=False))
        gaps = np.diff(np.concatenate([[0], gcuts, [nb_keep]])).astype(np.int64)
        runs, x = [], 0
        for r in range(K):
            x += int(gaps[r])
            runs.append((x, x + int(sizes[r])))
            x += int(sizes[r])
        assert x + int(gaps[K]) == T // bs
        # event r fires at the end of the kept gap that follows run r
        evs = [bs * runs[r + 1][0] if r + 1 < K else T for r in range(K)]
        Ls.append(L); Ts.append(T); Ks.append(K)
        runs_all.append(runs); evs_all.append(evs)

    nblk0 = np.array([T // bs + 1 for T in Ts], dtype=np.int32)
    MB = int(nblk0.max())
    NB = int(nblk0.sum())
    perm = rng.permutation(NB).astype(np.int32)
    table0 = np.full((n_seqs, MB), -1, dtype=np.int32)
    off = 0
    for b in range(n_seqs):
        n = int(nblk0[b])
        table0[b, :n] = perm[off:off + n]
        off += n

    R = max(Ks)
    keeps = np.zeros((R, n_seqs, MB), dtype=np.uint8)
    for b in range(n_seqs):
        logical = np.arange(int(nblk0[b]))          # logical ids currently listed
        for r in range(R):
            if r < Ks[b]:
                x0, x1 = runs_all[b][r]
                flags = (logical < x0) | (logical >= x1)
            else:
                flags = np.ones(len(logical), dtype=bool)
            keeps[r, b, :len(logical)] = flags
            logical = logical[flags]
    return DecodeBatch(table0=table0, nblk0=nblk0, keeps=keeps,
                       runs=runs_all, event_pos=evs_all,
                       live_len=np.array(Ls, dtype=np.int32),
                       pos=np.array(Ts, dtype=np.int32),
                       num_pool_blocks=NB, block=bs)


@dataclass
class Continuation:
    """Paged layout of training traces continued by decoding (see
    ``continuation_layout``)."""
    table0: np.ndarray      # [B, MB] physical block ids, -1 past nblk0
    nblk0: np.ndarray       # [B] listed blocks: the live set, then the fresh blocks
    live_len: np.ndarray    # [B] live tokens at the end of each trace
    live_tok: list          # per trace: trace indices of its live tokens, in order
    logical: list           # per trace: first trace index of each listed block
    num_pool_blocks: int
    keep: np.ndarray        # [B, MB] uint8 flags of the forced event over the listed blocks
    ev_spans: list          # per trace: the spans the forced event evicts
    ev_tokens: np.ndarray   # [B] tokens the forced event evicts
    t_ev: int               # trace index of the forced event


def continuation_layout(traces, N: int, ndec: int, event_after: int,
                        rng: np.random.Generator, block: int = BLOCK) -> Continuation:
    """Training traces of length ``N`` continued by ``ndec`` decoded tokens.

    Each trace's live set at its end fills whole ``block``-token blocks of one
    shared pool (physical ids a seeded permutation), followed by
    ``ndec / block`` fresh blocks for the decoded tokens at trace indices
    ``N, N + 1, ...``.  After ``event_after`` new tokens a forced compaction
    event at ``t_ev = N + event_after`` applies the trace's own strategy to
    its live spans plus the decoded span; ``keep`` holds that event's flags
    over the listed blocks.
    """
    B = len(traces)
    live_tok = [np.concatenate([np.arange(x, y) for (x, y) in tr.live_units]) for tr in traces]
    L0 = np.array([len(t) for t in live_tok])
    assert np.all(L0 % block == 0) and ndec % block == 0
    nfresh = ndec // block
    nblk0 = (L0 // block + nfresh).astype(np.int32)
    MB = int(nblk0.max())
    NB = int(nblk0.sum())
    perm = rng.permutation(NB).astype(np.int32)
    table0 = np.full((B, MB), -1, np.int32)
    logical = []
    off = 0
    for b in range(B):
        n = int(nblk0[b])
        table0[b, :n] = perm[off:off + n]
        off += n
        logical.append(np.concatenate([live_tok[b][::block], N + block * np.arange(nfresh)]))
    t_ev = N + event_after
    ev_spans = []
    for tr in traces:
        units = list(tr.live_units) + [(N, t_ev)]
        _, out = evict_units(units, t_ev, tr.strategy, tr.budget, tr.P, tr.overlap, tr.summary)
        ev_spans.append(out)
    keep = np.zeros((B, MB), np.uint8)
    ev_tokens = np.zeros(B, np.int64)
    for b in range(B):
        gone = np.zeros(N + ndec, bool)
        for (x, y) in ev_spans[b]:
            gone[x:y] = True
            ev_tokens[b] += y - x
        keep[b, :nblk0[b]] = ~gone[logical[b]]
    return Continuation(table0=table0, nblk0=nblk0, live_len=L0, live_tok=live_tok,
                        logical=logical, num_pool_blocks=NB, keep=keep, ev_spans=ev_spans,
                        ev_tokens=ev_tokens, t_ev=t_ev)


def normal_tensor(shape, seed: int, scale: float = 1.0, dtype=None,
                  device: str = "cpu"):
    """N(0,1)*scale tensor, drawn in fp32 and rounded (RNE) to ``dtype`` once.

    On the CPU the draw is numpy PCG64 (``default_rng(seed)``); on a GPU it is
    torch's seeded device generator.  Either way both sides of a comparison
    consume the same rounded values.
    """
    import torch
    dtype = dtype or torch.float32
    if str(device) == "cpu":
        x = np.random.default_rng(seed).standard_normal(tuple(shape), dtype=np.float32)
        t = torch.from_numpy(x)
        if scale != 1.0:
            t = t * scale
        return t.to(dtype)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        t = t * scale
    return t.to(dtype)
