"""fp64 reference implementation of the KV-streams hot path (CPU, numpy).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Slow on purpose: every
function is the plain definition, with an explicit boolean mask and no
blocking, fusion or online softmax.

Sources (the KV-streams paper, "KV-streams for Efficient Compaction in Agentic
Reinforcement Learning", as presented on the pages): "the explainer" is the
wqu.guru article "KV-streams: accelerating agentic RL training by operating
on the KV cache directly"; "the paper page" is the thelatestinai.com summary
of the paper (abstract, Fig. 2A, Fig. 3).

* RoPE at logical positions: cached keys keep the rotation of their original
  position, and new queries and keys continue the original position count
  (explainer, the paragraph on RoPE after compaction and the one after it).
* Eviction mask: training replays the logged compaction events; a token
  evicted at an event is invisible to every query from that event on, and
  every surviving entry is the one computed when its token was generated
  (explainer, trainer paragraph; paper page, Fig. 2A, where the mask stands
  for the eviction).  Written as M_ij = [j <= i] and [i < e_j].
* Block-table compaction: remove complete 16-token blocks and join the
  remaining block references, leaving no holes (explainer, the paragraph on
  vLLM's 16-token blocks and the one after it).
* Decode: attention of the new query over the live keys gathered through the
  compacted table.

Readings where the pages are silent: NeoX rotate-half pairing (k, k + D/2);
theta_k = pos * base^(-2k/D); softmax scale 1/sqrt(D); GQA maps query head h
to kv head floor(h / G).

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
closed forms, library routines, invariants and brute force.  No function is
"parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

KS_NEVER = 2**31 - 1
BLOCK = 16


# ---------------------------------------------------------------------------
# RoPE at logical position
# ---------------------------------------------------------------------------
def rope(x: np.ndarray, pos: np.ndarray, base: float = 10000.0,
         inverse: bool = False) -> np.ndarray:
    """Rotate-half RoPE of ``x`` [B, N, H, D] by positions ``pos`` [B, N].

    For k < D/2 and theta = pos * base^(-2k/D):
      x'[k]       = x[k] cos(theta) - x[k + D/2] sin(theta)
      x'[k + D/2] = x[k + D/2] cos(theta) + x[k] sin(theta)
    ``inverse`` rotates by -theta (the transpose of the rotation, i.e. the
    RoPE backward).  Positions are logical token positions.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    kk = np.arange(half, dtype=np.float64)
    inv_freq = np.power(float(base), -2.0 * kk / D)
    theta = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq  # [B,N,half]
    if inverse:
        theta = -theta
    c = np.cos(theta)[:, :, None, :]
    s = np.sin(theta)[:, :, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ---------------------------------------------------------------------------
# Eviction-masked attention
# ---------------------------------------------------------------------------
def eviction_mask(e: np.ndarray, rows: np.ndarray, n_keys: int) -> np.ndarray:
    """Boolean mask [len(rows), n_keys]: M_ij = (j <= i) and (i < e_j)."""
    rows = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(n_keys, dtype=np.int64)[None, :]
    ej = np.asarray(e, dtype=np.int64)[None, :n_keys]
    return (j <= rows) & (rows < ej)


def live_keys(e: np.ndarray, i: int) -> np.ndarray:
    """Indices of the keys live at query i: {j <= i : e_j > i}."""
    j = np.arange(i + 1)
    return j[np.asarray(e, dtype=np.int64)[: i + 1] > i]


def _scale(D, scale):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def attn_fwd_rows(q, k, v, e, b, h, rows, scale=None):
    """Output rows ``rows`` of query head ``h`` of trace ``b``.

    Returns (o [len(rows), D], lse [len(rows)]).  S_ij = scale q_i.k_j over
    the keys j of the causal prefix, masked by M; LSE_i = log sum_M exp S_ij;
    O_i = sum_M exp(S_ij - LSE_i) v_j.  Only the key columns live for at
    least one of the rows are formed (a column masked in every row adds
    nothing to any sum); the mask is applied element by element inside them.
    """
    Hq, Hkv, D = q.shape[2], k.shape[2], q.shape[3]
    kv = h // (Hq // Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    n_keys = int(rows.max()) + 1
    M = eviction_mask(e[b], rows, n_keys)
    cols = np.flatnonzero(M.any(axis=0))
    M = M[:, cols]
    qq = np.asarray(q[b, rows, h], dtype=np.float64)
    kk = np.asarray(k[b, cols, kv], dtype=np.float64)
    vv = np.asarray(v[b, cols, kv], dtype=np.float64)
    S = (qq @ kk.T) * _scale(D, scale)
    S = np.where(M, S, -np.inf)
    # a row that sees no key (only possible when a record breaks e_j > j)
    # is an empty softmax: O = 0, LSE = -inf
    empty = ~M.any(axis=1, keepdims=True)
    m = np.where(empty, 0.0, S.max(axis=1, keepdims=True, initial=-np.inf))
    Pu = np.exp(S - m)
    l = Pu.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))[:, 0]
    o = (Pu / np.where(empty, 1.0, l)) @ vv
    return o, lse


def attn_fwd(q, k, v, e, scale=None, row_chunk=512):
    """Full forward.  q [B,N,Hq,D], k/v [B,N,Hkv,D], e [B,N].

    Returns o [B,N,Hq,D] and lse [B,Hq,N] (fp64).
    """
    B, N, Hq, D = q.shape
    o = np.zeros((B, N, Hq, D))
    lse = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            for i0 in range(0, N, row_chunk):
                rows = np.arange(i0, min(N, i0 + row_chunk))
                ob, lb = attn_fwd_rows(q, k, v, e, b, h, rows, scale)
                o[b, rows, h] = ob
                lse[b, h, rows] = lb
    return o, lse


def _bwd_rows_core(q, k, v, e, do, b, h, rows, scale):
    """P, dS and the row-local pieces for query rows ``rows`` of head h.

    The sums run over the live set: a key column that no row of ``rows``
    may attend (M_ij = 0 in every row) has P = dS = 0 there, so only the
    columns ``cols`` live for at least one row are formed; the mask is still
    applied element by element inside them.
    """
    Hq, Hkv, D = q.shape[2], k.shape[2], q.shape[3]
    kv = h // (Hq // Hkv)
    sc = _scale(D, scale)
    rows = np.asarray(rows, dtype=np.int64)
    n_keys = int(rows.max()) + 1
    M = eviction_mask(e[b], rows, n_keys)
    cols = np.flatnonzero(M.any(axis=0))
    M = M[:, cols]
    qq = np.asarray(q[b, rows, h], dtype=np.float64)
    kk = np.asarray(k[b, cols, kv], dtype=np.float64)
    vv = np.asarray(v[b, cols, kv], dtype=np.float64)
    dd = np.asarray(do[b, rows, h], dtype=np.float64)
    S = (qq @ kk.T) * sc
    S = np.where(M, S, -np.inf)
    empty = ~M.any(axis=1, keepdims=True)              # rows that see no key: P = 0
    m = np.where(empty, 0.0, S.max(axis=1, keepdims=True, initial=-np.inf))
    Pu = np.exp(S - m)
    P = Pu / np.where(empty, 1.0, Pu.sum(axis=1, keepdims=True))   # softmax over live keys
    dP = dd @ vv.T                                     # dP_ij = dO_i . v_j
    Di = (P * dP).sum(axis=1, keepdims=True)           # sum_j P_ij dP_ij
    dS = P * (dP - Di)
    return qq, kk, dd, P, dS, sc, cols, kv


def attn_bwd(q, k, v, e, do, scale=None, row_chunk=512):
    """Full backward of the masked forward with respect to its inputs.

    Softmax backward (standard calculus, the pages are silent on it):
      dV_j = sum_i P_ij dO_i
      dP_ij = dO_i . v_j
      dS_ij = P_ij (dP_ij - sum_l P_il dP_il)
      dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i
    dK and dV sum over the query heads sharing a kv head.  Gradients are with
    respect to the (already rotated) q and k that the forward consumed.
    """
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    dq = np.zeros((B, N, Hq, D))
    dk = np.zeros((B, N, Hkv, D))
    dv = np.zeros((B, N, Hkv, D))
    for b in range(B):
        for h in range(Hq):
            for i0 in range(0, N, row_chunk):
                rows = np.arange(i0, min(N, i0 + row_chunk))
                qq, kk, dd, P, dS, sc, cols, kv = _bwd_rows_core(
                    q, k, v, e, do, b, h, rows, scale)
                dq[b, rows, h] = sc * (dS @ kk)
                dk[b, cols, kv] += sc * (dS.T @ qq)
                dv[b, cols, kv] += P.T @ dd
    return dq, dk, dv


def attn_bwd_rows(q, k, v, e, do, b, h, rows, scale=None):
    """dQ rows ``rows`` of query head ``h`` of trace ``b`` (fp64)."""
    _, kk, _, _, dS, sc, _, _ = _bwd_rows_core(q, k, v, e, do, b, h, rows, scale)
    return sc * (dS @ kk)


def attn_bwd_keys(q, k, v, e, do, b, kv, keys, scale=None, row_chunk=512):
    """dK, dV of keys ``keys`` of kv head ``kv`` of trace ``b`` (fp64).

    Sums over every query row that can see any of the keys (rows
    [min(keys), max over keys of min(e_j, N))) and over the kv head's query
    heads.  Returns (dk [len(keys), D], dv [len(keys), D]).
    """
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    keys = np.asarray(keys, dtype=np.int64)
    ek = np.asarray(e[b], dtype=np.int64)[keys]
    r0 = int(keys.min())
    r1 = int(min(N, ek.max()))
    dk = np.zeros((len(keys), D))
    dv = np.zeros((len(keys), D))
    for h in range(kv * G, (kv + 1) * G):
        for i0 in range(r0, r1, row_chunk):
            rows = np.arange(i0, min(r1, i0 + row_chunk))
            qq, kk, dd, P, dS, sc, cols, _ = _bwd_rows_core(
                q, k, v, e, do, b, h, rows, scale)
            # the requested keys among the formed columns (the others have
            # no live query in these rows)
            at = np.searchsorted(cols, keys)
            hit = at < len(cols)
            hit[hit] = cols[at[hit]] == keys[hit]
            idx = np.flatnonzero(hit)
            sel = at[idx]
            dk[idx] += sc * (dS[:, sel].T @ qq)
            dv[idx] += P[:, sel].T @ dd
    return dk, dv


# ---------------------------------------------------------------------------
# Block-table compaction
# ---------------------------------------------------------------------------
def compact_block_table(table, nblk, keep):
    """Splice out dropped blocks and join the survivors, order preserved.

    table int [B, MB] physical ids, nblk int [B] listed blocks, keep [B, MB]
    flags.  Returns (table' int32 [B, MB] with -1 past the end, n' int32 [B]).
    """
    table = np.asarray(table)
    B, MB = table.shape
    out = np.full((B, MB), -1, dtype=np.int32)
    n_out = np.zeros(B, dtype=np.int32)
    for b in range(B):
        kept = [int(table[b][x]) for x in range(int(nblk[b])) if keep[b][x]]
        out[b, :len(kept)] = kept
        n_out[b] = len(kept)
    return out, n_out


# ---------------------------------------------------------------------------
# Paged GQA decode
# ---------------------------------------------------------------------------
def paged_decode(q, k_pool, v_pool, table, seq_lens, scale=None):
    """One decode step over paged caches.

    q [B, Hq, D] (already rotated at its logical position); k_pool, v_pool
    [NB, Hkv, BS, D] (keys stored rotated at their own logical positions);
    table [B, MB]; seq_lens [B].  Sequence b attends the first seq_lens[b]
    tokens reached through its table.  Returns (out [B, Hq, D], lse [B, Hq]).

    The block size BS is the pool's third axis: 16 for the vLLM setup, 1 for
    SGLang's single-token blocks, whose table lists one pool slot per token
    (explainer, paragraph on padding completions to whole blocks).
    """
    B, Hq, D = q.shape
    Hkv, BS = k_pool.shape[1], k_pool.shape[2]
    G = Hq // Hkv
    sc = _scale(D, scale)
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(seq_lens[b])
        nb = (L + BS - 1) // BS
        blocks = [int(table[b][x]) for x in range(nb)]
        for kv in range(Hkv):
            keys = np.concatenate([np.asarray(k_pool[p, kv], dtype=np.float64)
                                   for p in blocks], axis=0)[:L]
            vals = np.concatenate([np.asarray(v_pool[p, kv], dtype=np.float64)
                                   for p in blocks], axis=0)[:L]
            for h in range(kv * G, (kv + 1) * G):
                s = keys @ np.asarray(q[b, h], dtype=np.float64) * sc
                m = s.max()
                w = np.exp(s - m)
                z = w.sum()
                out[b, h] = (w / z) @ vals
                lse[b, h] = m + math.log(z)
    return out, lse


# ---------------------------------------------------------------------------
# Input checks (counts of precondition violations)
# ---------------------------------------------------------------------------
def count_bad_e(e):
    """Per trace, the tokens whose eviction index does not exceed their own
    index (e_j <= j): such a token would be evicted before it exists."""
    e = np.asarray(e, dtype=np.int64)
    return np.array([sum(1 for j in range(e.shape[1]) if e[b, j] <= j)
                     for b in range(e.shape[0])], dtype=np.int32)


def count_bad_table(table, seq_lens, num_pool_blocks, block_size):
    """Per sequence, the entries among the first ceil(L/BS) of its table row
    (L clamped to the row) that are not pool indices, plus one if L is
    negative or longer than the row can hold."""
    table = np.asarray(table)
    B, MB = table.shape
    out = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(seq_lens[b])
        cap = block_size * MB
        n = 0 if L <= 0 else (min(L, cap) + block_size - 1) // block_size
        bad = sum(1 for x in range(n) if not (0 <= int(table[b, x]) < num_pool_blocks))
        out[b] = bad + (1 if (L < 0 or L > cap) else 0)
    return out

