"""A model of where the bf16 attention kernels round, for the gradient gates.

Test infrastructure (not an oracle): fp64 arithmetic with bf16 round-to-
nearest-even applied at the points where the HIP kernels store or feed bf16
values, so its distance from the fp64 oracle shows how far rounding alone
moves each output.  Rounding points, in order:
  * the rotated q and k (RoPE writes bf16);
  * forward: P = exp(S - max) rounded before the P V product, and the row sum
    taken over the rounded P; O stored as bf16;
  * backward: D_i = sum_d dO_id O_id from that bf16 O; dS = P (dP - D_i)
    rounded before the dS K product; dQ stored as bf16.
The mask is the eviction mask j <= i < e_j (KV-streams explainer, trainer
paragraph; paper page, Fig. 2A); the gradients follow the softmax calculus.
"""
import math

import numpy as np
import torch


def bf16_round(x):
    """Round to the nearest bf16 (ties to even), returned as float64."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def dq_rows(q, k, v, e, do, b, h, rows, scale=None, rounding=True, pos=None):
    """dQ of rows ``rows`` of query head ``h`` of trace ``b`` as the kernels
    round it.  q, k: rotated (fp64 or bf16 values); v, do: bf16 values.
    ``rounding=False`` skips every rounding point (plain fp64 dQ).  With
    ``pos`` (the rows' logical positions) the gradient is rotated back by
    -theta before its final rounding, as the RoPE-fused backward stores the
    gradient of the unrotated query."""
    rnd = bf16_round if rounding else (lambda x: np.asarray(x, dtype=np.float64))
    Hq, Hkv, D = q.shape[2], k.shape[2], q.shape[3]
    kv = h // (Hq // Hkv)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    n = int(rows.max()) + 1
    qq = rnd(q[b, rows, h])
    kk = rnd(k[b, :n, kv])
    vv = np.asarray(v[b, :n, kv], dtype=np.float64)
    dd = np.asarray(do[b, rows, h], dtype=np.float64)
    j = np.arange(n)[None, :]
    ej = np.asarray(e[b], dtype=np.int64)[None, :n]
    live = (j <= rows[:, None]) & (rows[:, None] < ej)
    S = np.where(live, (qq @ kk.T) * sc, -np.inf)
    empty = ~live.any(axis=1, keepdims=True)
    m = np.where(empty, 0.0, S.max(axis=1, keepdims=True))
    Pu = np.exp(S - m)
    Pb = rnd(Pu)
    lb = np.where(empty, 1.0, Pb.sum(axis=1, keepdims=True))
    o = rnd((Pb @ vv) / lb)
    with np.errstate(divide="ignore"):
        lse = m + np.log(np.where(empty, 1.0, Pu.sum(axis=1, keepdims=True)))
    P = np.where(empty, 0.0, np.exp(S - lse))
    dP = dd @ vv.T
    Di = (dd * o).sum(axis=1, keepdims=True)
    dS = rnd(P * (dP - Di))
    g = sc * (dS @ kk)
    if pos is not None:
        g = unrotate_rows(g, pos)
    return rnd(g)


def unrotate_rows(x, pos, base=10000.0):
    """Rotate rows x [n, D] by -theta at positions pos [n] (rotate-half
    pairing, fp64): the backward of RoPE for gradient rows."""
    import oracle as O

    x = np.asarray(x, dtype=np.float64)
    return O.rope(x[None, :, None, :], np.asarray(pos)[None], base, inverse=True)[0, :, 0]
