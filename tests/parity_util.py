"""Shared helpers of the GPU parity tests (comparison gates, conversions)."""
import sys

import numpy as np
import torch

# tolerances of the parity contract: max abs error <= 2e-2 for bf16 outputs
# (fp32 accumulation), <= 1e-5 for the fp32 path.  Because bf16 outputs of the
# N(0,1)*0.5 workloads are only ~1e-3..1e-1 in magnitude, the bf16 gate also
# bounds the error relative to the output's scale (max and L2).
#
# Gradients ("bf16grad") use the same bounds.  One term of the kernels'
# rounding is amplified on rows that see few keys: D_i = rowsum(dO o O) is
# formed from the bf16 O of the forward, so D_i carries ~2^-9 sum|dO||O|,
# and dS = P (dP - D_i) moves by P times that.  On a row whose dQ nearly
# cancels (two live keys with close dP) this is a few percent of the row's
# dQ, and when that row holds the largest |dQ| of a sample the normalised
# maximum rises above the bf16 floor.  The dQ-row gates therefore compare
# the normalised maximum with that of a model of the kernels' rounding
# points (tests/rounding_model.py): it may exceed 1.5e-2 only as far as the
# model's own error does (gate_rows_model).
ATOL = {"bf16": 2e-2, "bf16grad": 2e-2, "f32": 1e-5}
REL_MAX = {"bf16": 1.5e-2, "bf16grad": 1.5e-2, "f32": 1e-5}
REL_L2 = {"bf16": 1e-2, "bf16grad": 1e-2, "f32": 1e-6}


def announce(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def f64(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()


# below this output scale the relative metrics are meaningless (an exactly
# zero reference, e.g. dQ of a row that sees a single key); the absolute
# bound still applies there
SCALE_FLOOR = {"bf16": 1e-4, "bf16grad": 1e-4, "f32": 1e-6}


def errors(actual, ref, kind="bf16"):
    a, r = f64(actual), f64(ref)
    d = np.abs(a - r)
    if not d.size:
        return {"max_abs": 0.0, "rel_max": 0.0, "rel_l2": 0.0, "finite": True}
    fl = SCALE_FLOOR[kind]
    return {
        "max_abs": float(d.max()),
        "rel_max": float(d.max() / max(np.abs(r).max(), fl)),
        "rel_l2": float(np.linalg.norm(a - r) / max(np.linalg.norm(r), fl * np.sqrt(r.size))),
        "finite": bool(np.isfinite(a).all()),
    }


def passes(actual, ref, kind):
    er = errors(actual, ref, kind)
    ok = (er["finite"] and er["max_abs"] <= ATOL[kind] and er["rel_max"] <= REL_MAX[kind]
          and er["rel_l2"] <= REL_L2[kind])
    return ok, er


def gate(actual, ref, kind, what=""):
    ok, er = passes(actual, ref, kind)
    print(f"[gate] {what}: " + " ".join(f"{k}={v:.3g}" for k, v in er.items()
                                        if k != "finite"), file=sys.stderr, flush=True)
    assert ok, f"{what}: {er}"
    return er


def gate_rows_model(actual, ref, model, what=""):
    """Gradient rows against the oracle when the rounding model shows the
    D_i amplification: the normalised bounds against the oracle rise to
    twice (max) and 1.5 times (L2) the model's own errors, capped at 5e-2
    and 2e-2; max-abs stays 2e-2; and the GPU must match the model of its
    own rounding within the plain bf16 bounds (normalised by the oracle's
    scale)."""
    er = errors(actual, ref, "bf16grad")
    em = errors(model, ref, "bf16grad")
    eg = errors(actual, model, "bf16grad")
    fl = SCALE_FLOOR["bf16grad"]
    r_scale = max(float(np.abs(f64(ref)).max()) if np.size(f64(ref)) else 0.0, fl)
    m_scale = max(float(np.abs(f64(model)).max()) if np.size(f64(model)) else 0.0, fl)
    gm = eg["rel_max"] * m_scale / r_scale          # GPU - model, over max |ref|
    lim_max = min(5e-2, max(REL_MAX["bf16grad"], 2.0 * em["rel_max"]))
    lim_l2 = min(2e-2, max(REL_L2["bf16grad"], 1.5 * em["rel_l2"]))
    ok = (er["finite"] and er["max_abs"] <= ATOL["bf16grad"] and er["rel_max"] <= lim_max
          and er["rel_l2"] <= lim_l2 and gm <= REL_MAX["bf16grad"])
    print(f"[gate] {what}: " + " ".join(f"{k}={v:.3g}" for k, v in er.items() if k != "finite")
          + f" | model rel_max={em['rel_max']:.3g} rel_l2={em['rel_l2']:.3g}"
          + f" | gpu-vs-model rel_max={gm:.3g}", file=sys.stderr, flush=True)
    assert ok, f"{what}: {er} (model {em}, gpu-model {gm}, limits {lim_max}, {lim_l2})"
    return er


def oracle_bwd_keys(q, k, v, e, do, keys, workers=8):
    """dK, dV of ``keys`` for one (trace, kv group) from the oracle: q and do
    hold the group's query heads [1, N, G, D], k and v its kv head
    [1, N, 1, D].  The oracle runs once per query head in parallel threads
    (numpy releases the interpreter lock in its kernels) and the per-head
    contributions are summed, as the group's gradients sum over its heads."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle as O
    from threadpoolctl import threadpool_limits

    G = q.shape[2]

    def one(h):
        return O.attn_bwd_keys(q[:, :, h:h + 1], k, v, e, do[:, :, h:h + 1], 0, 0, keys)

    with threadpool_limits(limits=2), ThreadPoolExecutor(min(workers, G)) as ex:
        parts = list(ex.map(one, range(G)))
    return sum(p[0] for p in parts), sum(p[1] for p in parts)
