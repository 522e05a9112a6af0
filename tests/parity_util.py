"""Shared helpers of the GPU parity tests (comparison gates, conversions)."""
import sys

import numpy as np
import torch

# tolerances of the parity contract: max abs error <= 2e-2 for bf16 outputs
# (fp32 accumulation), <= 1e-5 for the fp32 path.  Because bf16 outputs of the
# N(0,1)*0.5 workloads are only ~1e-3..1e-1 in magnitude, the bf16 gate also
# bounds the error relative to the output's scale (max and L2).
#
# Gradients ("bf16grad") get a looser normalised-max bound.  The backward
# uses D_i = rowsum(dO o O) with O the bf16 output of the forward, so each
# row carries an error of about 2^-9 |dO| |O| in D_i.  On a row whose dQ is
# small against its inputs (e.g. a row that sees two keys whose values nearly
# cancel along dO) this is a few percent of that row's dQ, although the
# absolute error stays ~1e-3.  Rows with many live keys sit at the bf16
# rounding floor (~0.25% relative), which the L2 bound still enforces.
ATOL = {"bf16": 2e-2, "bf16grad": 2e-2, "f32": 1e-5}
REL_MAX = {"bf16": 1.5e-2, "bf16grad": 5e-2, "f32": 1e-5}
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
