"""CPU checks of the rounding model the dQ-row gates use (tests/rounding_model.py):
without its rounding points it is the oracle's dQ, and with them it stays at
the bf16 floor on rows with many live keys."""
import numpy as np

import oracle as O
import rounding_model as RM
from parity_util import errors
from workloads import build_trace, normal_tensor


def _case(seed=3, N=700):
    tr = build_trace(np.random.default_rng(seed), N, 64, 320, "recent", turn_len=(64, 128))
    e = tr.e[None].astype(np.int64)
    x = [normal_tensor(s, seed * 10 + i, 0.5).numpy().astype(np.float64)
         for i, s in enumerate(((1, N, 4, 128), (1, N, 2, 128), (1, N, 2, 128), (1, N, 4, 128)))]
    return e, x


def test_without_rounding_equals_oracle():
    e, (q, k, v, do) = _case()
    rows = np.array([0, 1, 2, 63, 64, 300, 511, 699])
    for h in range(4):
        ref = O.attn_bwd_rows(q, k, v, e, do, 0, h, rows)
        got = RM.dq_rows(q, k, v, e, do, 0, h, rows, rounding=False)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-13)


def test_rounding_stays_at_the_bf16_floor_on_long_rows():
    e, (q, k, v, do) = _case(seed=4)
    rows = np.arange(200, 700, 7)          # every row sees 64+ keys
    for h in range(4):
        ref = O.attn_bwd_rows(q, k, v, e, do, 0, h, rows)
        got = RM.dq_rows(q, k, v, e, do, 0, h, rows)
        er = errors(got, ref, "bf16grad")
        assert er["rel_l2"] <= 6e-3 and er["rel_max"] <= 1.5e-2, er
