"""The backward's parity bars (tests/bwd_bounds.py) are tight enough to
catch plausible mistakes: gradients with one planted in them (computed by
the oracle on changed inputs, on the CPU) fail the bar against the correct
gradients, in at least one tensor."""
import numpy as np
import pytest

import oracle
import swa_inputs as si
from bwd_bounds import bars, check

CASE = (1, 4, 2, 64, 200, 4, 40)   # B, Hq, Hkv, d, L, s, r


def inputs():
    B, Hq, Hkv, d, L, s, r = CASE
    g = np.random.default_rng(11)
    mk = lambda H: si.round_bf16(g.standard_normal((B, H, L, d)).astype(np.float32))
    q, k, v, do = mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)
    o = si.round_bf16(oracle.prefill_rows(q, k, v, s, r).reshape(B, Hq, L, d).astype(np.float32))
    return q, k, v, o, do


def fails(got, ref, bar):
    try:
        check("x", got, ref, bar)
    except AssertionError:
        return True
    return False


def planted(kind, q, k, v, o, do):
    B, Hq, Hkv, d, L, s, r = CASE
    if kind == "window one longer":
        return oracle.backward(q, k, v, o, do, s, r + 1)
    if kind == "one sink fewer":
        return oracle.backward(q, k, v, o, do, s - 1, r)
    if kind == "query row 150 dropped":
        do2 = do.copy()
        do2[:, :, 150] = 0
        dq, dk, dv = oracle.backward(q, k, v, o, do2, s, r)
        dq[:, :, 150] = oracle.backward(q, k, v, o, do, s, r)[0][:, :, 150]
        return dq, dk, dv
    if kind == "D from the wrong row":
        return oracle.backward(q, k, v, np.roll(o, 1, axis=2), do, s, r)
    if kind == "dq 1% off":
        dq, dk, dv = oracle.backward(q, k, v, o, do, s, r)
        return dq * 1.01, dk, dv
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["window one longer", "one sink fewer", "query row 150 dropped",
                                  "D from the wrong row", "dq 1% off"])
def test_bars_catch_planted_mistakes(kind):
    q, k, v, o, do = inputs()
    B, Hq, Hkv, d, L, s, r = CASE
    refs = oracle.backward(q, k, v, o, do, s, r)
    bs = bars(q, k, v, o, do, s, r)
    got = planted(kind, q, k, v, o, do)
    assert any(fails(gt, ref, bar) for gt, ref, bar in zip(got, refs, bs)), kind
    # and the correct gradients pass their own bars
    assert not any(fails(ref, ref, bar) for ref, bar in zip(refs, bs))
