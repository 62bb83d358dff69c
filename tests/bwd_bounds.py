"""Per-element error bars for the backward's parity tests (host side).

The GPU backward rounds the softmax weights P and the score gradients dS to
bf16 (relative error at most 2^-9) before they enter the dV, dK and dQ
products, and accumulates those products in fp32 from exact bf16 inputs.
Each gradient element is a sum of terms P_ti dO_t,e (dV), scale dS_ti q_t,e
(dK) or scale dS_ti k_i,e (dQ), so its error is at most 2^-9 of the sum of
the terms' magnitudes, plus the fp32 accumulation (about 2^-24 per term of
that same sum).  dS_ti = P_ti (dO_t . v_i - dO_t . o_t) itself comes from
two d-term fp32 dot products, off by at most d 2^-24 (< 2^-16 for d <= 128)
of P_ti (|dO_t| . |v_i| + |dO_t| . |o_t|), which matters where the two
nearly cancel (r = 1 makes dS exactly 0).  bars() returns 2^-8 of the
magnitude sums (twice the rounding bound), 2^-16 of the dot products'
magnitudes carried through the dQ and dK products, and a 1e-6 floor; the
magnitudes come from fp64 P and dS over the key sets oracle.key_set
enumerates.
"""
import numpy as np

import oracle


def masks(L, s, r):
    m = np.zeros((L, L), dtype=bool)
    for t in range(L):
        m[t, oracle.key_set(t, s, r)] = True
    return m


def bars(q, k, v, o, do, s, r, scale=None):
    """(bar_dq, bar_dk, bar_dv), shaped like q, k, v."""
    q, k, v, o, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, o, do))
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    m = masks(L, s, r)
    bq = np.zeros_like(q)
    bk = np.zeros_like(k)
    bv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            S = np.where(m, scale * (q[b, h] @ k[b, kv].T), -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dP = do[b, h] @ v[b, kv].T
            D = (do[b, h] * o[b, h]).sum(axis=1, keepdims=True)
            dS = np.abs(P * (dP - D))
            # magnitude of the fp32 dot products behind dP - D
            E = P * (np.abs(do[b, h]) @ np.abs(v[b, kv]).T + (np.abs(do[b, h]) * np.abs(o[b, h])).sum(axis=1, keepdims=True))
            W = 2.0 ** -8 * dS + 2.0 ** -16 * E
            bq[b, h] = scale * (W @ np.abs(k[b, kv]))
            bk[b, kv] += scale * (W.T @ np.abs(q[b, h]))
            bv[b, kv] += 2.0 ** -8 * (P.T @ np.abs(do[b, h]))
    return bq + 1e-6, bk + 1e-6, bv + 1e-6


def check(name, got, ref, bar):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{name}: non-finite"
    err = np.abs(got - ref)
    worst = float((err / bar).max()) if err.size else 0.0
    assert worst <= 1.0, f"{name}: max error {float(err.max())}, {worst:.2f}x its bar"
    return worst
