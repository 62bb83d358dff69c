"""Pins of the oracle's task-bound global tokens (causal form: a row in G
attends every key up to itself; any other row attends U(t) and the global
positions up to itself, each key once), against facts that do not go
through the oracle's key-set code: Python set constructions, closed-form
counts, dense causal attention by brute force, and the plain window where
the globals add nothing."""
import numpy as np
import pytest

import oracle


def brute_set(t, s, r, G):
    if t in set(G):
        return list(range(t + 1))
    u = {i for i in range(t + 1) if i < s or i >= t - r + 1}
    u |= {g for g in G if g <= t}
    return sorted(u)


@pytest.mark.parametrize("seed", range(6))
def test_key_sets_match_a_set_construction(seed):
    g = np.random.default_rng(seed)
    for _ in range(60):
        s, r, L = int(g.integers(0, 9)), int(g.integers(1, 30)), int(g.integers(1, 120))
        G = sorted(set(int(x) for x in g.integers(0, L, int(g.integers(0, 8)))))
        for t in range(L):
            got = list(oracle.key_set(t, s, r, globals_=G))
            assert got == brute_set(t, s, r, G), (t, s, r, G)


def test_key_set_sizes_closed_form():
    s, r, G = 4, 10, [2, 7, 20, 33, 50]
    for t in range(80):
        n = len(oracle.key_set(t, s, r, globals_=G))
        if t in G:
            assert n == t + 1
        else:
            extra = sum(1 for x in G if s <= x < max(s, t - r + 1) and x <= t)
            assert n == min(t + 1, s + r) + extra


def test_no_globals_is_the_plain_window():
    g = np.random.default_rng(1)
    B, Hq, Hkv, L, d, s, r = 1, 2, 1, 70, 16, 3, 9
    q, k, v = (g.standard_normal((B, H, L, d)).astype(np.float32) for H in (Hq, Hkv, Hkv))
    a = oracle.prefill_rows(q, k, v, s, r)
    b = oracle.prefill_rows(q, k, v, s, r, globals_=[])
    assert np.array_equal(a, b)


def dense_causal(q, k, v, scale):
    """Softmax attention over keys 0..t for every row, by a full matrix."""
    L = q.shape[0]
    S = (q.astype(np.float64) @ k.astype(np.float64).T) * scale
    S[np.triu(np.ones((L, L), dtype=bool), 1)] = -np.inf
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    return P @ v.astype(np.float64)


def test_every_position_global_is_dense_causal():
    g = np.random.default_rng(2)
    L, d, s, r = 50, 8, 2, 5
    q, k, v = (g.standard_normal((1, 1, L, d)).astype(np.float32) for _ in range(3))
    got = oracle.prefill_rows(q, k, v, s, r, globals_=list(range(L)))
    want = dense_causal(q[0, 0], k[0, 0], v[0, 0], 1 / np.sqrt(d))
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_global_rows_dense_and_other_rows_see_globals():
    g = np.random.default_rng(3)
    L, d, s, r = 90, 8, 3, 7
    G = [10, 40, 41, 77]
    q, k, v = (g.standard_normal((1, 1, L, d)).astype(np.float32) for _ in range(3))
    got = oracle.prefill_rows(q, k, v, s, r, globals_=G)
    dense = dense_causal(q[0, 0], k[0, 0], v[0, 0], 1 / np.sqrt(d))
    for t in range(L):
        if t in G:
            assert np.allclose(got[t], dense[t], rtol=0, atol=1e-12), t
        else:
            keys = brute_set(t, s, r, G)
            x = (k[0, 0, keys].astype(np.float64) @ q[0, 0, t].astype(np.float64)) / np.sqrt(d)
            w = np.exp(x - x.max())
            want = (w[:, None] * v[0, 0, keys].astype(np.float64)).sum(0) / w.sum()
            assert np.allclose(got[t], want, rtol=0, atol=1e-12), t


def test_globals_among_sinks_or_in_the_window_add_nothing():
    """A global position already in U(t) (a sink, or inside the window) is
    counted once: rows that are not global equal the plain rows."""
    g = np.random.default_rng(4)
    L, d, s, r = 60, 8, 4, 20
    G = [1, 3]                      # sinks
    q, k, v = (g.standard_normal((1, 1, L, d)).astype(np.float32) for _ in range(3))
    a = oracle.prefill_rows(q, k, v, s, r)
    b = oracle.prefill_rows(q, k, v, s, r, globals_=G)
    rows = [t for t in range(L) if t not in G]
    assert np.array_equal(a[rows], b[rows])
    # a global at 50 is inside the window of rows 50..59 (r = 20)
    c = oracle.prefill_rows(q, k, v, s, r, globals_=[50])
    assert np.array_equal(a[51:], c[51:])
    assert not np.allclose(a[50], c[50])     # row 50 itself is a global row


def test_bad_globals_rejected():
    q = np.zeros((1, 1, 8, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.prefill_rows(q, q, q, 1, 2, globals_=[3, 3])
    with pytest.raises(ValueError):
        oracle.prefill_rows(q, q, q, 1, 2, globals_=[5, 2])
    with pytest.raises(ValueError):
        oracle.prefill_rows(q, q, q, 1, 2, globals_=[1], dilation=2)
