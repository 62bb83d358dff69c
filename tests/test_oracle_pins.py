"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Each test ties one oracle function to something other than itself: a brute
force written in a different shape (dense matrix softmax, complex-number
rotation), a closed form, an invariant, or a number the pages print
(tests/golden/pages_facts.json).  The mistakes they are meant to catch: a
wrong window edge (off by one), sinks counted twice, a dropped sink, a wrong
scale, a wrong GQA head map, a transposed operand, a wrong slot rule, a wrong
RoPE pairing / sign / frequency, and positions taken from the sequence instead
of from the cache.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def rng(seed):
    return np.random.default_rng(np.random.SeedSequence([4321, seed]))


def dense_causal(q, k, v, scale):
    """Eq.(1) of the softmax-attention section (Blurry Window Attention page):
    softmax(Q K^T * scale + M) V with M the causal -inf mask, as a matrix."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    L = q.shape[0]
    S = q @ k.T * scale
    S[np.triu(np.ones((L, L), dtype=bool), 1)] = -np.inf
    S -= S.max(axis=1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(axis=1, keepdims=True)
    return P @ v


# --------------------------------------------------------------------------
# the softmax core against dense causal attention
# --------------------------------------------------------------------------
@pytest.mark.parametrize("B,Hq,Hkv,L,d,s,r", [
    (1, 1, 1, 17, 8, 0, 17),      # r = L: whole causal prefix
    (2, 4, 2, 23, 16, 0, 40),     # r > L, GQA 2 q-heads per kv-head
    (1, 6, 3, 31, 8, 5, 26),      # s + r = L: sinks and window cover every prefix
    (1, 2, 1, 12, 4, 12, 1),      # s = L: every key is a sink
])
def test_dense_limit_matches_brute_force(B, Hq, Hkv, L, d, s, r):
    g = rng(1)
    q = g.standard_normal((B, Hq, L, d)).astype(np.float32)
    k = g.standard_normal((B, Hkv, L, d)).astype(np.float32)
    v = g.standard_normal((B, Hkv, L, d)).astype(np.float32)
    scale = 1.0 / np.sqrt(d)
    got = oracle.prefill_rows(q, k, v, s, r).reshape(B, Hq, L, d)
    grp = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            want = dense_causal(q[b, h], k[b, h // grp], v[b, h // grp], scale)
            np.testing.assert_allclose(got[b, h], want, rtol=0, atol=1e-12)


def test_scale_is_applied():
    """Doubling the scale equals doubling q (scores are linear in both)."""
    g = rng(2)
    q = g.standard_normal((1, 1, 20, 8)).astype(np.float32)
    k = g.standard_normal((1, 1, 20, 8)).astype(np.float32)
    v = g.standard_normal((1, 1, 20, 8)).astype(np.float32)
    a = oracle.prefill_rows(q, k, v, 2, 5, scale=0.7)
    b = oracle.prefill_rows(2 * q, k, v, 2, 5, scale=0.35)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    c = oracle.prefill_rows(q, k, v, 2, 5, scale=0.35)
    assert np.abs(a - c).max() > 1e-3


# --------------------------------------------------------------------------
# window edge and key set
# --------------------------------------------------------------------------
def test_r1_s0_returns_own_value():
    """r = 1, s = 0: the only key is the query's own, so O_t = V_t exactly."""
    g = rng(3)
    q = g.standard_normal((2, 3, 40, 16)).astype(np.float32) * 5
    k = g.standard_normal((2, 3, 40, 16)).astype(np.float32) * 5
    v = g.standard_normal((2, 3, 40, 16)).astype(np.float32)
    out = oracle.prefill_rows(q, k, v, 0, 1).reshape(v.shape)
    assert np.array_equal(out, v.astype(np.float64))


@pytest.mark.parametrize("s,r", [(0, 1), (0, 5), (4, 1), (4, 28), (3, 3), (7, 2), (16, 64)])
def test_key_count_closed_form(s, r):
    for t in range(0, 3 * (s + r) + 5):
        ks = oracle.key_set(t, s, r)
        assert len(ks) == min(t + 1, s + r)
        # brute force over all earlier positions, straight from the set's definition
        want = [i for i in range(t + 1) if i < s or i >= t - r + 1]
        assert ks.tolist() == want


@pytest.mark.parametrize("s,r", [(0, 3), (4, 6), (2, 1), (5, 30)])
def test_uniform_probe_reveals_key_set(s, r):
    """Q = 0 makes every weight equal; with one-hot values V_i = e_i the output
    row is the indicator of the attended set divided by its size."""
    L = 40
    q = np.zeros((1, 1, L, L), dtype=np.float32)
    k = rng(4).standard_normal((1, 1, L, L)).astype(np.float32)
    v = np.eye(L, dtype=np.float32)[None, None]
    out = oracle.prefill_rows(q, k, v, s, r).reshape(L, L)
    for t in range(L):
        sinks = np.arange(min(s, t + 1))
        window = np.arange(max(0, t - r + 1), t + 1)
        members = np.union1d(sinks, window)
        assert len(members) == min(t + 1, s + r)
        want = np.zeros(L)
        want[members] = 1.0 / len(members)
        np.testing.assert_allclose(out[t], want, rtol=0, atol=1e-15)


def test_constant_values_give_constant_output():
    """Softmax weights sum to one (eq:attn-fixed-softmax-sink), so V = c gives
    O = c for any scores, including scores far beyond exp's fp64 range."""
    g = rng(5)
    L, d = 50, 8
    q = (g.standard_normal((1, 2, L, d)) * 60).astype(np.float32)
    k = (g.standard_normal((1, 2, L, d)) * 60).astype(np.float32)
    v = np.full((1, 2, L, d), 3.25, dtype=np.float32)
    out = oracle.prefill_rows(q, k, v, 4, 9)
    np.testing.assert_allclose(out, 3.25, rtol=0, atol=1e-12)


def test_gqa_head_map():
    """q-head h reads kv-head h // (Hq/Hkv): contiguous groups."""
    g = rng(6)
    L, d = 12, 8
    q = g.standard_normal((1, 4, L, d)).astype(np.float32)
    k = g.standard_normal((1, 2, L, d)).astype(np.float32)
    v = g.standard_normal((1, 2, L, d)).astype(np.float32)
    out = oracle.prefill_rows(q, k, v, 2, 4).reshape(1, 4, L, d)
    for h in range(4):
        single = oracle.prefill_rows(q[:, h:h + 1], k[:, h // 2:h // 2 + 1], v[:, h // 2:h // 2 + 1], 2, 4)
        np.testing.assert_array_equal(out[0, h], single.reshape(L, d))


def test_qpos0_offsets_rows():
    """Rows of a later chunk equal the same rows computed from position 0."""
    g = rng(7)
    L, d = 30, 8
    q = g.standard_normal((1, 1, L, d)).astype(np.float32)
    k = g.standard_normal((1, 1, L, d)).astype(np.float32)
    v = g.standard_normal((1, 1, L, d)).astype(np.float32)
    full = oracle.prefill_rows(q, k, v, 3, 7)
    part = oracle.prefill_rows(q[:, :, 18:], k, v, 3, 7, qpos0=18)
    np.testing.assert_array_equal(full[18:], part)


# --------------------------------------------------------------------------
# rolling-buffer cache and decode
# --------------------------------------------------------------------------
@pytest.mark.parametrize("s,r", [(0, 1), (0, 4), (3, 1), (3, 5), (4, 7), (1, 2)])
def test_cache_holds_exactly_the_key_set(s, r):
    """After tokens 0..T-1 the written slots hold exactly U(T-1), for every T."""
    d = 2
    sim = oracle.RollingCacheSim(1, 1, d, s, r)
    for T in range(1, 4 * (s + r) + 3):
        tok = np.full((1, 1, 1, d), T - 1, dtype=np.float32)
        sim.append(tok, tok, T - 1)
        held = sorted(sim.pos[sim.valid_slots()].tolist())
        assert held == oracle.key_set(T - 1, s, r).tolist()
        # every slot's content is the token it claims to hold
        for sl in sim.valid_slots():
            assert sim.k[0, 0, sl, 0] == sim.pos[sl]
        assert sim.k.shape[2] == s + r


def test_cache_slot_closed_form():
    """Slot j >= s holds p_j = (T-1) - (((T-1) - (j-s)) mod r) when p_j >= s;
    sink slot j is written iff j < T."""
    for s, r in [(0, 5), (4, 7), (2, 3), (5, 1)]:
        sim = oracle.RollingCacheSim(1, 1, 1, s, r)
        for T in range(1, 40):
            sim.append(np.zeros((1, 1, 1, 1), np.float32), np.zeros((1, 1, 1, 1), np.float32), T - 1)
            for j in range(s + r):
                if j < s:
                    want = j if j < T else -1
                else:
                    if (j - s) > T - 1:
                        want = -1
                    else:
                        p = (T - 1) - (((T - 1) - (j - s)) % r)
                        want = p if p >= s else -1
                assert sim.pos[j] == want, (s, r, T, j)


def test_bulk_append_equals_token_by_token():
    g = rng(8)
    s, r, d = 3, 5, 4
    toks_k = g.standard_normal((2, 2, 23, d)).astype(np.float32)
    toks_v = g.standard_normal((2, 2, 23, d)).astype(np.float32)
    a = oracle.RollingCacheSim(2, 2, d, s, r)
    a.append(toks_k, toks_v, 0)
    b = oracle.RollingCacheSim(2, 2, d, s, r)
    for p in range(23):
        b.append(toks_k[:, :, p:p + 1], toks_v[:, :, p:p + 1], p)
    np.testing.assert_array_equal(a.pos, b.pos)
    np.testing.assert_array_equal(np.nan_to_num(a.k, nan=7), np.nan_to_num(b.k, nan=7))


@pytest.mark.parametrize("s,r,T", [(4, 6, 3), (4, 6, 10), (4, 6, 11), (4, 6, 37), (0, 8, 50), (2, 1, 9)])
def test_decode_on_rolling_buffer_equals_last_prefill_row(s, r, T):
    g = rng(9)
    B, Hq, Hkv, d = 2, 4, 2, 16
    k = g.standard_normal((B, Hkv, T, d)).astype(np.float32)
    v = g.standard_normal((B, Hkv, T, d)).astype(np.float32)
    q = g.standard_normal((B, Hq, T, d)).astype(np.float32)
    sim = oracle.RollingCacheSim(B, Hkv, d, s, r)
    sim.append(k, v, 0)
    rows = np.array([[b, h, T - 1] for b in range(B) for h in range(Hq)])
    last = oracle.prefill_rows(q, k, v, s, r, rows=rows)
    for n, (b, h, _) in enumerate(rows):
        dec = oracle.decode_row(sim, q[b, h, T - 1], b, h, Hq)
        np.testing.assert_allclose(dec, last[n], rtol=0, atol=1e-13)


def test_decode_order_invariance():
    """Softmax attention over a set ignores the order of its members (the
    permutation-invariance remark of section 3 of the Blurry Window Attention
    page), which lets decode read slots in physical order."""
    g = rng(10)
    q = g.standard_normal(16).astype(np.float32)
    K = g.standard_normal((37, 16)).astype(np.float32)
    V = g.standard_normal((37, 16)).astype(np.float32)
    perm = g.permutation(37)
    np.testing.assert_allclose(oracle.attend_set(q, K, V), oracle.attend_set(q, K[perm], V[perm]),
                               rtol=0, atol=1e-14)


def test_pages_cache_facts():
    facts = json.load(open(GOLDEN))
    rb = facts["rolling_buffer_saving"]
    W = rb["window"]
    for case in rb["cases"]:
        T = case["seq_len"]
        sim = oracle.RollingCacheSim(1, 1, 1, 0, W)
        ones = np.ones((1, 1, T, 1), np.float32)
        # bulk append through the simulator's own slot rule
        sim.append(ones, ones, 0)
        assert len(sim.valid_slots()) == W
        assert T // len(sim.valid_slots()) == case["saving"]
    rf = facts["receptive_field"]
    assert rf["layers"] * rf["window"] == rf["tokens"]
    for case in facts["streaming_cache_budget"]["cases"]:
        s, r = case["sinks"], case["recent"]
        sim = oracle.RollingCacheSim(1, 1, 1, s, r)
        ones = np.ones((1, 1, 3000, 1), np.float32)
        sim.append(ones, ones, 0)
        assert len(sim.valid_slots()) == case["cache_slots"]
        assert len(oracle.key_set(2999, s, r)) == case["cache_slots"]
    sc = facts["sink_count_default"]
    for w in (8, 64, 1024):
        assert len(oracle.key_set(5000, sc["sinks"], w - 4)) == w


# --------------------------------------------------------------------------
# RoPE re-positioning
# --------------------------------------------------------------------------
def test_rope_closed_forms():
    # d = 2: theta_0 = 1, so position p turns (1, 0) to (cos p, sin p)
    for p in (0, 1, 7, 4095):
        np.testing.assert_allclose(oracle.rope([1.0, 0.0], p, 10000.0), [np.cos(p), np.sin(p)], atol=1e-15)
    # d = 4, base 1e4: theta_1 = 1e4^(-1/2) = 0.01; pairs are (0, 2) and (1, 3)
    e = np.eye(4)
    np.testing.assert_allclose(oracle.rope(e[1], 100, 1e4), [0, np.cos(1.0), 0, np.sin(1.0)], atol=1e-14)
    np.testing.assert_allclose(oracle.rope(e[0], 100, 1e4), [np.cos(100.0), 0, np.sin(100.0), 0], atol=1e-13)
    np.testing.assert_allclose(oracle.rope(e[3], 100, 1e4), [0, -np.sin(1.0), 0, np.cos(1.0)], atol=1e-14)


def test_rope_relative_and_norm():
    g = rng(11)
    d = 128
    q, k = g.standard_normal(d), g.standard_normal(d)
    for a, b, c in [(5, 2, 17), (4095, 0, 3), (100, 100, 1000)]:
        x = oracle.rope(q, a, 1e4) @ oracle.rope(k, b, 1e4)
        y = oracle.rope(q, a + c, 1e4) @ oracle.rope(k, b + c, 1e4)
        assert abs(x - y) < 1e-10
        assert abs(np.linalg.norm(oracle.rope(q, a, 1e4)) - np.linalg.norm(q)) < 1e-12


def rope_complex(x, pos, base):
    """Rotation as complex multiplication: z_j = x_j + i x_{j+d/2}, z_j e^{i pos theta_j}."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    theta = base ** (-np.arange(h) * 2.0 / d)
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * np.multiply.outer(pos, theta))
    return np.concatenate([z.real, z.imag], axis=-1)


def dense_rope_causal(q, k, v, scale, base):
    L = q.shape[0]
    pos = np.arange(L)
    return dense_causal(rope_complex(q, pos, base), rope_complex(k, pos, base), v, scale)


def test_rope_before_cache_fills_is_plain_rope():
    """While t < s + r the cache holds every earlier token, cache positions are
    true positions, and the result is plain RoPE causal attention."""
    g = rng(12)
    L, d, s, r, base = 24, 16, 4, 20, 500.0
    q = g.standard_normal((1, 1, L, d)).astype(np.float32)
    k = g.standard_normal((1, 1, L, d)).astype(np.float32)
    v = g.standard_normal((1, 1, L, d)).astype(np.float32)
    got = oracle.prefill_rows(q, k, v, s, r, rope_base=base).reshape(L, d)
    want = dense_rope_causal(q[0, 0], k[0, 0], v[0, 0], 1 / np.sqrt(d), base)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_rope_full_cache_is_rope_over_compacted_cache():
    """Once the cache is full, row t equals plain RoPE causal attention at the
    last row of the sequence made of the cache contents only (sinks followed
    by the recent window), i.e. positions 0 .. s+r-1 inside the cache."""
    g = rng(13)
    L, d, s, r, base = 60, 16, 3, 9, 300.0
    q = g.standard_normal((1, 1, L, d)).astype(np.float32)
    k = g.standard_normal((1, 1, L, d)).astype(np.float32)
    v = g.standard_normal((1, 1, L, d)).astype(np.float32)
    got = oracle.prefill_rows(q, k, v, s, r, rope_base=base).reshape(L, d)
    for t in range(s + r - 1, L):
        idx = np.concatenate([np.arange(s), np.arange(t - r + 1, t + 1)])
        want = dense_rope_causal(q[0, 0, idx], k[0, 0, idx], v[0, 0, idx], 1 / np.sqrt(d), base)[-1]
        np.testing.assert_allclose(got[t], want, rtol=0, atol=1e-12)


def test_rope_full_cache_ignores_absolute_position():
    """Two histories of different length with the same sinks and the same last
    r tokens give the same last row: positions come from the cache."""
    g = rng(14)
    d, s, r, base = 16, 4, 6, 1e4
    sink = g.standard_normal((s, d)).astype(np.float32)
    tail_q = g.standard_normal((r, d)).astype(np.float32)
    tail_k = g.standard_normal((r, d)).astype(np.float32)
    tail_v = g.standard_normal((r, d)).astype(np.float32)
    outs = []
    for mid in (0, 7, 31):
        m = g.standard_normal((3, mid, d)).astype(np.float32)
        qq = np.concatenate([g.standard_normal((s, d)).astype(np.float32), m[0], tail_q])
        kk = np.concatenate([sink, m[1], tail_k])
        vv = np.concatenate([g.standard_normal((s, d)).astype(np.float32), m[2], tail_v])
        # values of the sinks matter too: use the same ones in every history
        vv[:s] = tail_v[:1]
        L = qq.shape[0]
        rows = np.array([[0, 0, L - 1]])
        outs.append(oracle.prefill_rows(qq[None, None], kk[None, None], vv[None, None], s, r,
                                        rope_base=base, rows=rows)[0])
    np.testing.assert_allclose(outs[0], outs[1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(outs[0], outs[2], rtol=0, atol=1e-12)
    # rotating at true sequence positions instead would change the row
    L = qq.shape[0]
    idx = np.concatenate([np.arange(s), np.arange(L - r, L)])
    qt = rope_complex(qq[L - 1], L - 1, base)
    kt = rope_complex(kk[idx], idx, base)
    x = kt @ qt / np.sqrt(d)
    w = np.exp(x - x.max())
    true_pos = (w / w.sum()) @ vv[idx].astype(np.float64)
    assert np.abs(true_pos - outs[2]).max() > 1e-3


# ---- dilated window (glossary entry on dilated SWA and the Longformer
# section of the t6page page: attended positions skip delta-1 tokens; the
# count of window keys, r, is unchanged)

def _dilated_set(t, s, r, dil):
    """The definition, written as a set: sinks up to t, then r positions back
    from t in steps of dil, each key once."""
    return sorted({i for i in range(t + 1) if i < s} | {t - dil * m for m in range(r) if t - dil * m >= 0})


@pytest.mark.parametrize("s,r,dil", [(0, 1, 3), (0, 4, 2), (2, 3, 3), (4, 5, 4), (3, 2, 7), (1, 6, 1)])
def test_dilated_key_set_brute_force(s, r, dil):
    for t in range(0, 40):
        assert list(oracle.key_set(t, s, r, dil)) == _dilated_set(t, s, r, dil), (t, s, r, dil)


@pytest.mark.parametrize("s,r,dil", [(0, 4, 2), (4, 3, 5), (2, 10, 3)])
def test_dilated_key_count_closed_form(s, r, dil):
    # |U| = min(s, t+1) + (t >= s ? min(r, floor((t - s) / dil) + 1) : 0)
    for t in range(0, 60):
        win = min(r, (t - s) // dil + 1) if t >= s else 0
        assert len(oracle.key_set(t, s, r, dil)) == min(s, t + 1) + win


def test_dilated_rows_equal_attention_over_explicit_sets():
    """Rows with a dilation equal softmax attention over the key set written
    out by hand (attend_set: a separate routine of the oracle)."""
    g = np.random.default_rng(21)
    B, Hq, Hkv, L, d, s, r, dil = 1, 4, 2, 50, 16, 3, 5, 4
    q = g.standard_normal((B, Hq, L, d)).astype(np.float32)
    k = g.standard_normal((B, Hkv, L, d)).astype(np.float32)
    v = g.standard_normal((B, Hkv, L, d)).astype(np.float32)
    got = oracle.prefill_rows(q, k, v, s, r, dilation=dil).reshape(B, Hq, L, d)
    for h in range(Hq):
        kvh = h // (Hq // Hkv)
        for t in range(L):
            keys = _dilated_set(t, s, r, dil)
            want = oracle.attend_set(q[0, h, t], k[0, kvh, keys], v[0, kvh, keys])
            assert np.abs(got[0, h, t] - want).max() < 1e-12, (h, t)


def test_dilation_one_is_the_plain_window():
    g = np.random.default_rng(22)
    q = g.standard_normal((1, 2, 40, 8)).astype(np.float32)
    k = g.standard_normal((1, 2, 40, 8)).astype(np.float32)
    v = g.standard_normal((1, 2, 40, 8)).astype(np.float32)
    a = oracle.prefill_rows(q, k, v, 2, 7)
    b = oracle.prefill_rows(q, k, v, 2, 7, dilation=1)
    assert np.array_equal(a, b)
