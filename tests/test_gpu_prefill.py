"""Prefill on the GPU (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import swa_inputs as si
from gpu_common import TOL, all_rows, bits, dev, host, max_err, rows_of, say

pytestmark = pytest.mark.gpu


def run_prefill(q, k, v, s, r, dtype, **kw):
    import sliding_window_attention_sink_amd as swa
    o = swa.prefill(dev(q, dtype), dev(k, dtype), dev(v, dtype), s, r, **kw)
    torch.cuda.synchronize()
    return o


def case_inputs(case_id, B, Hq, Hkv, L, d, dtype, scale=1.0):
    wid = 1000 + case_id
    q = si.draw(wid, si.TENSOR_Q, B, Hq, L, d, scale=scale, dtype=dtype)
    k = si.draw(wid, si.TENSOR_K, B, Hkv, L, d, scale=scale, dtype=dtype)
    v = si.draw(wid, si.TENSOR_V, B, Hkv, L, d, scale=scale, dtype=dtype)
    return q, k, v


# (case, dtype, B, Hq, Hkv, d, L, s, r): several tiles, ragged tails, GQA,
# sinks beyond one tile, the r = 1 and r >= L limits, L < s.
CASES = [
    (1, "f32", 2, 4, 2, 64, 333, 4, 28),
    (2, "f32", 1, 2, 2, 128, 200, 0, 1),
    (3, "f32", 1, 2, 1, 128, 300, 70, 40),
    (4, "f32", 1, 1, 1, 64, 100, 0, 500),
    (5, "f32", 1, 3, 3, 64, 5, 4, 2),
    (6, "bf16", 1, 4, 2, 128, 1000, 4, 300),
    (7, "bf16", 2, 2, 2, 64, 700, 4, 100),
    (8, "bf16", 1, 4, 4, 128, 600, 0, 4096),
    (9, "bf16", 1, 2, 2, 128, 300, 0, 1),
    (10, "bf16", 1, 2, 2, 128, 520, 70, 130),
    (11, "bf16", 1, 2, 2, 128, 7, 4, 2),
    (12, "bf16", 1, 8, 1, 128, 389, 1, 64),
    (13, "bf16", 1, 2, 2, 128, 1, 4, 28),
    # sinks packed into the masked head of the first band tile: with r = 100
    # every later query block masks 29 keys there (256-row and 128-row
    # blocks alike), so s = 4 and s = 29 pack and s = 30 keeps its own tile
    (14, "bf16", 1, 2, 2, 128, 1500, 4, 100),
    (15, "bf16", 1, 4, 2, 128, 1100, 29, 100),
    (16, "bf16", 1, 4, 2, 128, 1100, 30, 100),
    (17, "bf16", 2, 2, 2, 64, 1300, 4, 100),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{c[0]}_{c[1]}_L{c[6]}_s{c[7]}_r{c[8]}" for c in CASES])
def test_prefill_matches_oracle(gpu, case):
    cid, dtype, B, Hq, Hkv, d, L, s, r = case
    q, k, v = case_inputs(cid, B, Hq, Hkv, L, d, dtype)
    say("prefill case", case)
    o = host(run_prefill(q, k, v, s, r, dtype))
    ref = oracle.prefill_rows(q, k, v, s, r).reshape(B, Hq, L, d)
    err = max_err(o, ref)
    assert err <= TOL[dtype], f"max-abs error {err}"
    if r == 1 and s == 0:
        # O_t = V_t: a single weight of 1.  bf16 output is exact; in fp32 the
        # folded scale (exp2 of an fma) leaves the weight within an ulp of 1.
        want = np.repeat(v, Hq // Hkv, axis=1).astype(np.float64)
        if dtype == "bf16":
            assert np.array_equal(o, want)
        else:
            assert max_err(o, want) <= 1e-6


def test_prefill_f32_l256_all_rows(gpu):
    w = si.WORKLOADS[1]
    q, k, v = si.prefill_inputs(w)
    say("fp32 prefill", w.name)
    o = host(run_prefill(q, k, v, w.s, w.r, w.dtype))
    ref = oracle.prefill_rows(q, k, v, w.s, w.r).reshape(o.shape)
    assert max_err(o, ref) <= TOL["f32"]


def sample_rows(B, H, L, n, seed, edge=130):
    g = np.random.default_rng(seed)
    rows = [np.stack([g.integers(0, B, n), g.integers(0, H, n), g.integers(0, L, n)], axis=1)]
    for b, h in [(0, 0), (B - 1, H - 1)]:
        ii = np.concatenate([np.arange(0, min(edge, L)), np.arange(max(0, L - edge), L)])
        rows.append(np.stack([np.full(ii.size, b), np.full(ii.size, h), ii], axis=1))
    return np.unique(np.concatenate(rows), axis=0)


@pytest.mark.parametrize("wid", [2, 3])
def test_full_workload_sampled_rows(gpu, wid):
    """Full-size bf16 prefills (GQA 32/8, L=8192, s=0, r=4096; and B=4, H=32,
    L=16384, s=4, r=1020), in the launch configuration the benchmark times,
    checked on sampled rows (every head touched at random rows, plus
    the first and last query tiles of two heads)."""
    w = si.WORKLOADS[wid]
    q, k, v = si.prefill_inputs(w)
    say("prefill", w.name)
    o_dev = run_prefill(q, k, v, w.s, w.r, w.dtype)
    rows = sample_rows(w.B, w.Hq, w.L, 3000, wid)
    got = host(o_dev[rows[:, 0], rows[:, 1], rows[:, 2]])
    ref = oracle.prefill_rows(q, k, v, w.s, w.r, rows=rows)
    err = max_err(got, ref)
    assert err <= TOL["bf16"], f"max-abs error {err}"


def test_uniform_probe_gives_window_mean(gpu):
    """Q = 0: every weight is equal, O_t = mean of V over U(t) (closed form)."""
    B, H, L, d, s, r = 1, 2, 777, 128, 4, 50
    _, k, v = case_inputs(40, B, H, H, L, d, "bf16")
    q = np.zeros_like(k)
    say("uniform probe")
    o = host(run_prefill(q, k, v, s, r, "bf16"))
    for t in range(L):
        idx = np.union1d(np.arange(min(s, t + 1)), np.arange(max(0, t - r + 1), t + 1))
        want = v[:, :, idx].astype(np.float64).mean(axis=2)
        assert np.abs(o[:, :, t] - want).max() <= 1e-2, t


def test_constant_values(gpu):
    B, H, L, d = 1, 2, 300, 128
    q, k, _ = case_inputs(41, B, H, H, L, d, "bf16", scale=3.0)
    v = np.full_like(k, 1.5)
    say("constant values")
    o = host(run_prefill(q, k, v, 4, 60, "bf16"))
    # the weights sum to one: O = 1.5 up to the bf16 rounding of P inside
    # P V (relative 2^-9) and of the output, i.e. within one bf16 ulp (2^-7)
    assert np.abs(o - 1.5).max() <= 2.0 ** -7


def test_large_sink_scores(gpu):
    """Sink scores near 100 (beyond fp32 exp's range without max subtraction)
    that dominate the softmax mass: tests the running-max numerics."""
    B, H, L, d, s, r = 1, 2, 640, 128, 4, 100
    g = np.random.default_rng(7)
    u = g.standard_normal(d)
    u /= np.linalg.norm(u)
    # q = N(0,1) + 3u and sink keys c*u: sink scores c*(3 + N(0,1))/sqrt(d), about 100
    q = si.round_bf16((g.standard_normal((B, H, L, d)) + 3.0 * u).astype(np.float32))
    k = si.round_bf16(g.standard_normal((B, H, L, d)).astype(np.float32))
    v = si.round_bf16(g.standard_normal((B, H, L, d)).astype(np.float32))
    k[:, :, :s] = si.round_bf16((u * (100.0 * np.sqrt(d) / 3.0)).astype(np.float32))
    say("large sink scores")
    o = host(run_prefill(q, k, v, s, r, "bf16"))
    ref = oracle.prefill_rows(q, k, v, s, r).reshape(o.shape)
    assert max_err(o, ref) <= TOL["bf16"]


def test_score_jump_mid_band(gpu):
    """Keys that score far above everything before them in the middle of the
    band (and a second, higher jump later): rows that meet them must raise
    the running max and rescale O after many tiles at the lower max; rows
    just past them must fall back to small weights."""
    B, Hq, Hkv, L, d, s, r = 1, 4, 2, 900, 128, 4, 400
    g = np.random.default_rng(11)
    u = g.standard_normal(d)
    u /= np.linalg.norm(u)
    q = si.round_bf16((g.standard_normal((B, Hq, L, d)) + 2.0 * u).astype(np.float32))
    k = si.round_bf16(g.standard_normal((B, Hkv, L, d)).astype(np.float32))
    v = si.round_bf16(g.standard_normal((B, Hkv, L, d)).astype(np.float32))
    # scores about 2*c/sqrt(d) * |u|^2: +30 for keys 500..505, +60 for 700..703
    k[:, :, 500:506] = si.round_bf16((u * (15.0 * np.sqrt(d))).astype(np.float32))
    k[:, :, 700:704] = si.round_bf16((u * (30.0 * np.sqrt(d))).astype(np.float32))
    say("score jump mid band")
    o = host(run_prefill(q, k, v, s, r, "bf16"))
    ref = oracle.prefill_rows(q, k, v, s, r).reshape(o.shape)
    assert max_err(o, ref) <= TOL["bf16"]


# (case, dtype, B, Hq, Hkv, d, L, s, r, dilation): residue classes of unequal
# length, sinks past the first tile, dilation beyond the window and beyond L
DILATED = [
    (60, "bf16", 1, 4, 2, 128, 700, 4, 60, 3),
    (61, "bf16", 2, 2, 2, 64, 333, 0, 40, 2),
    (62, "bf16", 1, 2, 1, 128, 500, 70, 20, 7),
    (63, "f32", 1, 2, 2, 64, 257, 4, 28, 4),
    (64, "bf16", 1, 2, 2, 128, 90, 4, 8, 100),
    (66, "bf16", 2, 8, 2, 128, 3, 4, 16, 2),        # L < s: every row a sink row
    (67, "bf16", 1, 4, 4, 64, 5, 4, 16, 3),         # L = s + 1: one class row
    (68, "f32", 1, 4, 2, 128, 611, 2, 33, 5),
    (69, "bf16", 1, 4, 2, 128, 1500, 1, 64, 2),     # several query tiles per class, ragged tail
]


@pytest.mark.parametrize("case", DILATED, ids=[f"dil{c[0]}_{c[1]}_L{c[6]}_d{c[9]}" for c in DILATED])
def test_dilated_prefill_matches_oracle(gpu, case):
    import sliding_window_attention_sink_amd as swa
    cid, dtype, B, Hq, Hkv, d, L, s, r, dil = case
    q, k, v = case_inputs(cid, B, Hq, Hkv, L, d, dtype)
    say("dilated prefill", case)
    o = swa.prefill_dilated(dev(q, dtype), dev(k, dtype), dev(v, dtype), s, r, dil)
    torch.cuda.synchronize()
    ref = oracle.prefill_rows(q, k, v, s, r, dilation=dil).reshape(B, Hq, L, d)
    assert max_err(host(o), ref) <= TOL[dtype]


def test_dilated_main_workload_sampled_rows(gpu):
    """Dilation 4 on the main workload's tensors at full size (L = 8192,
    32/8 heads): sampled rows, plus the first and last rows of one head."""
    import sliding_window_attention_sink_amd as swa
    w = si.WORKLOADS[2]
    q, k, v = si.prefill_inputs(w)
    say("dilated main workload")
    o = host(swa.prefill_dilated(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), w.s, w.r, 4))
    rows = sample_rows(w.B, w.Hq, w.L, 200, 31)
    ref = oracle.prefill_rows(q, k, v, w.s, w.r, rows=rows, dilation=4)
    got = np.stack([o[b, h, t] for b, h, t in rows])
    assert max_err(got, ref) <= TOL["bf16"]


def test_dilated_4_plus_1020_sampled_rows(gpu):
    """Dilation 8 at the 4+1020 workload's full size (B = 4, H = 32,
    L = 16384): query tiles of 256 rows, classes of 2048 and 2047 rows
    after the 4 sinks, a reach of 8188 positions."""
    import sliding_window_attention_sink_amd as swa
    w = si.WORKLOADS[3]
    q, k, v = si.prefill_inputs(w)
    say("dilated 4+1020 workload")
    o = host(swa.prefill_dilated(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), w.s, w.r, 8))
    rows = sample_rows(w.B, w.Hq, w.L, 160, 37)
    ref = oracle.prefill_rows(q, k, v, w.s, w.r, rows=rows, dilation=8)
    got = np.stack([o[b, h, t] for b, h, t in rows])
    assert max_err(got, ref) <= TOL["bf16"]


def test_dilation_one_is_plain_prefill(gpu):
    import sliding_window_attention_sink_amd as swa
    q, k, v = case_inputs(65, 1, 4, 2, 400, 128, "bf16")
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    say("dilation 1")
    a = swa.prefill(qd, kd, vd, 4, 50)
    b = swa.prefill_dilated(qd, kd, vd, 4, 50, 1)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(b))


def test_deterministic_and_guarded(gpu):
    """Two runs are bit-identical; nothing is written outside the output."""
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, L, d = 1, 4, 2, 450, 128
    q, k, v = case_inputs(42, B, Hq, Hkv, L, d, "bf16")
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    n = B * Hq * L * d
    pad = 4096
    buf = torch.full((n + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[pad:pad + n].view(B, Hq, L, d)
    say("determinism / guard")
    swa.prefill(qd, kd, vd, 4, 100, out=out)
    first = out.clone()
    swa.prefill(qd, kd, vd, 4, 100, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(bits(first), bits(out))
    assert (buf[:pad] == 7.0).all() and (buf[pad + n:] == 7.0).all()


def test_stream_argument(gpu):
    """Work goes to the stream that is passed (here a side stream)."""
    import sliding_window_attention_sink_amd as swa
    q, k, v = case_inputs(43, 1, 2, 2, 256, 128, "bf16")
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    side = torch.cuda.Stream()
    say("side stream")
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o = swa.prefill(qd, kd, vd, 4, 60)
    side.synchronize()
    ref = oracle.prefill_rows(q, k, v, 4, 60).reshape(o.shape)
    assert max_err(host(o), ref) <= TOL["bf16"]


def test_dominant_sinks_at_the_4_plus_1020_length(gpu):
    """Sinks that take most of the softmax mass, at the StreamingLLM
    workload's length and heads (one sequence of B = 4, H = 32, L = 16384,
    4 + 1020): Q = N(0,1) + 3u and the four sink keys 30u for a unit vector
    u per head, so sink scores sit near 8 against window scores near 0.
    The realised sink mass (from fp64 scores on the sampled rows) is above
    one half, and the sampled rows match the oracle."""
    import sliding_window_attention_sink_amd as swa
    w = si.WORKLOADS[3]
    B, H, L, d, s, r = 1, w.Hq, w.L, w.d, w.s, w.r
    g = np.random.default_rng(31)
    u = g.standard_normal((B, H, 1, d))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    q = si.round_bf16((g.standard_normal((B, H, L, d)) + 3.0 * u).astype(np.float32))
    k = si.round_bf16(g.standard_normal((B, H, L, d)).astype(np.float32))
    k[:, :, :s] = si.round_bf16(np.broadcast_to(30.0 * u, (B, H, s, d)).astype(np.float32))
    v = si.round_bf16(g.standard_normal((B, H, L, d)).astype(np.float32))
    say("dominant sinks 16384")
    o = swa.prefill(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), s, r)
    torch.cuda.synchronize()
    rows = np.array([[0, h, t] for h in range(0, H, 3) for t in list(range(0, L, 997)) + [L - 1]])
    ref = oracle.prefill_rows(q, k, v, s, r, rows=rows)
    got = rows_of(host(o), rows)
    assert max_err(got, ref) <= TOL["bf16"]
    # realised sink mass over the sampled rows past the first window
    mass = []
    for _, h, t in rows:
        if t < s + r:
            continue
        keys = oracle.key_set(int(t), s, r)
        x = (k[0, h, keys].astype(np.float64) @ q[0, h, t].astype(np.float64)) / np.sqrt(d)
        p = np.exp(x - x.max())
        mass.append(p[:s].sum() / p.sum())
    print("realised sink mass: mean %.3f, min %.3f" % (np.mean(mass), np.min(mass)))
    assert np.mean(mass) > 0.5
