"""Rolling-cache append and split-K decode on the GPU against the oracle's
token-by-token cache simulator (bit-exact slots) and its fp64 decode row."""
import numpy as np
import pytest
import torch

import oracle
import swa_inputs as si
from gpu_common import TOL, bits, dev, host, max_err, say

pytestmark = pytest.mark.gpu


def sim_bits(sim):
    """The simulator's cache as bf16 bit patterns; never-written slots NaN."""
    return si.bf16_bits(sim.k), si.bf16_bits(sim.v)


def assert_cache_equal(kc, vc, sim):
    kb, vb = sim_bits(sim)
    written = sim.pos >= 0
    gk, gv = bits(kc).astype(np.uint16), bits(vc).astype(np.uint16)
    assert np.array_equal(gk[:, :, written], kb[:, :, written])
    assert np.array_equal(gv[:, :, written], vb[:, :, written])
    # never-written slots keep the caller's poison (NaN)
    idle = torch.from_numpy(np.nonzero(~written)[0]).to(kc.device)
    assert torch.isnan(kc[:, :, idle].float()).all() and torch.isnan(vc[:, :, idle].float()).all()


@pytest.mark.parametrize("s,r,pos0,n", [
    (4, 60, 0, 3), (4, 60, 0, 64), (4, 60, 0, 200), (4, 60, 2, 5), (4, 60, 70, 1), (4, 60, 61, 130),
    (0, 32, 0, 100), (3, 5, 0, 17), (70, 30, 0, 75), (70, 30, 50, 40),
])
def test_append_bit_exact(gpu, s, r, pos0, n):
    import sliding_window_attention_sink_amd as swa
    B, Hkv, d = 2, 3, 128
    g = np.random.default_rng(s * 1000 + r * 10 + n)
    hist_k = si.round_bf16(g.standard_normal((B, Hkv, pos0 + n, d)).astype(np.float32))
    hist_v = si.round_bf16(g.standard_normal((B, Hkv, pos0 + n, d)).astype(np.float32))
    kc, vc = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan"))
    sim = oracle.RollingCacheSim(B, Hkv, d, s, r)
    say("append", s, r, pos0, n)
    if pos0:
        swa.cache_append(dev(hist_k[:, :, :pos0], "bf16"), dev(hist_v[:, :, :pos0], "bf16"), kc, vc, 0, s, r)
        sim.append(hist_k[:, :, :pos0], hist_v[:, :, :pos0], 0)
    swa.cache_append(dev(hist_k[:, :, pos0:], "bf16"), dev(hist_v[:, :, pos0:], "bf16"), kc, vc, pos0, s, r)
    sim.append(hist_k[:, :, pos0:], hist_v[:, :, pos0:], pos0)
    torch.cuda.synchronize()
    assert_cache_equal(kc, vc, sim)


@pytest.mark.parametrize("n,pos0,d,base", [
    (300, 0, 128, 1e4), (70, 4090, 64, 500.0), (33, 131000, 128, 1e4), (5, (1 << 29) + 12345, 128, 1e4),
])
def test_rope_keys_matches_oracle(gpu, n, pos0, d, base):
    """Keys rotated at their positions (pairs j, j + d/2, angle p * base^(-2j/d)):
    every element against the oracle's fp64 rotation of the same bf16 row,
    within one bf16 step; positions up to 2^29 (fp64 angles in turns)."""
    import sliding_window_attention_sink_amd as swa
    B, Hkv = 2, 3
    g = np.random.default_rng(n + d + pos0 % 1000)
    k = si.round_bf16(g.standard_normal((B, Hkv, n, d)).astype(np.float32))
    say("rope keys", n, pos0, d, base)
    got = host(swa.rope_keys(dev(k, "bf16"), pos0, base))
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(Hkv):
            for i in range(n):
                ref = oracle.rope(k[b, h, i], pos0 + i, base)
                assert np.all(np.abs(got[b, h, i] - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-5), (b, h, i)


@pytest.mark.parametrize("B,Hq,Hkv,d,s,r,n_split", [
    (2, 8, 2, 128, 4, 60, 0),
    (2, 8, 2, 128, 4, 60, 3),
    (1, 4, 4, 64, 4, 60, 2),
    (1, 16, 2, 128, 0, 96, 0),
    (1, 2, 1, 128, 70, 30, 1),
])
def test_decode_steps_match_oracle(gpu, B, Hq, Hkv, d, s, r, n_split):
    """Append one token, then decode with it, for T = 1 .. 2(s+r)+20: empty
    slots (poisoned with NaN), the filling cache and the wrapped buffer."""
    import sliding_window_attention_sink_amd as swa
    steps = 2 * (s + r) + 20
    g = np.random.default_rng(B * 100 + Hq + d + s + r)
    K = si.round_bf16(g.standard_normal((B, Hkv, steps, d)).astype(np.float32))
    V = si.round_bf16(g.standard_normal((B, Hkv, steps, d)).astype(np.float32))
    Q = si.round_bf16(g.standard_normal((B, Hq, steps, d)).astype(np.float32))
    kc, vc = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan"))
    Kd, Vd, Qd = dev(K, "bf16"), dev(V, "bf16"), dev(Q, "bf16")
    outs = torch.empty((steps, B, Hq, d), dtype=torch.bfloat16, device="cuda")
    say("decode steps", B, Hq, Hkv, d, s, r, n_split)
    for t in range(steps):
        swa.cache_append(Kd[:, :, t:t + 1].contiguous(), Vd[:, :, t:t + 1].contiguous(), kc, vc, t, s, r)
        swa.decode(Qd[:, :, t].contiguous(), kc, vc, t + 1, s, r, n_split=n_split, out=outs[t])
    torch.cuda.synchronize()
    got = host(outs)
    rows = np.array([[b, h, t] for t in range(steps) for b in range(B) for h in range(Hq)])
    ref = oracle.prefill_rows(Q, K, V, s, r, rows=rows).reshape(steps, B, Hq, d)
    err = max_err(got, ref)
    assert err <= TOL["bf16"], f"max-abs error {err}"


@pytest.mark.parametrize("B,Hq,Hkv,d,s,r,n_split", [
    (2, 8, 2, 128, 4, 60, 0),
    (1, 4, 2, 64, 3, 40, 3),
    (1, 2, 1, 128, 70, 30, 1),
])
def test_decode_step_equals_append_then_decode(gpu, B, Hq, Hkv, d, s, r, n_split):
    """The fused step gives the bytes of cache_append + decode: outputs and
    caches bit-identical at every T (sink slots, filling, wrapped), and the
    outputs match the oracle."""
    import sliding_window_attention_sink_amd as swa
    steps = 2 * (s + r) + 10
    g = np.random.default_rng(B * 1000 + Hq + d + s + r)
    K = si.round_bf16(g.standard_normal((B, Hkv, steps, d)).astype(np.float32))
    V = si.round_bf16(g.standard_normal((B, Hkv, steps, d)).astype(np.float32))
    Q = si.round_bf16(g.standard_normal((B, Hq, steps, d)).astype(np.float32))
    kc1, vc1 = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan"))
    kc2, vc2 = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan"))
    Kd, Vd, Qd = dev(K, "bf16"), dev(V, "bf16"), dev(Q, "bf16")
    o1 = torch.empty((steps, B, Hq, d), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty_like(o1)
    say("decode step fused", B, Hq, Hkv, d, s, r, n_split)
    for t in range(steps):
        kt, vt, qt = Kd[:, :, t].contiguous(), Vd[:, :, t].contiguous(), Qd[:, :, t].contiguous()
        swa.cache_append(kt.unsqueeze(2), vt.unsqueeze(2), kc1, vc1, t, s, r)
        swa.decode(qt, kc1, vc1, t + 1, s, r, n_split=n_split, out=o1[t])
        swa.decode_step(qt, kt, vt, kc2, vc2, t + 1, s, r, n_split=n_split, out=o2[t])
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2))
    assert np.array_equal(bits(kc1), bits(kc2)) and np.array_equal(bits(vc1), bits(vc2))
    rows = np.array([[b, h, t] for t in range(steps) for b in range(B) for h in range(Hq)])
    ref = oracle.prefill_rows(Q, K, V, s, r, rows=rows).reshape(steps, B, Hq, d)
    assert max_err(host(o2), ref) <= TOL["bf16"]


@pytest.mark.parametrize("B,Hq,Hkv,d,s,r,n_split,base", [
    (1, 8, 2, 128, 4, 60, 0, 1e4),
    (2, 4, 4, 64, 3, 45, 3, 500.0),
    (1, 2, 1, 128, 70, 30, 1, 1e4),
])
def test_decode_rope_matches_oracle(gpu, B, Hq, Hkv, d, s, r, n_split, base):
    """RoPE re-positioning (the streaming generation step; keys stored
    rotated at their positions): T = 1 .. 2(s+r)+20 through sink, filling and wrapped
    slots, fused and unfused steps, against the fp64 row definition."""
    import sliding_window_attention_sink_amd as swa
    steps = 2 * (s + r) + 20
    g = np.random.default_rng(B * 77 + Hq + d + s + r)
    K = si.round_bf16(g.standard_normal((B, Hkv, steps, d)).astype(np.float32))
    V = si.round_bf16(g.standard_normal((B, Hkv, steps, d)).astype(np.float32))
    Q = si.round_bf16(g.standard_normal((B, Hq, steps, d)).astype(np.float32))
    kc1, vc1 = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan"))
    kc2, vc2 = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan"))
    Kd, Vd, Qd = dev(K, "bf16"), dev(V, "bf16"), dev(Q, "bf16")
    Kd = swa.rope_keys(Kd, 0, base)      # keys enter rotated at their positions
    o1 = torch.empty((steps, B, Hq, d), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty_like(o1)
    say("decode rope", B, Hq, Hkv, d, s, r, n_split, base)
    for t in range(steps):
        kt, vt, qt = Kd[:, :, t].contiguous(), Vd[:, :, t].contiguous(), Qd[:, :, t].contiguous()
        swa.cache_append(kt.unsqueeze(2), vt.unsqueeze(2), kc1, vc1, t, s, r)
        swa.decode(qt, kc1, vc1, t + 1, s, r, rope_base=base, n_split=n_split, out=o1[t])
        swa.decode_step(qt, kt, vt, kc2, vc2, t + 1, s, r, rope_base=base, n_split=n_split, out=o2[t])
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2))
    rows = np.array([[b, h, t] for t in range(steps) for b in range(B) for h in range(Hq)])
    ref = oracle.prefill_rows(Q, K, V, s, r, rope_base=base, rows=rows).reshape(steps, B, Hq, d)
    assert max_err(host(o1), ref) <= TOL["bf16"]


def test_decode_rope_equals_one_token_chunks(gpu):
    """Decode with RoPE is chunked prefill with chunk 1: the two kernels
    agree on every step of a run past the wrap."""
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, d, s, r, base = 1, 4, 2, 128, 4, 100, 1e4
    steps = 300
    g = np.random.default_rng(3)
    K = si.round_bf16(g.standard_normal((B, Hkv, steps, d)).astype(np.float32))
    V = si.round_bf16(g.standard_normal((B, Hkv, steps, d)).astype(np.float32))
    Q = si.round_bf16(g.standard_normal((B, Hq, steps, d)).astype(np.float32))
    kc, vc = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan"))
    Kd, Vd, Qd = dev(K, "bf16"), dev(V, "bf16"), dev(Q, "bf16")
    Kd = swa.rope_keys(Kd, 0, base)
    say("decode rope vs chunk 1")
    worst = 0.0
    for t in range(steps):
        kt, vt = Kd[:, :, t:t + 1].contiguous(), Vd[:, :, t:t + 1].contiguous()
        qt = Qd[:, :, t:t + 1].contiguous()
        op = swa.prefill(qt, kt, vt, s, r, rope_base=base, k_cache=kc if t else None, v_cache=vc if t else None,
                         pos0=t)
        swa.cache_append(kt, vt, kc, vc, t, s, r)
        od = swa.decode(qt[:, :, 0].contiguous(), kc, vc, t + 1, s, r, rope_base=base)
        worst = max(worst, max_err(host(od), host(op[:, :, 0]).astype(np.float64)))
    assert worst <= TOL["bf16"], worst


def test_decode_split_counts_agree(gpu):
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, d, s, r, T = 2, 8, 2, 128, 4, 1020, 3000
    g = np.random.default_rng(5)
    K = si.round_bf16(g.standard_normal((B, Hkv, T, d)).astype(np.float32))
    V = si.round_bf16(g.standard_normal((B, Hkv, T, d)).astype(np.float32))
    q = si.round_bf16(g.standard_normal((B, Hq, d)).astype(np.float32))
    kc, vc = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan"))
    say("decode split counts")
    swa.cache_append(dev(K, "bf16"), dev(V, "bf16"), kc, vc, 0, s, r)
    qd = dev(q, "bf16")
    sim = oracle.RollingCacheSim(B, Hkv, d, s, r)
    sim.append(K, V, 0)
    ref = np.stack([[oracle.decode_row(sim, q[b, h], b, h, Hq) for h in range(Hq)] for b in range(B)])
    for ns in (1, 2, 4, 5, 16, 33, 64):
        o = host(swa.decode(qd, kc, vc, T, s, r, n_split=ns))
        assert max_err(o, ref) <= TOL["bf16"], ns


def test_decode_b64_gqa_full(gpu):
    """Decode at full size (B=64, GQA 32/8, d=128, s=4, r=4092): 8192-token pre-fill in one append call (most of
    it superseded), cache bit-exact; 1024 decode steps (even steps as
    cache_append + decode, odd steps as the fused decode_step, the bench's
    launch), sampled steps of both kinds checked against the oracle, and the
    final cache bit-exact."""
    import sliding_window_attention_sink_amd as swa
    w = si.WORKLOADS[4]
    hk, hv = si.decode_history(w)
    say("decode full size: pre-fill", w.name)
    kc, vc = swa.new_cache(w.B, w.Hkv, w.d, w.s, w.r, torch.bfloat16, "cuda", fill=float("nan"))
    hkd, hvd = dev(hk, "bf16"), dev(hv, "bf16")
    swa.cache_append(hkd, hvd, kc, vc, 0, w.s, w.r)
    torch.cuda.synchronize()
    del hkd, hvd
    sim = oracle.RollingCacheSim(w.B, w.Hkv, w.d, w.s, w.r)
    sim.append(hk, hv, 0)
    assert_cache_equal(kc, vc, sim)
    del hk, hv

    qs, ks, vs = si.decode_steps(w)
    qd, kd, vd = dev(qs, "bf16"), dev(ks, "bf16"), dev(vs, "bf16")
    outs = torch.empty((w.steps, w.B, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    say("decode full size: steps", w.name)
    for i in range(w.steps):
        T = w.L + i + 1
        if i % 2 == 0:
            swa.cache_append(kd[i].unsqueeze(2), vd[i].unsqueeze(2), kc, vc, T - 1, w.s, w.r)
            swa.decode(qd[i], kc, vc, T, w.s, w.r, out=outs[i])
        else:
            swa.decode_step(qd[i], kd[i], vd[i], kc, vc, T, w.s, w.r, out=outs[i])
    torch.cuda.synchronize()
    check = {0: 64, 1: 64, 510: 64, 511: 64, 1023: None}
    g = np.random.default_rng(4)
    for i in range(w.steps):
        sim.append(ks[i][:, :, None], vs[i][:, :, None], w.L + i)
        if i in check:
            n = check[i]
            pairs = [(b, h) for b in range(w.B) for h in range(w.Hq)]
            if n is not None:
                pairs = [pairs[j] for j in g.choice(len(pairs), n, replace=False)]
            got = host(outs[i])
            ref = np.stack([oracle.decode_row(sim, qs[i, b, h], b, h, w.Hq) for b, h in pairs])
            err = max_err(np.stack([got[b, h] for b, h in pairs]), ref)
            assert err <= TOL["bf16"], (i, err)
    assert_cache_equal(kc, vc, sim)


def test_decode_rope_full_size_sampled(gpu):
    """The RoPE-re-positioning generation step at the bench's size (B=64,
    GQA 32/8, d=128, s=4, r=4092, 8192-token history): 8 fused steps on the
    RoPE cache, every head of two sequences checked against the fp64
    row definition (keys of U(t) at cache positions 0..|U(t)|-1)."""
    import sliding_window_attention_sink_amd as swa
    w = si.WORKLOADS[4]
    base, nsteps, pick = 1e4, 8, [3, w.B - 1]
    hk, hv = si.decode_history(w)
    qs, ks, vs = si.decode_steps(w, steps=nsteps)
    say("decode rope full size: pre-fill", w.name)
    kc, vc = swa.new_cache(w.B, w.Hkv, w.d, w.s, w.r, torch.bfloat16, "cuda", fill=float("nan"))
    hkd, hvd = dev(hk, "bf16"), dev(hv, "bf16")
    swa.cache_append(swa.rope_keys(hkd, 0, base), hvd, kc, vc, 0, w.s, w.r)
    torch.cuda.synchronize()
    del hkd, hvd
    qd, kd, vd = dev(qs, "bf16"), dev(ks, "bf16"), dev(vs, "bf16")
    # step i's key rotated at its position L + i
    kd = torch.stack([swa.rope_keys(kd[i].unsqueeze(2), w.L + i, base)[:, :, 0] for i in range(nsteps)])
    outs = torch.empty((nsteps, w.B, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    say("decode rope full size: steps", w.name)
    for i in range(nsteps):
        swa.decode_step(qd[i], kd[i], vd[i], kc, vc, w.L + i + 1, w.s, w.r, rope_base=base, out=outs[i])
    torch.cuda.synchronize()
    got = host(outs)[:, pick]                                   # [steps, 2, Hq, d]
    # the two sequences' full token streams, for the oracle's row definition
    T = w.L + nsteps
    K = np.concatenate([hk[pick], ks[:, pick].transpose(1, 2, 0, 3)], axis=2)
    V = np.concatenate([hv[pick], vs[:, pick].transpose(1, 2, 0, 3)], axis=2)
    Q = np.zeros((len(pick), w.Hq, T, w.d), dtype=np.float32)
    Q[:, :, w.L:] = qs[:, pick].transpose(1, 2, 0, 3)
    rows = np.array([[b, h, w.L + i] for i in range(nsteps) for b in range(len(pick)) for h in range(w.Hq)])
    ref = oracle.prefill_rows(Q, K, V, w.s, w.r, rope_base=base, rows=rows).reshape(nsteps, len(pick), w.Hq, w.d)
    assert max_err(got, ref) <= TOL["bf16"]


def test_decode_full_attention_32k_sampled(gpu):
    """Full attention over a 32768-token context on the decode workload's
    shape (B = 64, GQA 32/8, d = 128): a cache of 4 + 32764 slots, every slot
    valid, the size the bench's cache-size sweep times; every head of three
    sequences against the fp64 decode row over all slots."""
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, d, s, r = 64, 32, 8, 128, 4, 32764
    S = s + r
    g = torch.Generator(device="cuda").manual_seed(21)
    kc = torch.randn((B, Hkv, S, d), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((B, Hkv, S, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    say("decode 32k full attention")
    o = swa.decode(q, kc, vc, S + 100, s, r)
    torch.cuda.synchronize()
    G = Hq // Hkv
    for b in (0, 31, B - 1):
        kh, vh, qh = host(kc[b]), host(vc[b]), host(q[b])
        got = host(o[b])
        for h in range(Hq):
            ref = oracle.attend_set(qh[h], kh[h // G], vh[h // G])
            assert max_err(got[h], ref) <= TOL["bf16"], (b, h)
