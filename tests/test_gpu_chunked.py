"""Chunked streaming prefill over the rolling cache, with and without RoPE
re-positioning, against the oracle's row definition over the whole history."""
import numpy as np
import pytest
import torch

import oracle
import swa_inputs as si
from gpu_common import TOL, dev, guard_intact, guarded, host, max_err, say

pytestmark = pytest.mark.gpu


def run_chunked(q, k, v, s, r, chunk, rope_base, *, save_at=None):
    """Prefill chunk by chunk (attend over cache + chunk, then append the
    chunk), all on the current stream.  Returns O [B,Hq,L,d] on the device.
    With save_at, the cache is copied to host after that many tokens, freed
    and restored (checkpoint / resume)."""
    import sliding_window_attention_sink_amd as swa
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    if rope_base:
        kd = swa.rope_keys(kd, 0, rope_base)    # every key rotated once, at its position
    kc, vc = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan"))
    out = torch.empty_like(qd)
    for p0 in range(0, L, chunk):
        p1 = min(L, p0 + chunk)
        qc, kk, vv = (x[:, :, p0:p1].contiguous() for x in (qd, kd, vd))
        o = swa.prefill(qc, kk, vv, s, r, rope_base=rope_base,
                        k_cache=kc if p0 else None, v_cache=vc if p0 else None, pos0=p0)
        out[:, :, p0:p1] = o
        swa.cache_append(kk, vv, kc, vc, p0, s, r)
        if save_at is not None and p1 == save_at:
            torch.cuda.synchronize()
            saved = (kc.cpu(), vc.cpu())
            del kc, vc
            torch.cuda.empty_cache()
            kc, vc = saved[0].to("cuda"), saved[1].to("cuda")
    torch.cuda.synchronize()
    return out


def seq_inputs(seed, B, Hq, Hkv, L, d):
    g = np.random.default_rng(seed)
    mk = lambda H: si.round_bf16(g.standard_normal((B, H, L, d)).astype(np.float32))
    return mk(Hq), mk(Hkv), mk(Hkv)


@pytest.mark.parametrize("rope_base", [0.0, 10000.0, 500.0])
@pytest.mark.parametrize("chunk", [64, 100, 256])
def test_chunked_matches_oracle(gpu, rope_base, chunk):
    B, Hq, Hkv, L, d, s, r = 1, 4, 2, 600, 128, 4, 92
    q, k, v = seq_inputs(11, B, Hq, Hkv, L, d)
    say("chunked", chunk, rope_base)
    o = host(run_chunked(q, k, v, s, r, chunk, rope_base))
    ref = oracle.chunked_rows(q, k, v, s, r, rope_base=rope_base, rows=None).reshape(o.shape)
    err = max_err(o, ref)
    assert err <= TOL["bf16"], f"max-abs error {err}"


@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
@pytest.mark.parametrize("Hq,Hkv,chunk", [(4, 2, 500), (2, 2, 1000)])
def test_chunked_long_window_cache_tiles(gpu, rope_base, Hq, Hkv, chunk):
    """Bands with many cached key tiles: r = 700 slots (the wrap falls inside
    a 64-key tile), chunk starts not on tile boundaries, GQA pairs and MHA;
    the contiguous cache-tile loads and the straddling tile's per-row path."""
    B, L, d, s, r = 1, 3000, 128, 4, 700
    q, k, v = seq_inputs(12, B, Hq, Hkv, L, d)
    say("chunked long window", Hq, Hkv, chunk, rope_base)
    o = host(run_chunked(q, k, v, s, r, chunk, rope_base))
    ref = oracle.chunked_rows(q, k, v, s, r, rope_base=rope_base, rows=None).reshape(o.shape)
    err = max_err(o, ref)
    assert err <= TOL["bf16"], f"max-abs error {err}"


@pytest.mark.parametrize("s,r,d,Hq,Hkv,chunk", [
    (64, 40, 128, 4, 2, 96),     # one full sink tile, the largest s that turns; GQA pairs
    (65, 40, 128, 2, 2, 96),     # two sink tiles: the band re-reads its queries; MHA halves
    (1, 70, 64, 2, 2, 128),      # one sink, d = 64, MHA
    (4, 60, 64, 8, 2, 200),      # four q-heads per kv-head, d = 64, items straddling s+r-1
])
def test_rope_sink_turn_boundaries(gpu, s, r, d, Hq, Hkv, chunk):
    """RoPE with one sink tile and every row of a work item at or past s+r-1:
    the sink keys are turned by -(s+r-1) in LDS and scored with the query as
    read, the band takes the query rotated to t.  Around it: two sink tiles
    (s = 65), items whose rows straddle s+r-1 (both keep the second read of
    the queries), d = 64, GQA pairs and MHA halves."""
    B, L = 1, 700
    q, k, v = seq_inputs(14, B, Hq, Hkv, L, d)
    say("rope sink turn", s, r, d, Hq, Hkv, chunk)
    o = host(run_chunked(q, k, v, s, r, chunk, 10000.0))
    ref = oracle.chunked_rows(q, k, v, s, r, rope_base=10000.0, rows=None).reshape(o.shape)
    err = max_err(o, ref)
    assert err <= TOL["bf16"], f"max-abs error {err}"


def test_single_chunk_rope_equals_plain_rope_prefill(gpu):
    """One chunk holding the whole sequence: the RoPE path without a cache."""
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, L, d, s, r = 1, 2, 2, 500, 64, 4, 60
    q, k, v = seq_inputs(12, B, Hq, Hkv, L, d)
    say("single chunk rope d=64")
    o = swa.prefill(dev(q, "bf16"), swa.rope_keys(dev(k, "bf16"), 0, 10000.0), dev(v, "bf16"), s, r,
                    rope_base=10000.0)
    ref = oracle.prefill_rows(q, k, v, s, r, rope_base=10000.0).reshape(o.shape)
    assert max_err(host(o), ref) <= TOL["bf16"]


def test_chunk_size_independence_and_resume(gpu):
    """Chunking is only a schedule: chunk sizes 64 and 512 give the same rows,
    and saving/restoring the cache mid-stream changes nothing (bit-exact)."""
    B, Hq, Hkv, L, d, s, r = 1, 2, 2, 1024, 128, 4, 252
    q, k, v = seq_inputs(13, B, Hq, Hkv, L, d)
    say("chunk independence / resume")
    a = run_chunked(q, k, v, s, r, 64, 10000.0)
    b = run_chunked(q, k, v, s, r, 512, 10000.0)
    c = run_chunked(q, k, v, s, r, 64, 10000.0, save_at=448)
    assert torch.equal(a, c)
    assert max_err(host(a), host(b)) <= TOL["bf16"]


def run_chunked_fused(q, k, v, s, r, chunk, rope_base, *, first=None):
    """The chunked prefill with the append fused in: chunk i reads cache pair
    i % 2 and writes the cache after it to pair (i + 1) % 2.  first: a
    different size for the first chunk (any size is allowed at pos0 = 0).
    Returns O on the device and the last cache pair written."""
    import sliding_window_attention_sink_amd as swa
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    if rope_base:
        kd = swa.rope_keys(kd, 0, rope_base)
    caches = [swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan")) for _ in range(2)]
    out = torch.empty_like(qd)
    bounds = [0] + list(range(first if first else chunk, L, chunk)) + [L]
    for i, (p0, p1) in enumerate(zip(bounds[:-1], bounds[1:])):
        qc, kk, vv = (x[:, :, p0:p1].contiguous() for x in (qd, kd, vd))
        kc, vc = caches[i % 2]
        kx, vx = caches[(i + 1) % 2]
        out[:, :, p0:p1] = swa.prefill_append(qc, kk, vv, s, r, kx, vx, rope_base=rope_base,
                                              k_cache=kc if p0 else None, v_cache=vc if p0 else None, pos0=p0)
    torch.cuda.synchronize()
    return out, caches[(len(bounds) - 1) % 2]


def filled_slots(s, r, T):
    """Cache slots that hold a token after tokens 0 .. T-1 were appended."""
    sl = set(range(min(s, T)))
    sl |= {s + p % r for p in range(max(s, T - r), T)}
    return sorted(sl)


@pytest.mark.parametrize("B,Hq,Hkv,d,s,r,L,pos0,rope", [
    (1, 4, 2, 128, 4, 60, 64, 0, 0.0),          # first chunk, GQA pairs
    (1, 4, 2, 128, 4, 60, 60, 200, 1e4),        # L = r, RoPE, full cache
    (2, 2, 2, 64, 4, 100, 300, 500, 0.0),       # MHA halves, d = 64, superseded tokens, ragged
    (1, 8, 2, 128, 70, 50, 30, 20, 0.0),        # pos0 <= s, L < r: sinks from the cache and the chunk
    (1, 4, 4, 128, 0, 64, 200, 1000, 1e4),      # no sinks
    (1, 6, 2, 128, 4, 28, 517, 4096, 0.0),      # three q-heads per kv-head (256-row halves)
    (1, 2, 2, 128, 4, 2000, 2100, 5000, 1e4),   # long bands: copy steps every 2nd X half-slot
    (1, 8, 2, 128, 4, 1500, 1600, 3000, 0.0),   # long bands, GQA pairs
    (2, 2, 2, 64, 4, 900, 1000, 2000, 1e4),     # long bands, d = 64 (32-row copy steps)
])
def test_prefill_append_equals_separate_calls(gpu, B, Hq, Hkv, d, s, r, L, pos0, rope):
    """swa_prefill_append against swa_prefill + swa_cache_append: the same rows
    bit for bit, the next cache equal to the appended copy on every slot that
    holds a token, the NaN-poisoned empty slots unwritten, the current cache
    unchanged."""
    import sliding_window_attention_sink_amd as swa
    g = np.random.default_rng(L + pos0)
    mk = lambda H, n: si.round_bf16(g.standard_normal((B, H, n, d)).astype(np.float32))
    hk, hv = mk(Hkv, max(pos0, 1)), mk(Hkv, max(pos0, 1))
    q, k, v = mk(Hq, L), mk(Hkv, L), mk(Hkv, L)
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    kc, vc = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan"))
    if pos0:
        swa.cache_append(dev(hk, "bf16"), dev(hv, "bf16"), kc, vc, 0, s, r)
    kc0, vc0 = kc.clone(), vc.clone()
    kx, vx = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan"))
    say("prefill_append vs separate", B, Hq, Hkv, d, s, r, L, pos0, rope)
    cache = dict(k_cache=kc if pos0 else None, v_cache=vc if pos0 else None, pos0=pos0, rope_base=rope)
    of = swa.prefill_append(qd, kd, vd, s, r, kx, vx, **cache)
    op = swa.prefill(qd, kd, vd, s, r, **cache)
    kr, vr = kc.clone(), vc.clone()
    swa.cache_append(kd, vd, kr, vr, pos0, s, r)
    torch.cuda.synchronize()
    assert torch.equal(of, op)
    assert torch.equal(kc.view(torch.int16), kc0.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), vc0.view(torch.int16))
    full = filled_slots(s, r, pos0 + L)
    empty = sorted(set(range(s + r)) - set(full))
    for got, ref in ((kx, kr), (vx, vr)):
        assert torch.equal(got[:, :, full].view(torch.int16), ref[:, :, full].view(torch.int16))
        assert bool(torch.isnan(got[:, :, empty].float()).all())


@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
@pytest.mark.parametrize("chunk,first", [(100, None), (256, 88), (92, 48)])
def test_prefill_append_chunked_matches_oracle(gpu, rope_base, chunk, first):
    """The chunked prefill through swa_prefill_append (two cache pairs in
    turn; chunks of at least r = 92 tokens after a first chunk of any size,
    ending on the sequence's end) against
    the oracle's rows over the whole history, and its final cache against
    the separate-append run's."""
    B, Hq, Hkv, L, d, s, r = 1, 4, 2, 600, 128, 4, 92
    q, k, v = seq_inputs(15, B, Hq, Hkv, L, d)
    say("chunked fused", chunk, first, rope_base)
    o, (kx, vx) = run_chunked_fused(q, k, v, s, r, chunk, rope_base, first=first)
    ref = oracle.chunked_rows(q, k, v, s, r, rope_base=rope_base, rows=None).reshape(o.shape)
    err = max_err(host(o), ref)
    assert err <= TOL["bf16"], f"max-abs error {err}"
    import sliding_window_attention_sink_amd as swa
    kd = dev(k, "bf16")
    if rope_base:
        kd = swa.rope_keys(kd, 0, rope_base)
    kr, vr = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda")
    swa.cache_append(kd, dev(v, "bf16"), kr, vr, 0, s, r)
    torch.cuda.synchronize()
    assert torch.equal(kx.view(torch.int16), kr.view(torch.int16))
    assert torch.equal(vx.view(torch.int16), vr.view(torch.int16))


def test_prefill_append_guarded(gpu):
    """The fused call writes the next cache pair and the output, nothing
    around them (canary regions before and after each buffer)."""
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, L, d, s, r, pos0 = 1, 4, 2, 300, 128, 4, 120, 700
    q, k, v = seq_inputs(16, B, Hq, Hkv, L, d)
    h = seq_inputs(17, B, Hkv, Hkv, pos0, d)
    kc, vc = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda")
    swa.cache_append(dev(h[1], "bf16"), dev(h[2], "bf16"), kc, vc, 0, s, r)
    kb, kx = guarded((B, Hkv, s + r, d), torch.bfloat16, -3.0)
    vb, vx = guarded((B, Hkv, s + r, d), torch.bfloat16, -3.0)
    ob, o = guarded((B, Hq, L, d), torch.bfloat16, -5.0)
    say("guarded prefill_append")
    swa.prefill_append(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), s, r, kx, vx, k_cache=kc, v_cache=vc,
                       pos0=pos0, out=o)
    torch.cuda.synchronize()
    assert guard_intact(kb, -3.0) and guard_intact(vb, -3.0) and guard_intact(ob, -5.0)
    hk = np.concatenate([h[1], k], axis=2)
    hv = np.concatenate([h[2], v], axis=2)
    T = pos0 + L
    for slot in filled_slots(s, r, T):
        p = slot if slot < s else max(pt for pt in range(max(s, T - r), T) if s + pt % r == slot)
        assert np.array_equal(host(kx)[:, :, slot], hk[:, :, p]) and np.array_equal(host(vx)[:, :, slot], hv[:, :, p])


def test_chunked_rope_131072_full(gpu):
    """Chunked streaming prefill at full size (B=1, H=32, d=128, 131072 tokens
    in 32 chunks of 4096, s=4, r=4092, RoPE base 1e4): every 64th row, all
    heads, against the oracle; the fused-append run (the benchmark's step)
    gives the same rows bit for bit."""
    w = si.WORKLOADS[5]
    q, k, v = si.chunk_inputs(w, 0, w.L)
    say("chunked prefill full size", w.name)
    o = run_chunked(q, k, v, w.s, w.r, w.chunk, w.rope_base)
    of, _ = run_chunked_fused(q, k, v, w.s, w.r, w.chunk, w.rope_base)
    assert torch.equal(o, of)
    del of
    t = np.arange(0, w.L, w.check_every)
    rows = np.array([[0, h, tt] for h in range(w.Hq) for tt in t])
    got = host(o[0][:, t]).reshape(-1, w.d)
    ref = oracle.chunked_rows(q, k, v, w.s, w.r, rope_base=w.rope_base, rows=rows)
    err = max_err(got, ref)
    assert err <= TOL["bf16"], f"max-abs error {err}"
