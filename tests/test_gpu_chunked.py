"""Chunked streaming prefill over the rolling cache, with and without RoPE
re-positioning, against the oracle's row definition over the whole history."""
import numpy as np
import pytest
import torch

import oracle
import swa_inputs as si
from gpu_common import TOL, dev, host, max_err, say

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


def test_chunked_rope_131072_full(gpu):
    """Chunked streaming prefill at full size (B=1, H=32, d=128, 131072 tokens
    in 32 chunks of 4096, s=4, r=4092, RoPE base 1e4): every 64th row, all heads, against the oracle."""
    w = si.WORKLOADS[5]
    q, k, v = si.chunk_inputs(w, 0, w.L)
    say("chunked prefill full size", w.name)
    o = run_chunked(q, k, v, w.s, w.r, w.chunk, w.rope_base)
    t = np.arange(0, w.L, w.check_every)
    rows = np.array([[0, h, tt] for h in range(w.Hq) for tt in t])
    got = host(o[0][:, t]).reshape(-1, w.d)
    ref = oracle.chunked_rows(q, k, v, w.s, w.r, rope_base=w.rope_base, rows=rows)
    err = max_err(got, ref)
    assert err <= TOL["bf16"], f"max-abs error {err}"
