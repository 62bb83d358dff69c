"""Canary regions around every output and cache buffer the library writes:
a call writes exactly its output (the bytes before and after stay as the
caller set them) and the written values are right.  Prefill and backward
outputs have their own guarded tests (test_gpu_prefill, test_gpu_backward,
test_gpu_global)."""
import numpy as np
import pytest
import torch

import oracle
import swa_inputs as si
from gpu_common import TOL, dev, guard_intact, guarded, host, max_err, say

pytestmark = pytest.mark.gpu


def normal(g, shape):
    return si.round_bf16(g.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("n_split", [1, 3])
def test_decode_and_append_guarded(gpu, n_split):
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, d, s, r, T = 2, 8, 2, 128, 4, 60, 150
    g = np.random.default_rng(n_split)
    K, V = normal(g, (B, Hkv, T, d)), normal(g, (B, Hkv, T, d))
    q = normal(g, (B, Hq, d))
    S = s + r
    kb, kc = guarded((B, Hkv, S, d), torch.bfloat16, float("nan"))
    vb, vc = guarded((B, Hkv, S, d), torch.bfloat16, float("nan"))
    ob, o = guarded((B, Hq, d), torch.bfloat16, -7.0)
    say("guarded append + decode", n_split)
    swa.cache_append(dev(K, "bf16"), dev(V, "bf16"), kc, vc, 0, s, r)
    swa.decode(dev(q, "bf16"), kc, vc, T, s, r, n_split=n_split, out=o)
    torch.cuda.synchronize()
    # NaN canaries: compare bit patterns (NaN != NaN)
    for buf in (kb, vb):
        bits = buf.view(torch.int16)
        nan_bits = torch.tensor([float("nan")], dtype=torch.bfloat16).view(torch.int16).item()
        assert bool((bits[:4096] == nan_bits).all()) and bool((bits[-4096:] == nan_bits).all())
    assert guard_intact(ob, -7.0)
    sim = oracle.RollingCacheSim(B, Hkv, d, s, r)
    sim.append(K, V, 0)
    got = host(o)
    for b in range(B):
        for h in range(Hq):
            ref = oracle.decode_row(sim, q[b, h], b, h, Hq)
            assert max_err(got[b, h], ref) <= TOL["bf16"]


def test_fused_step_guarded(gpu):
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, d, s, r = 1, 4, 2, 64, 2, 30
    g = np.random.default_rng(9)
    steps = 70
    K, V, Q = normal(g, (B, Hkv, steps, d)), normal(g, (B, Hkv, steps, d)), normal(g, (B, Hq, steps, d))
    kb, kc = guarded((B, Hkv, s + r, d), torch.bfloat16, 0.5)
    vb, vc = guarded((B, Hkv, s + r, d), torch.bfloat16, 0.5)
    Kd, Vd, Qd = dev(K, "bf16"), dev(V, "bf16"), dev(Q, "bf16")
    say("guarded fused steps")
    for t in range(steps):
        ob, o = guarded((B, Hq, d), torch.bfloat16, 9.0)
        swa.decode_step(Qd[:, :, t].contiguous(), Kd[:, :, t].contiguous(), Vd[:, :, t].contiguous(), kc, vc,
                        t + 1, s, r, out=o)
        torch.cuda.synchronize()
        assert guard_intact(ob, 9.0), t
    assert guard_intact(kb, 0.5) and guard_intact(vb, 0.5)


def test_dilated_output_guarded(gpu):
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, d, L, s, r, dil = 1, 4, 2, 128, 300, 4, 40, 3
    g = np.random.default_rng(4)
    q, k, v = normal(g, (B, Hq, L, d)), normal(g, (B, Hkv, L, d)), normal(g, (B, Hkv, L, d))
    ob, o = guarded((B, Hq, L, d), torch.bfloat16, 5.0)
    say("guarded dilated")
    swa.prefill_dilated(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), s, r, dil, out=o)
    torch.cuda.synchronize()
    assert guard_intact(ob, 5.0)
    ref = oracle.prefill_rows(q, k, v, s, r, dilation=dil).reshape(B, Hq, L, d)
    assert max_err(host(o), ref) <= TOL["bf16"]


def test_rope_keys_guarded(gpu):
    import sliding_window_attention_sink_amd as swa
    B, Hkv, n, d = 2, 3, 100, 128
    g = np.random.default_rng(6)
    k = normal(g, (B, Hkv, n, d))
    kb, kr = guarded((B, Hkv, n, d), torch.bfloat16, -2.0)
    say("guarded rope keys")
    swa.rope_keys(dev(k, "bf16"), 1000, 1e4, out=kr)
    torch.cuda.synchronize()
    assert guard_intact(kb, -2.0)
