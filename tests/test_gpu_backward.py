"""Backward (training) on the GPU, through the C ABI, against the oracle's
fp64 gradients.  The kernels recompute P from bf16 q, k in fp32 and
accumulate in fp32: each gradient element is a sum of at most L * Hq / Hkv
fp32 products, so the error stays near sqrt(terms) * 2^-24 of the sum of
magnitudes; the bar is 1e-4 of max(1, largest |gradient|) per tensor."""
import numpy as np
import pytest
import torch

import oracle
import swa_inputs as si
from gpu_common import dev, host, say

pytestmark = pytest.mark.gpu
REL = 1e-4


def bf16_normal(g, shape):
    return si.round_bf16(g.standard_normal(shape).astype(np.float32))


def run_backward(q, k, v, do, s, r):
    """Forward on the GPU (its bf16 output is the O both sides use), then the
    backward.  Returns host arrays o, dq, dk, dv."""
    import sliding_window_attention_sink_amd as swa
    qd, kd, vd, dod = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(do, "bf16")
    od = swa.prefill(qd, kd, vd, s, r)
    dq, dk, dv = swa.backward(qd, kd, vd, od, dod, s, r)
    torch.cuda.synchronize()
    return host(od), host(dq), host(dk), host(dv)


def check(name, got, ref):
    err = float(np.abs(got - ref).max())
    bar = REL * max(1.0, float(np.abs(ref).max()))
    assert np.isfinite(got).all(), f"{name}: non-finite"
    assert err <= bar, f"{name}: max-abs error {err} > {bar}"


# (B, Hq, Hkv, d, L, s, r): ragged tails, GQA up to 8, r = 1, r >= L, more
# sinks than positions, and sink keys with two query segments past their
# first r queries (L - r > 1024)
CASES = [
    (1, 2, 2, 128, 300, 4, 28),
    (2, 4, 2, 64, 257, 0, 1),
    (1, 8, 1, 128, 333, 4, 100),
    (1, 2, 1, 128, 1500, 4, 100),
    (1, 2, 2, 64, 50, 70, 40),
    (1, 4, 4, 128, 400, 0, 1000),
    (2, 4, 2, 128, 700, 30, 64),
]


@pytest.mark.parametrize("case", CASES, ids=["B%dH%d-%dd%d_L%d_s%d_r%d" % c for c in CASES])
def test_backward_matches_oracle(gpu, case):
    B, Hq, Hkv, d, L, s, r = case
    g = np.random.default_rng(sum(case))
    q, k, v = (bf16_normal(g, (B, H, L, d)) for H in (Hq, Hkv, Hkv))
    do = bf16_normal(g, (B, Hq, L, d))
    say("backward", case)
    o, dq, dk, dv = run_backward(q, k, v, do, s, r)
    rq, rk, rv = oracle.backward(q, k, v, o, do, s, r)
    check("dq", dq, rq)
    check("dk", dk, rk)
    check("dv", dv, rv)


def test_backward_sum_rules_at_bench_size(gpu):
    """GQA 32/8, d = 128, L = 8192, s = 4, r = 4092 (the backward the bench
    times): per (batch, kv-head) the value gradients sum to the group's
    summed dout and the key gradients to zero up to the rounding of o; the
    dq rows of a prefix against the oracle (row t depends on keys <= t
    only)."""
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, d, L, s, r = 1, 32, 8, 128, 8192, 4, 4092
    g = torch.Generator(device="cuda").manual_seed(7)
    mk = lambda H: torch.randn(B, H, L, d, device="cuda", generator=g).to(torch.bfloat16)
    q, k, v, do = mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)
    say("backward bench size")
    o = swa.prefill(q, k, v, s, r)
    dq, dk, dv = swa.backward(q, k, v, o, do, s, r)
    torch.cuda.synchronize()
    # sum_i dK_i = scale sum_t q_t dout_t . (P_t V - o_t): zero for the exact
    # output, and here o is the forward's bf16 output (within 2^-9 of it, per
    # element), so the sum is bounded by scale sum_t |q_t| 2^-8 |dout_t| . |o_t|
    # plus the fp32 accumulation allowance
    G = Hq // Hkv
    rt = (do.double().abs() * o.double().abs()).sum(dim=-1, keepdim=True) * 2.0 ** -8
    bound = (d ** -0.5) * (q.double().abs() * rt).reshape(B, Hkv, G, L, d).sum(dim=(2, 3))
    bound += REL * dk.double().abs().sum(dim=2)
    ksum = dk.double().sum(dim=2)
    assert bool((ksum.abs() <= bound).all()), float((ksum.abs() / bound).max())
    want = do.double().reshape(B, Hkv, Hq // Hkv, L, d).sum(dim=(2, 3))
    vsum = dv.double().sum(dim=2)
    assert float((vsum - want).abs().max()) <= REL * max(1.0, float(want.abs().max()))
    # rows of the first 600 positions, every head: dq there depends on the
    # prefix only, so the oracle runs on the prefix
    P = 600
    qh, kh, vh, oh, doh = (host(x[:, :, :P]) for x in (q, k, v, o, do))
    rq, _, _ = oracle.backward(qh, kh, vh, oh, doh, s, r)
    check("dq prefix", host(dq[:, :, :P]), rq)
