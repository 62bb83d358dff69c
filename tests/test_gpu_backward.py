"""Backward (training) on the GPU, through the C ABI, against the oracle's
fp64 gradients, element by element.  The bar of every element is 2^-8 of
the magnitude sum of its terms (tests/bwd_bounds.py: the kernels round P and
dS to bf16 before the products and sum in fp32)."""
import numpy as np
import pytest
import torch

import oracle
import swa_inputs as si
from bwd_bounds import bars, check
from gpu_common import dev, host, say

pytestmark = pytest.mark.gpu


def bf16_normal(g, shape):
    return si.round_bf16(g.standard_normal(shape).astype(np.float32))


def run_backward(q, k, v, do, s, r, o=None):
    """The GPU backward; o is the GPU forward's output unless given.  Returns
    host arrays o, dq, dk, dv."""
    import sliding_window_attention_sink_amd as swa
    qd, kd, vd, dod = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(do, "bf16")
    od = swa.prefill(qd, kd, vd, s, r) if o is None else dev(o, "bf16")
    dq, dk, dv = swa.backward(qd, kd, vd, od, dod, s, r)
    torch.cuda.synchronize()
    return host(od), host(dq), host(dk), host(dv)


def check_all(q, k, v, o, do, s, r, got):
    refs = oracle.backward(q, k, v, o, do, s, r)
    for name, gt, ref, bar in zip(("dq", "dk", "dv"), got, refs, bars(q, k, v, o, do, s, r)):
        check(name, gt, ref, bar)


# (B, Hq, Hkv, d, L, s, r): ragged tails, GQA up to 8, r = 1, r >= L, more
# sinks than positions, sink keys whose queries span several segments of
# the dK/dV kernel (L - r > 256 blocks of queries for one q-head), sinks
# beyond the first key tile (s > 128)
CASES = [
    (1, 2, 2, 128, 300, 4, 28),
    (2, 4, 2, 64, 257, 0, 1),
    (1, 8, 1, 128, 333, 4, 100),
    (1, 2, 1, 128, 1500, 4, 100),
    (1, 2, 2, 64, 50, 70, 40),
    (1, 4, 4, 128, 400, 0, 1000),
    (2, 4, 2, 128, 700, 30, 64),
    (1, 1, 1, 128, 9000, 4, 60),
    (1, 2, 1, 64, 700, 200, 50),
    (1, 4, 1, 128, 31, 2, 5),
]


@pytest.mark.parametrize("case", CASES, ids=["B%dH%d-%dd%d_L%d_s%d_r%d" % c for c in CASES])
def test_backward_matches_oracle(gpu, case):
    B, Hq, Hkv, d, L, s, r = case
    g = np.random.default_rng(sum(case))
    q, k, v = (bf16_normal(g, (B, H, L, d)) for H in (Hq, Hkv, Hkv))
    do = bf16_normal(g, (B, Hq, L, d))
    say("backward", case)
    o, dq, dk, dv = run_backward(q, k, v, do, s, r)
    check_all(q, k, v, o, do, s, r, (dq, dk, dv))


def test_backward_with_the_oracles_forward():
    """o from the oracle's fp64 forward rounded to bf16, given to both sides
    (no GPU forward anywhere in the expected gradients)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    B, Hq, Hkv, d, L, s, r = 1, 4, 2, 128, 600, 4, 90
    g = np.random.default_rng(5)
    q, k, v = (bf16_normal(g, (B, H, L, d)) for H in (Hq, Hkv, Hkv))
    do = bf16_normal(g, (B, Hq, L, d))
    o = si.round_bf16(oracle.prefill_rows(q, k, v, s, r).reshape(B, Hq, L, d).astype(np.float32))
    say("backward with the oracle's forward")
    _, dq, dk, dv = run_backward(q, k, v, do, s, r, o=o)
    check_all(q, k, v, o, do, s, r, (dq, dk, dv))


def test_backward_deterministic_and_guarded(gpu):
    """Two calls give the same bits (no atomics: split key tiles are summed
    in a fixed order); canary bytes around every output stay untouched."""
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, d, L, s, r = 1, 4, 1, 128, 3000, 4, 100
    g = torch.Generator(device="cuda").manual_seed(3)
    mk = lambda H: torch.randn(B, H, L, d, device="cuda", generator=g).to(torch.bfloat16)
    q, k, v, do = mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)
    o = swa.prefill(q, k, v, s, r)
    pad = 4096
    outs = []
    for _ in range(2):
        bufs = [torch.full((n + 2 * pad,), 7.25, dtype=torch.float32, device="cuda") for n in
                (q.numel(), k.numel(), k.numel())]
        views = [bb[pad:pad + x.numel()].view(x.shape) for bb, x in zip(bufs, (q, k, k))]
        swa.backward(q, k, v, o, do, s, r, dq=views[0], dk=views[1], dv=views[2])
        torch.cuda.synchronize()
        for bb in bufs:
            assert bool((bb[:pad] == 7.25).all()) and bool((bb[-pad:] == 7.25).all())
        outs.append([x.clone() for x in views])
    for a_, b_ in zip(*outs):
        assert torch.equal(a_, b_)


def test_backward_at_bench_size(gpu):
    """GQA 32/8, d = 128, L = 8192, s = 4, r = 4092: dk and dv of kv-head 0
    element by element against the oracle (its four q-heads), dq of a
    600-row prefix of every head, and the value-gradient sum rule of every
    kv-head."""
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, d, L, s, r = 1, 32, 8, 128, 8192, 4, 4092
    g = torch.Generator(device="cuda").manual_seed(7)
    mk = lambda H: torch.randn(B, H, L, d, device="cuda", generator=g).to(torch.bfloat16)
    q, k, v, do = mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)
    say("backward bench size")
    o = swa.prefill(q, k, v, s, r)
    dq, dk, dv = swa.backward(q, k, v, o, do, s, r)
    torch.cuda.synchronize()
    G = Hq // Hkv
    # sum_i dV_i = the group's summed dout (rows of P sum to one)
    want = do.double().reshape(B, Hkv, G, L, d).sum(dim=(2, 3))
    vsum = dv.double().sum(dim=2)
    assert float((vsum - want).abs().max()) <= 2.0 ** -8 * float(want.abs().max()) + 1e-3
    # kv-head 0 in full: its q-heads 0 .. G-1
    qh, kh, vh, oh, doh = (host(x[:, :G] if x.shape[1] == Hq else x[:, :1]) for x in (q, k, v, o, do))
    rq, rk, rv = oracle.backward(qh, kh, vh, oh, doh, s, r)
    bq, bk, bv = bars(qh, kh, vh, oh, doh, s, r)
    check("dk kv-head 0", host(dk[:, :1]), rk, bk)
    check("dv kv-head 0", host(dv[:, :1]), rv, bv)
    check("dq heads 0-3", host(dq[:, :G]), rq, bq)
    # rows of the first 600 positions, every head: dq there depends on the
    # prefix only, so the oracle runs on the prefix
    P = 600
    qh, kh, vh, oh, doh = (host(x[:, :, :P]) for x in (q, k, v, o, do))
    rq, _, _ = oracle.backward(qh, kh, vh, oh, doh, s, r)
    bq, _, _ = bars(qh, kh, vh, oh, doh, s, r)
    check("dq prefix", host(dq[:, :, :P]), rq, bq)
