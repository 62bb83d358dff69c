"""Task-bound global tokens (swa_prefill_global) on the GPU against the
oracle: a global row attends every key up to itself, other rows add the
global positions up to themselves to U(t), each key once."""
import numpy as np
import pytest
import torch

import oracle
import swa_inputs as si
from gpu_common import TOL, dev, host, max_err, say

pytestmark = pytest.mark.gpu


def inputs(seed, B, Hq, Hkv, L, d):
    g = np.random.default_rng(seed)
    mk = lambda H: si.round_bf16(g.standard_normal((B, H, L, d)).astype(np.float32))
    return mk(Hq), mk(Hkv), mk(Hkv)


# (B, Hq, Hkv, d, L, s, r, G): globals among the sinks, inside the window,
# just past it, at 0 and at L-1, more than 32 of them (two key blocks),
# GQA and d = 64, ragged L
CASES = [
    (1, 2, 1, 128, 300, 4, 28, [0, 2, 50, 51, 120, 299]),
    (2, 4, 2, 64, 257, 0, 16, [7, 100, 101, 102, 200]),
    (1, 8, 2, 128, 700, 3, 64, list(range(5, 700, 19))),       # 37 globals
    (1, 2, 2, 128, 130, 4, 200, [10, 60]),                      # window covers everything
    (1, 4, 4, 64, 1000, 30, 1, [29, 30, 31, 500, 999]),         # r = 1, globals at the sink edge
    (2, 2, 1, 128, 65, 70, 10, [3, 64]),                        # sinks beyond L
    # dense global rows batched 16 / (q-heads per kv-head) positions a launch
    (1, 2, 2, 128, 500, 4, 32, list(range(7, 500, 25))),       # 20 rows: launches of 16 + 4
    (1, 8, 1, 128, 333, 0, 50, [0, 100, 332]),                  # 8 q-heads: 2 + 1, a row at 0
    (1, 16, 1, 64, 200, 2, 30, [1, 40, 41, 199]),               # 16 q-heads: one position a launch
]


@pytest.mark.parametrize("case", CASES, ids=["B%dH%d-%dd%d_L%d_s%d_r%d_ng%d" % (c[:7] + (len(c[7]),))
                                             for c in CASES])
def test_global_matches_oracle(gpu, case):
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, d, L, s, r, G = case
    q, k, v = inputs(sum(case[:7]) + len(G), B, Hq, Hkv, L, d)
    say("global", case)
    o = host(swa.prefill_global(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), s, r, G))
    torch.cuda.synchronize()
    ref = oracle.prefill_rows(q, k, v, s, r, globals_=G).reshape(o.shape)
    assert max_err(o, ref) <= TOL["bf16"]


def test_no_globals_is_plain_prefill(gpu):
    import sliding_window_attention_sink_amd as swa
    q, k, v = inputs(3, 1, 4, 2, 333, 128)
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    say("global ng=0")
    a = swa.prefill_global(qd, kd, vd, 4, 50, [])
    b = swa.prefill(qd, kd, vd, 4, 50)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_global_output_guarded(gpu):
    """Canary rows before and after the output stay untouched."""
    import sliding_window_attention_sink_amd as swa
    B, Hq, Hkv, d, L, s, r, G = 1, 2, 1, 128, 200, 4, 20, [10, 150]
    q, k, v = inputs(9, B, Hq, Hkv, L, d)
    pad = 4096
    buf = torch.full((B * Hq * L * d + 2 * pad,), 3.5, dtype=torch.bfloat16, device="cuda")
    out = buf[pad:pad + B * Hq * L * d].view(B, Hq, L, d)
    say("global guarded")
    swa.prefill_global(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), s, r, G, out=out)
    torch.cuda.synchronize()
    assert bool((buf[:pad] == 3.5).all()) and bool((buf[-pad:] == 3.5).all())
    ref = oracle.prefill_rows(q, k, v, s, r, globals_=G).reshape(B, Hq, L, d)
    assert max_err(host(out), ref) <= TOL["bf16"]


def test_global_at_the_4_plus_1020_workload_size(gpu):
    """B = 4, H = 32, L = 16384, 4 sinks + 1020 recent (the StreamingLLM
    workload's tensors, sink keys from the mean query) with eight global
    tokens, one among the sinks and one inside a later window: every global
    row of every head, the rows right after each global, and random rows,
    against the oracle."""
    import sliding_window_attention_sink_amd as swa
    w = si.WORKLOADS[3]
    G = [2, 100, 2000, 2001, 7777, 12000, 12500, 16383]
    q, k, v = si.prefill_inputs(w)
    say("global 4+1020 size", w.name)
    o = swa.prefill_global(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), w.s, w.r, G)
    torch.cuda.synchronize()
    g = np.random.default_rng(5)
    pick = set()
    for b in range(w.B):
        for h in range(w.Hq):
            for t in G:
                pick.add((b, h, t))
                if t + 1 < w.L:
                    pick.add((b, h, t + 1))
    for _ in range(1500):
        pick.add((int(g.integers(0, w.B)), int(g.integers(0, w.Hq)), int(g.integers(0, w.L))))
    rows = np.array(sorted(pick))
    ref = oracle.prefill_rows(q, k, v, w.s, w.r, rows=rows, globals_=G)
    idx = torch.from_numpy(rows).to(o.device)
    got = host(o[idx[:, 0], idx[:, 1], idx[:, 2]])
    assert max_err(got, ref) <= TOL["bf16"]
