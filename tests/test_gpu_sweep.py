"""Seeded random sweep over the whole path against the oracle.

The targeted cases elsewhere aim at one code path each (sink packing, the
contiguous cache-tile runs, single-edge masks, skipped MFMA clusters, the
split-K merge).  Here every case draws its own configuration (batch, head
grouping, head dim, length, sinks, window, dtype, chunk boundaries, RoPE
base, decode splits) from a fixed seed, so the paths meet in combinations no
hand-picked case names.  Three kinds of case:

* prefill: one call over the whole sequence, fp32 or bf16;
* stream: bf16 chunked prefill over the rolling cache with irregular chunk
  lengths (1 token up to several tiles; some chunks start inside the sink
  range), then fused append + decode steps,
  all with one RoPE base (0 = none); every row is checked against the row
  definition over the whole history;
* dilated: the dilated-window prefill;
* backward (own draws): dq, dk, dv against the oracle's gradients, the
  forward's bf16 output as o;
* global tokens (own draws): every row of the global-token prefill, with up
  to 64 globals anywhere in the sequence (among the sinks, inside or past
  the window).

Large forward cases compare a random sample of rows (first and last rows
always in).
"""
import numpy as np
import pytest
import torch

import bwd_bounds
import oracle
import swa_inputs as si
from gpu_common import TOL, dev, host, max_err, rows_of, say

N_CASES = 120
ORACLE_PAIRS = 60_000_000  # (row, key) pairs above which rows are sampled
SAMPLE_ROWS = 2500


def sweep_case(i: int) -> dict:
    """Configuration of sweep case i (pure function of i)."""
    g = np.random.default_rng(np.random.SeedSequence([0x5EE9, i]))
    kind = ["prefill", "stream", "prefill", "stream", "dilated", "prefill"][i % 6]
    Hkv = int(g.choice([1, 2, 4]))
    grp = int(g.choice([1, 2, 4, 8]))
    while Hkv * grp > 16:
        grp //= 2
    c = dict(i=i, kind=kind, B=int(g.choice([1, 2])), Hq=Hkv * grp, Hkv=Hkv, d=int(g.choice([64, 128])))
    c["dtype"] = "f32" if kind != "stream" and g.random() < 0.3 else "bf16"
    c["L"] = int(g.choice([int(g.integers(1, 64)), int(g.integers(64, 700)), int(g.integers(700, 1600))],
                          p=[0.15, 0.45, 0.4]))
    c["s"] = int(g.choice([0, 1, 4, int(g.integers(2, 40)), int(g.integers(40, 140))], p=[0.25, 0.1, 0.3, 0.2, 0.15]))
    c["r"] = int(g.choice([1, int(g.integers(2, 70)), int(g.integers(70, 400)), int(g.integers(400, 1300)), 4096],
                          p=[0.08, 0.22, 0.35, 0.25, 0.1]))
    if kind == "stream":
        c["rope"] = float(g.choice([0.0, 500.0, 10000.0]))
        sizes, total = [], 0
        while total < c["L"]:
            n = int(g.choice([1, 7, 64, 100, 256, 333, int(g.integers(1, 600))]))
            if len(sizes) >= 24:
                n = c["L"] - total
            n = min(n, c["L"] - total)
            sizes.append(n)
            total += n
        c["chunks"] = sizes
        c["n_dec"] = int(g.integers(1, 6))
        c["n_split"] = int(g.choice([0, 1, 2, 3, 7]))
    if kind == "dilated":
        c["dil"] = int(g.choice([2, 3, 4, 7, int(g.integers(8, 300))]))
    return c


def case_id(c):
    extra = {"stream": lambda: "_rope%g_ch%d_dec%d" % (c["rope"], len(c["chunks"]), c["n_dec"]),
             "dilated": lambda: "_dil%d" % c["dil"]}.get(c["kind"], lambda: "")()
    return "%02d_%s_%s_B%dH%d-%dd%d_L%d_s%d_r%d%s" % (c["i"], c["kind"], c["dtype"], c["B"], c["Hq"], c["Hkv"], c["d"],
                                                  c["L"], c["s"], c["r"], extra)


CASES = [sweep_case(i) for i in range(N_CASES)]


def inputs(c, L):
    g = np.random.default_rng(np.random.SeedSequence([0x5EE9, c["i"], 1]))
    mk = lambda H: g.standard_normal((c["B"], H, L, c["d"])).astype(np.float32)
    q, k, v = mk(c["Hq"]), mk(c["Hkv"]), mk(c["Hkv"])
    if c["dtype"] == "bf16":
        q, k, v = si.round_bf16(q), si.round_bf16(k), si.round_bf16(v)
    return q, k, v


def pick_rows(c, L, g, keep_from=None):
    """Every row, or a random sample with the first and last rows of each
    (b, h) and every row from position keep_from on."""
    B, Hq = c["B"], c["Hq"]
    keys = min(L, c["s"] + c["r"])
    bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(L), indexing="ij")
    rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    if B * Hq * L * keys <= ORACLE_PAIRS:
        return rows
    keep = (rows[:, 2] == 0) | (rows[:, 2] == L - 1)
    if keep_from is not None:
        keep |= rows[:, 2] >= keep_from
    edge = rows[keep]
    pick = rows[g.choice(len(rows), size=SAMPLE_ROWS, replace=False)]
    return np.unique(np.concatenate([edge, pick]), axis=0)


def test_sweep_cases_cover_the_paths():
    """The drawn configurations reach the corners the sweep is for (CPU)."""
    kinds = {c["kind"] for c in CASES}
    assert kinds == {"prefill", "stream", "dilated"}
    assert any(c["dtype"] == "f32" for c in CASES) and any(c["dtype"] == "bf16" for c in CASES)
    assert any(c["r"] == 1 for c in CASES) and any(c["r"] >= c["L"] for c in CASES)
    assert any(c["s"] == 0 for c in CASES) and any(c["s"] > 64 for c in CASES)
    assert any(c["L"] < 64 for c in CASES) and any(c["L"] > 1000 for c in CASES)
    assert any(c["Hq"] // c["Hkv"] >= 4 for c in CASES) and any(c["Hq"] == c["Hkv"] for c in CASES)
    assert {64, 128} <= {c["d"] for c in CASES}
    streams = [c for c in CASES if c["kind"] == "stream"]
    assert {0.0} < {c["rope"] for c in streams}
    assert any(1 in c["chunks"] for c in streams)
    assert any(len(c["chunks"]) > 4 for c in streams)
    assert any(c["L"] > c["s"] + c["r"] for c in streams)   # the rolling buffer wraps
    # a chunk that starts inside the sink range: some sinks cached, some in the chunk
    assert any(any(0 < p < c["s"] for p in np.cumsum(c["chunks"][:-1])) for c in streams)
    for c in streams:
        assert sum(c["chunks"]) == c["L"] and min(c["chunks"]) >= 1


@pytest.mark.gpu
@pytest.mark.parametrize("c", CASES, ids=[case_id(c) for c in CASES])
def test_sweep_matches_oracle(gpu, c):
    import sliding_window_attention_sink_amd as swa
    say("sweep", case_id(c))
    B, Hq, Hkv, d, s, r, dt = c["B"], c["Hq"], c["Hkv"], c["d"], c["s"], c["r"], c["dtype"]
    L = c["L"]
    g = np.random.default_rng(np.random.SeedSequence([0x5EE9, c["i"], 2]))
    if c["kind"] == "prefill":
        q, k, v = inputs(c, L)
        o = host(swa.prefill(dev(q, dt), dev(k, dt), dev(v, dt), s, r))
        rows = pick_rows(c, L, g)
        ref = oracle.prefill_rows(q, k, v, s, r, rows=rows)
        got = rows_of(o, rows)
    elif c["kind"] == "dilated":
        q, k, v = inputs(c, L)
        o = host(swa.prefill_dilated(dev(q, dt), dev(k, dt), dev(v, dt), s, r, c["dil"]))
        rows = pick_rows(c, L, g)
        ref = oracle.prefill_rows(q, k, v, s, r, rows=rows, dilation=c["dil"])
        got = rows_of(o, rows)
    else:
        n_dec, base = c["n_dec"], c["rope"]
        T = L + n_dec
        q, k, v = inputs(c, T)
        qd, kd, vd = dev(q, dt), dev(k, dt), dev(v, dt)
        if base:
            kd = swa.rope_keys(kd, 0, base)
        kc, vc = swa.new_cache(B, Hkv, d, s, r, torch.bfloat16, "cuda", fill=float("nan"))
        out = torch.empty((B, Hq, T, d), dtype=torch.bfloat16, device="cuda")
        p0 = 0
        for n in c["chunks"]:
            qc, kk, vv = (x[:, :, p0:p0 + n].contiguous() for x in (qd, kd, vd))
            out[:, :, p0:p0 + n] = swa.prefill(qc, kk, vv, s, r, rope_base=base, k_cache=kc if p0 else None,
                                               v_cache=vc if p0 else None, pos0=p0)
            swa.cache_append(kk, vv, kc, vc, p0, s, r)
            p0 += n
        for t in range(L, T):
            out[:, :, t] = swa.decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                           vd[:, :, t].contiguous(), kc, vc, t + 1, s, r, rope_base=base,
                                           n_split=c["n_split"])
        torch.cuda.synchronize()
        o = host(out)
        rows = pick_rows(c, T, g, keep_from=L)
        ref = oracle.prefill_rows(q, k, v, s, r, rope_base=base, rows=rows)
        got = rows_of(o, rows)
    err = max_err(got, ref)
    assert err <= TOL[dt], f"max-abs error {err} over {len(ref)} rows"


# ---- backward: its own seeded draws (bf16 inputs, the forward's output as o)
N_BWD = 24


def bwd_case(i: int) -> dict:
    g = np.random.default_rng(np.random.SeedSequence([0xB4D, i]))
    Hkv = int(g.choice([1, 2, 4]))
    grp = int(g.choice([1, 2, 4, 8]))
    while Hkv * grp > 16:
        grp //= 2
    return dict(i=i, kind="backward", dtype="bf16", B=int(g.choice([1, 2])), Hq=Hkv * grp, Hkv=Hkv,
                d=int(g.choice([64, 128])),
                L=int(g.choice([int(g.integers(1, 40)), int(g.integers(40, 500)), int(g.integers(500, 1200))],
                               p=[0.15, 0.5, 0.35])),
                s=int(g.choice([0, 1, 4, int(g.integers(2, 40)), int(g.integers(40, 140))], p=[0.3, 0.1, 0.3, 0.2, 0.1])),
                r=int(g.choice([1, int(g.integers(2, 70)), int(g.integers(70, 400)), 4096], p=[0.1, 0.35, 0.4, 0.15])))


BWD_CASES = [bwd_case(i) for i in range(N_BWD)]


def test_backward_sweep_cases_cover_the_paths():
    """Dense limit, r = 1, sinks past the window (the sink segments), GQA
    and both head dims among the drawn backward cases (CPU)."""
    assert any(c["r"] == 1 for c in BWD_CASES) and any(c["r"] >= c["L"] for c in BWD_CASES)
    assert any(c["s"] > 0 and c["L"] > c["s"] + c["r"] for c in BWD_CASES)
    assert any(c["Hq"] // c["Hkv"] >= 4 for c in BWD_CASES) and {64, 128} <= {c["d"] for c in BWD_CASES}
    assert any(c["L"] % 8 for c in BWD_CASES)   # a partial group of eight rows / keys


@pytest.mark.gpu
@pytest.mark.parametrize("c", BWD_CASES, ids=["%02d_B%dH%d-%dd%d_L%d_s%d_r%d" % (c["i"], c["B"], c["Hq"], c["Hkv"], c["d"],
                                                                            c["L"], c["s"], c["r"]) for c in BWD_CASES])
def test_backward_sweep_matches_oracle(gpu, c):
    """Gradients element by element within the bars of tests/bwd_bounds.py
    (2^-8 of each element's term magnitudes; the bar of the targeted
    backward tests)."""
    import sliding_window_attention_sink_amd as swa
    say("backward sweep", c)
    B, Hq, Hkv, d, L, s, r = c["B"], c["Hq"], c["Hkv"], c["d"], c["L"], c["s"], c["r"]
    g = np.random.default_rng(np.random.SeedSequence([0xB4D, c["i"], 1]))
    q, k, v, do = (si.round_bf16(g.standard_normal((B, H, L, d)).astype(np.float32)) for H in (Hq, Hkv, Hkv, Hq))
    qd, kd, vd, dod = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(do, "bf16")
    od = swa.prefill(qd, kd, vd, s, r)
    dq, dk, dv = swa.backward(qd, kd, vd, od, dod, s, r)
    torch.cuda.synchronize()
    o = host(od)
    refs = oracle.backward(q, k, v, o, do, s, r)
    for name, got, ref, bar in zip(("dq", "dk", "dv"), (dq, dk, dv), refs, bwd_bounds.bars(q, k, v, o, do, s, r)):
        bwd_bounds.check(name, host(got), ref, bar)


# ---- task-bound global tokens: their own seeded draws (bf16)
N_GLB = 24


def glb_case(i: int) -> dict:
    g = np.random.default_rng(np.random.SeedSequence([0x610B, i]))
    Hkv = int(g.choice([1, 2, 4]))
    grp = int(g.choice([1, 2, 4, 8, 16]))
    while Hkv * grp > 16:
        grp //= 2
    L = int(g.choice([int(g.integers(1, 64)), int(g.integers(64, 700)), int(g.integers(700, 1500))],
                     p=[0.15, 0.45, 0.4]))
    c = dict(i=i, kind="global", dtype="bf16", B=int(g.choice([1, 2])), Hq=Hkv * grp, Hkv=Hkv,
             d=int(g.choice([64, 128])), L=L,
             s=int(g.choice([0, 1, 4, int(g.integers(2, 40)), int(g.integers(40, 140))], p=[0.25, 0.1, 0.3, 0.2, 0.15])),
             r=int(g.choice([1, int(g.integers(2, 70)), int(g.integers(70, 400)), 4096], p=[0.1, 0.4, 0.35, 0.15])))
    ng = int(min(L, g.choice([1, int(g.integers(2, 9)), int(g.integers(9, 40)), 64], p=[0.2, 0.4, 0.3, 0.1])))
    c["globals"] = sorted(int(x) for x in g.choice(L, size=ng, replace=False))
    return c


GLB_CASES = [glb_case(i) for i in range(N_GLB)]


def glb_id(c):
    return "%02d_B%dH%d-%dd%d_L%d_s%d_r%d_ng%d" % (c["i"], c["B"], c["Hq"], c["Hkv"], c["d"], c["L"], c["s"], c["r"],
                                                  len(c["globals"]))


def test_global_sweep_cases_cover_the_paths():
    """Globals among the sinks and past the window, 64 globals (one full
    key tile), 16 q-heads per kv-head (one dense row a launch), both head
    dims (CPU)."""
    assert any(c["globals"][0] < c["s"] for c in GLB_CASES)
    assert any(c["globals"][-1] >= c["s"] + c["r"] for c in GLB_CASES)
    assert any(len(c["globals"]) == 64 for c in GLB_CASES)
    assert any(c["Hq"] // c["Hkv"] == 16 for c in GLB_CASES)
    assert {64, 128} <= {c["d"] for c in GLB_CASES}
    for c in GLB_CASES:
        assert len(set(c["globals"])) == len(c["globals"]) and max(c["globals"]) < c["L"]


@pytest.mark.gpu
@pytest.mark.parametrize("c", GLB_CASES, ids=[glb_id(c) for c in GLB_CASES])
def test_global_sweep_matches_oracle(gpu, c):
    import sliding_window_attention_sink_amd as swa
    say("global sweep", glb_id(c))
    B, Hq, Hkv, d, L, s, r = c["B"], c["Hq"], c["Hkv"], c["d"], c["L"], c["s"], c["r"]
    g = np.random.default_rng(np.random.SeedSequence([0x610B, c["i"], 1]))
    q, k, v = (si.round_bf16(g.standard_normal((B, H, L, d)).astype(np.float32)) for H in (Hq, Hkv, Hkv))
    o = host(swa.prefill_global(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), s, r, c["globals"]))
    torch.cuda.synchronize()
    ref = oracle.prefill_rows(q, k, v, s, r, globals_=c["globals"]).reshape(o.shape)
    err = max_err(o, ref)
    assert err <= TOL["bf16"], f"max-abs error {err}"
