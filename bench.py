#!/usr/bin/env python3
"""Throughput of sliding-window attention with sinks on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--only-main]

One step = one banded prefill of the GQA Mistral-style workload (B=1, Hq=32,
Hkv=8, d=128, L=8192, s=0, r=4096, bf16), inputs resident in HBM.  The JSON
line's value is its algorithmic TFLOP/s: only the (query, key) pairs of the
sink + window key set count, 4*d flops each.  Alongside it (under "extra")
the same run times the StreamingLLM 4+1020 prefill (B=4, H=32, L=16384), the
rolling-buffer decode loop (B=64, 32/8 heads, 4+4092 slots, append + decode
per step, as one fused launch and as two) and the chunked RoPE streaming prefill (131072 tokens in chunks of
4096) and the main workload's backward (dq, dk, dv).  The "cpu_baseline"
leg times the fp64 oracle on a bounded sample of the main workload's rows.

Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

MAIN_KERNEL = "prefill_pp_kernel<128>"
# HBM bytes per launch of MAIN_KERNEL on the main workload, from rocprofv3
# FETCH_SIZE / WRITE_SIZE runs scaled by a plain-copy calibration; valid only
# while the kernel sources hash to the value recorded beside it.
TRAFFIC_NOTE = os.path.join(ROOT, "profiles", "prefill_pp_kernel_gqa32x8_L8192_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "sliding_window_attention_sink_amd", "csrc", f)
                  for f in ("prefill_bf16.hip", "prefill_common.h", "swa_internal.h")]


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """Bytes per launch from the counter note, or None if absent or stale."""
    try:
        text = open(TRAFFIC_NOTE).read()
    except OSError:
        return None
    m_b = re.search(r"^traffic_bytes_per_launch:\s*([0-9]+)\s*$", text, re.M)
    m_h = re.search(r"^kernel_sources_sha256:\s*([0-9a-f]{64})\s*$", text, re.M)
    if not (m_b and m_h) or m_h.group(1) != kernel_sources_sha256():
        return None
    return int(m_b.group(1))


MFMA_NOTE = os.path.join(ROOT, "profiles", "prefill_pp_kernel_gqa32x8_L8192_mfma.md")


def recorded_mfma_busy():
    """Fraction of the main kernel's cycles with the matrix units busy, from
    the SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE counter note, or None if
    absent or stale."""
    try:
        text = open(MFMA_NOTE).read()
    except OSError:
        return None
    m_u = re.search(r"^mfma_busy_frac:\s*([0-9.]+)\s*$", text, re.M)
    m_h = re.search(r"^kernel_sources_sha256:\s*([0-9a-f]{64})\s*$", text, re.M)
    if not (m_u and m_h) or m_h.group(1) != kernel_sources_sha256():
        return None
    return float(m_u.group(1))


SCLK_NOTE = os.path.join(ROOT, "profiles", "prefill_pp_kernel_gqa32x8_L8192_sclk.md")


def recorded_sclk():
    """Shader clock (GHz) during the main kernel's timed launches, from the
    GRBM_COUNT note, or None if absent or stale."""
    try:
        text = open(SCLK_NOTE).read()
    except OSError:
        return None
    m_c = re.search(r"^sclk_ghz_timed:\s*([0-9.]+)\s*$", text, re.M)
    m_h = re.search(r"^kernel_sources_sha256:\s*([0-9a-f]{64})\s*$", text, re.M)
    if not (m_c and m_h) or m_h.group(1) != kernel_sources_sha256():
        return None
    return float(m_c.group(1))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def key_count_sum(L: int, s: int, r: int, pos0: int = 0) -> int:
    """sum over query rows t = pos0 .. pos0+L-1 of |U(t)| = min(t+1, s+r)."""
    t = np.arange(pos0, pos0 + L, dtype=np.int64)
    return int(np.minimum(t + 1, s + r).sum())


def prefill_flops(w) -> float:
    return 4.0 * w.d * key_count_sum(w.L, w.s, w.r) * w.B * w.Hq


class LaunchTimer:
    """HIP events around each launch, on the stream the kernels go to."""

    def __init__(self, torch, stream):
        self.torch, self.stream, self.pairs = torch, stream, []

    def __enter__(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self._start = e
        return self

    def __exit__(self, *exc):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.append((self._start, e))

    def mean_ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs]))


SETTLE_MS = 150.0


class Settler:
    """Brings the GPU clock to its loaded level before a timed region.

    After an idle spell (here: staging each workload's inputs on the CPU) the
    graphics clock ramps up over the first ~20 ms of load: on the main
    workload the first 50 back-to-back launches run at ~0.45 ms each, every
    later one at ~0.38 ms.  Each timed region is therefore preceded by
    SETTLE_MS of back-to-back launches of the main prefill kernel on random
    tensors of the main workload's shape (untimed; the steady-state rate is
    what the metric asks for, and the cold rate is reported beside it)."""

    def __init__(self, torch, swa, w, ms: float = SETTLE_MS):
        self.torch, self.swa, self.w, self.ms = torch, swa, w, ms
        self.t = None

    def __call__(self):
        torch, w, ms = self.torch, self.w, self.ms
        if self.t is None:
            g = torch.Generator(device="cuda").manual_seed(7)
            q = torch.randn((w.B, w.Hq, w.L, w.d), generator=g, device="cuda").to(torch.bfloat16)
            k = torch.randn((w.B, w.Hkv, w.L, w.d), generator=g, device="cuda").to(torch.bfloat16)
            v = torch.randn((w.B, w.Hkv, w.L, w.d), generator=g, device="cuda").to(torch.bfloat16)
            self.t = (q, k, v, torch.empty_like(q))
        q, k, v, o = self.t
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(8):
                self.swa.prefill(q, k, v, w.s, w.r, out=o)
            torch.cuda.synchronize()


def _no_settle():
    return None


def to_dev(torch, x, dtype):
    return torch.from_numpy(x).to("cuda").to(dtype).contiguous()


def bench_prefill(torch, swa, w, steps, warmup, settle=_no_settle):
    q, k, v = __import__("swa_inputs").prefill_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = to_dev(torch, q, dt), to_dev(torch, k, dt), to_dev(torch, v, dt)
    del q, k, v
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream()
    settle()
    for _ in range(warmup):
        swa.prefill(qd, kd, vd, w.s, w.r, out=out)
    torch.cuda.synchronize()
    # one step is one launch of the kernel, so the events around the K
    # back-to-back launches give its mean launch duration; events between
    # launches would add a cache flush and a stall to every launch
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        swa.prefill(qd, kd, vd, w.s, w.r, out=out)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    flops = prefill_flops(w)
    return {"ms": ms, "kernel_ms": ms, "flops": flops, "tflops": flops / ms / 1e9}


def bench_window_sweep(torch, swa, w, windows, steps=10, settle=_no_settle):
    """Prefill of the main workload's tensors at several window sizes r (s as
    given), up to r >= L, i.e. full causal attention: time and cache size."""
    q, k, v = __import__("swa_inputs").prefill_inputs(w)
    qd, kd, vd = (to_dev(torch, x, torch.bfloat16) for x in (q, k, v))
    del q, k, v
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream()
    res = {}
    settle()
    for r in windows:
        for _ in range(2):
            swa.prefill(qd, kd, vd, w.s, r, out=out)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            swa.prefill(qd, kd, vd, w.s, r, out=out)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        flops = 4.0 * w.d * key_count_sum(w.L, w.s, r) * w.B * w.Hq
        res["r%d" % r] = {"ms": ms, "tflops": flops / ms / 1e9,
                          "cache_slots": min(w.s + r, w.L), "full_attention": w.s + r >= w.L}
    return res


def dilated_key_count_sum(L: int, s: int, r: int, dil: int) -> int:
    """sum over rows t of |U(t)| with a dilated window: min(s, t+1) sinks plus
    min(r, (t-s)//dil + 1) window keys for t >= s."""
    t = np.arange(L, dtype=np.int64)
    win = np.where(t >= s, np.minimum(r, (t - s) // dil + 1), 0)
    return int((np.minimum(s, t + 1) + win).sum())


def bench_dilated(torch, swa, w, dilations, steps=10, settle=_no_settle):
    """Dilated-window prefill of the main workload's tensors (gather, banded
    prefill of the residue classes, scatter), algorithmic TFLOP/s."""
    q, k, v = __import__("swa_inputs").prefill_inputs(w)
    qd, kd, vd = (to_dev(torch, x, torch.bfloat16) for x in (q, k, v))
    del q, k, v
    out = torch.empty_like(qd)
    desc = swa.make_desc(w.B, w.Hq, w.Hkv, w.d, w.s, w.r, torch.bfloat16)
    stream = torch.cuda.current_stream()
    res = {}
    settle()
    for dil in dilations:
        ws = torch.empty(max(16, swa._lib.swa_prefill_dilated_workspace_bytes(desc, w.L, dil)), dtype=torch.uint8,
                         device="cuda")
        for _ in range(2):
            swa.prefill_dilated(qd, kd, vd, w.s, w.r, dil, out=out, workspace=ws)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            swa.prefill_dilated(qd, kd, vd, w.s, w.r, dil, out=out, workspace=ws)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        flops = 4.0 * w.d * dilated_key_count_sum(w.L, w.s, w.r, dil) * w.B * w.Hq
        res["dilation%d" % dil] = {"ms": ms, "tflops": flops / ms / 1e9, "reach": w.s + dil * (w.r - 1) + 1}
        del ws
    return res


def bench_backward(torch, swa, w, steps=3, settle=_no_settle):
    """Backward (dq, dk, dv) of the main workload's rows for a random upstream
    gradient.  Algorithmic flops: 10 d per (query, key) pair of the key set
    (scores, dout.v, and the dq, dk, dv products); the kernels execute 14 d
    (the scores and dout.v twice each) on the vector units."""
    q, k, v = __import__("swa_inputs").prefill_inputs(w)
    qd, kd, vd = (to_dev(torch, x, torch.bfloat16) for x in (q, k, v))
    del q, k, v
    g = torch.Generator(device="cuda").manual_seed(11)
    dod = torch.randn(qd.shape, device="cuda", generator=g).to(torch.bfloat16)
    od = swa.prefill(qd, kd, vd, w.s, w.r)
    dq = torch.empty(qd.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(kd.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(kd.shape, dtype=torch.float32, device="cuda")
    desc = swa.make_desc(w.B, w.Hq, w.Hkv, w.d, w.s, w.r, torch.bfloat16)
    ws = torch.empty(swa._lib.swa_backward_workspace_bytes(desc, w.L), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    swa.backward(qd, kd, vd, od, dod, w.s, w.r, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    settle()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        swa.backward(qd, kd, vd, od, dod, w.s, w.r, dq=dq, dk=dk, dv=dv, workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    pairs = key_count_sum(w.L, w.s, w.r) * w.B * w.Hq
    return {"ms": ms, "tflops": 10.0 * w.d * pairs / ms / 1e9,
            "executed_fp32_tflops": 14.0 * w.d * pairs / ms / 1e9,
            "frac_fp32_vector_peak": 14.0 * w.d * pairs / ms / 1e9 / PEAK_F32_TFLOPS}


def bench_decode(torch, swa, w, steps=None, settle=_no_settle):
    si = __import__("swa_inputs")
    steps = w.steps if steps is None else steps
    hk, hv = si.decode_history(w)
    kc, vc = swa.new_cache(w.B, w.Hkv, w.d, w.s, w.r, torch.bfloat16, "cuda")
    hkd, hvd = to_dev(torch, hk, torch.bfloat16), to_dev(torch, hv, torch.bfloat16)
    del hk, hv
    swa.cache_append(hkd, hvd, kc, vc, 0, w.s, w.r)
    torch.cuda.synchronize()
    del hkd, hvd
    qs, ks, vs = si.decode_steps(w, steps=steps)
    qd, kd, vd = (to_dev(torch, x, torch.bfloat16) for x in (qs, ks, vs))
    del qs, ks, vs
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    desc = swa.make_desc(w.B, w.Hq, w.Hkv, w.d, w.s, w.r, torch.bfloat16)
    ws = torch.empty(swa.decode_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    kn = [kd[i].unsqueeze(2) for i in range(steps)]
    vn = [vd[i].unsqueeze(2) for i in range(steps)]
    # warm-up on a copy of the cache state would change T; run 8 steps on a
    # scratch cache instead
    kc2, vc2 = kc.clone(), vc.clone()
    for i in range(8):
        swa.cache_append(kn[i], vn[i], kc2, vc2, w.L + i, w.s, w.r)
        swa.decode(qd[i], kc2, vc2, w.L + i + 1, w.s, w.r, out=out, workspace=ws)
    torch.cuda.synchronize()
    del kc2, vc2
    settle()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # the same steps as separate append and decode launches, on a copy of
    # the cache (for comparison; not the reported step time)
    kc3, vc3 = kc.clone(), vc.clone()
    t0.record(stream)
    for i in range(steps):
        T = w.L + i + 1
        swa.cache_append(kn[i], vn[i], kc3, vc3, T - 1, w.s, w.r)
        swa.decode(qd[i], kc3, vc3, T, w.s, w.r, out=out, workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_separate = t0.elapsed_time(t1) / steps
    del kc3, vc3
    knd = [kd[i] for i in range(steps)]
    vnd = [vd[i] for i in range(steps)]
    t0.record(stream)
    for i in range(steps):
        swa.decode_step(qd[i], knd[i], vnd[i], kc, vc, w.L + i + 1, w.s, w.r, out=out, workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    # the streaming generation step with RoPE re-positioning (pre-rotation
    # cache): more fused steps on the same cache, rope_base 1e4
    nr = min(256, steps)
    t0.record(stream)
    for i in range(nr):
        swa.decode_step(qd[i], knd[i], vnd[i], kc, vc, w.L + steps + i + 1, w.s, w.r, rope_base=1e4, out=out,
                        workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_rope = t0.elapsed_time(t1) / nr
    # the decode launch alone: back-to-back launches at the last step's T
    nd = min(64, steps)
    t0.record(stream)
    for i in range(nd):
        swa.decode(qd[steps - 1], kc, vc, w.L + steps + nr, w.s, w.r, out=out, workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    decode_ms = t0.elapsed_time(t1) / nd
    S = w.s + w.r
    kv = w.B * w.Hkv * S * w.d * 2 * 2
    qo = 2 * w.B * w.Hq * w.d * 2
    app = w.B * w.Hkv * w.d * 2 * 2
    step_bytes = kv + qo + app
    return {"ms": ms, "ms_separate": ms_separate, "ms_rope": ms_rope, "rope_steps": nr, "decode_ms": decode_ms, "bytes_per_step": step_bytes, "steps": steps,
            "gbs": step_bytes / ms / 1e6, "decode_kernel_bytes": kv + qo}


def bench_chunked(torch, swa, w, reps=2, settle=_no_settle):
    si = __import__("swa_inputs")
    q, k, v = si.chunk_inputs(w, 0, w.L)
    qd, kd, vd = (to_dev(torch, x, torch.bfloat16) for x in (q, k, v))
    del q, k, v
    C = w.chunk
    chunks = [(p0, min(w.L, p0 + C)) for p0 in range(0, w.L, C)]
    parts = [tuple(x[:, :, a:b].contiguous() for x in (qd, kd, vd)) for a, b in chunks]
    out = torch.empty_like(qd[:, :, :C])
    desc = swa.make_desc(w.B, w.Hq, w.Hkv, w.d, w.s, w.r, torch.bfloat16, rope_base=w.rope_base)
    ws = torch.empty(max(16, swa.prefill_workspace_bytes(desc, C)), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def one_pass(timer=None):
        kc, vc = swa.new_cache(w.B, w.Hkv, w.d, w.s, w.r, torch.bfloat16, "cuda")
        for (a, b), (qc, kk, vv) in zip(chunks, parts):
            o = out[:, :, :b - a]
            if timer is not None:
                with timer:
                    swa.prefill(qc, kk, vv, w.s, w.r, rope_base=w.rope_base, k_cache=kc if a else None,
                                v_cache=vc if a else None, pos0=a, out=o, workspace=ws)
            else:
                swa.prefill(qc, kk, vv, w.s, w.r, rope_base=w.rope_base, k_cache=kc if a else None,
                            v_cache=vc if a else None, pos0=a, out=o, workspace=ws)
            swa.cache_append(kk, vv, kc, vc, a, w.s, w.r)

    one_pass()
    torch.cuda.synchronize()
    settle()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        one_pass()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    # per-call prefill durations from an extra, untimed pass (events around
    # each call slow the pass they sit in)
    timer = LaunchTimer(torch, stream)
    one_pass(timer)
    torch.cuda.synchronize()
    flops = 4.0 * w.d * key_count_sum(w.L, w.s, w.r) * w.B * w.Hq
    return {"ms": ms, "flops": flops, "tflops": flops / ms / 1e9, "prefill_call_ms": timer.mean_ms()}


def bench_decode_window_sweep(torch, swa, w, slots=(1024, 2048, 4096, 8192, 32768), settle=_no_settle):
    """Decode launch time against the cache size, on the decode workload's
    shape (B sequences, GQA, d, s sinks): caches of s + r slots for several
    r, the largest being full attention over a 32768-token context.  Time
    and KV bytes scale with the slots; the cache of a 4096-token window is
    8x smaller than the full cache at 32K context.  Random bf16 caches (the
    decode reads every valid slot; the values do not change the work)."""
    out_res = {}
    g = torch.Generator(device="cuda").manual_seed(11)
    q = torch.randn((w.B, w.Hq, w.d), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    for S in slots:
        r = S - w.s
        kc = torch.randn((w.B, w.Hkv, S, w.d), generator=g, device="cuda").to(torch.bfloat16)
        vc = torch.randn((w.B, w.Hkv, S, w.d), generator=g, device="cuda").to(torch.bfloat16)
        desc = swa.make_desc(w.B, w.Hq, w.Hkv, w.d, w.s, r, torch.bfloat16)
        ws = torch.empty(max(16, swa.decode_workspace_bytes(desc)), dtype=torch.uint8, device="cuda")
        T = S + 100                                      # every slot valid
        for _ in range(3):
            swa.decode(q, kc, vc, T, w.s, r, out=out, workspace=ws)
        settle()
        n = 32
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(n):
            swa.decode(q, kc, vc, T, w.s, r, out=out, workspace=ws)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / n
        kv = w.B * w.Hkv * S * w.d * 2 * 2
        out_res["slots%d" % S] = {"us": ms * 1e3, "kv_bytes": kv, "GB/s": (kv + 2 * w.B * w.Hq * w.d * 2) / ms / 1e6,
                                  "full_attention_32k": S == 32768}
        del kc, vc, ws
        torch.cuda.empty_cache()
    return out_res


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle, as it stands, on random rows of the main workload."""
    import oracle
    import swa_inputs as si
    q, k, v = si.prefill_inputs(w)
    g = np.random.default_rng(99)
    done_rows, done_keys, elapsed = 0, 0, 0.0
    batch = 512
    while elapsed < budget_s:
        rows = np.stack([g.integers(0, w.B, batch), g.integers(0, w.Hq, batch), g.integers(0, w.L, batch)], axis=1)
        t0 = time.perf_counter()
        _, nk = oracle.prefill_rows(q, k, v, w.s, w.r, rows=rows, return_nkeys=True)
        elapsed += time.perf_counter() - t0
        done_rows += batch
        done_keys += int(nk.sum())
        batch = min(batch * 2, 16384)
    flops = 4.0 * w.d * done_keys
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "%d random query rows of %s (%d keys), fp64, %.1f s" % (done_rows, w.name, done_keys, elapsed),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


def cpu_model() -> str:
    """The host CPU's model name (first entry of /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-main", action="store_true", help="time the main workload only")
    ap.add_argument("--extra", default="3,4,5,6,7,8,9,1",
                    help="other workloads to time alongside (comma list of 1,3,4,5, 6 = window sweep of the "
                         "main workload, 7 = its dilated-window prefill, 8 = decode against the cache size, "
                         "9 = the main workload's backward, or 'none')")
    ap.add_argument("--decode-steps", type=int, default=None, help="decode steps (default: the workload's 1024)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed back-to-back main-kernel launches before each timed region, in ms (0: none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 1 GiB device copies (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sliding_window_attention_sink_amd as swa
    import swa_inputs as si

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    swa.load()

    if args.copy_calibration:
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE per dispatch of
        # this kernel are the counters' reading for 1 GiB read + 1 GiB written
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 2, "dispatches": 3}))
        return

    w = si.WORKLOADS[2]
    log("main workload", w.name)
    settle = Settler(torch, swa, w, args.settle_ms) if args.settle_ms > 0 else _no_settle
    main_res = bench_prefill(torch, swa, w, args.steps, args.warmup, settle)
    log("main", main_res)

    extra = {}
    todo = set() if (args.only_main or args.extra == "none") else {int(x) for x in args.extra.split(",") if x}
    if 3 in todo:
        w3 = si.WORKLOADS[3]
        r3 = bench_prefill(torch, swa, w3, max(5, args.steps // 2), 2, settle)
        extra[w3.name] = {"tflops": r3["tflops"], "ms": r3["ms"], "kernel_ms": r3["kernel_ms"],
                          "frac_bf16_peak": r3["tflops"] / PEAK_BF16_TFLOPS}
        log("w3", r3)
        torch.cuda.empty_cache()
    if 4 in todo:
        w4 = si.WORKLOADS[4]
        r4 = bench_decode(torch, swa, w4, args.decode_steps, settle)
        dec_gbs = r4["decode_kernel_bytes"] / r4["decode_ms"] / 1e6
        extra[w4.name] = {"GB/s": r4["gbs"], "us_per_step": r4["ms"] * 1e3, "steps": r4["steps"],
                          "us_per_step_separate_append_decode": r4["ms_separate"] * 1e3,
                          "rope1e4_us_per_step": r4["ms_rope"] * 1e3, "rope1e4_steps": r4["rope_steps"],
                          "rope1e4_GB/s": r4["bytes_per_step"] / r4["ms_rope"] / 1e6,
                          "bytes_per_step": r4["bytes_per_step"], "frac_hbm_peak": r4["gbs"] / PEAK_HBM_GBS,
                          "decode_launch_us": r4["decode_ms"] * 1e3, "decode_launch_GB/s": dec_gbs,
                          "decode_launch_frac_hbm_peak": dec_gbs / PEAK_HBM_GBS}
        log("w4", r4)
        torch.cuda.empty_cache()
    if 5 in todo:
        w5 = si.WORKLOADS[5]
        r5 = bench_chunked(torch, swa, w5, settle=settle)
        extra[w5.name] = {"tflops": r5["tflops"], "ms": r5["ms"], "frac_bf16_peak": r5["tflops"] / PEAK_BF16_TFLOPS,
                          "prefill_call_ms": r5["prefill_call_ms"]}
        log("w5", r5)
        torch.cuda.empty_cache()
    if 6 in todo:
        # window sweep on the main workload's tensors, to the full-attention limit
        extra["window_sweep_" + w.name] = bench_window_sweep(torch, swa, w, [512, 1024, 2048, 4096, 8192], settle=settle)
        torch.cuda.empty_cache()
    if 7 in todo:
        extra["dilated_" + w.name] = bench_dilated(torch, swa, w, [2, 4], settle=settle)
        torch.cuda.empty_cache()
    if 8 in todo:
        w4 = si.WORKLOADS[4]
        extra["decode_window_sweep_" + w4.name] = bench_decode_window_sweep(torch, swa, w4, settle=settle)
        torch.cuda.empty_cache()
    if 9 in todo:
        extra["backward_" + w.name] = bench_backward(torch, swa, w, settle=settle)
        log("backward", extra["backward_" + w.name])
        torch.cuda.empty_cache()
    if 1 in todo:
        w1 = si.WORKLOADS[1]
        r1 = bench_prefill(torch, swa, w1, 20, 3, settle)
        extra[w1.name] = {"tflops": r1["tflops"], "ms": r1["ms"], "frac_f32_peak": r1["tflops"] / PEAK_F32_TFLOPS}

    if todo:
        # the same measurement from a cold start: after an idle second, no
        # settle phase (the clock is still ramping during these launches)
        time.sleep(1.0)
        rc = bench_prefill(torch, swa, w, args.steps, args.warmup)
        extra["main_cold_start"] = {"ms": rc["ms"], "tflops": rc["tflops"], "frac_bf16_peak": rc["tflops"] / PEAK_BF16_TFLOPS}
        log("main cold", rc)

    achieved = main_res["flops"] / main_res["kernel_ms"] / 1e9
    sclk = recorded_sclk()
    line = {
        "metric": "SWA+sink prefill TFLOP/s and decode KV GB/s, % of roofline, 1 MI355X",
        "value": main_res["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "L": w.L, "s": w.s, "r": w.r,
                   "global_batch": w.B, "seq_len": w.L, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": MAIN_KERNEL, "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": recorded_traffic(), "mfma_busy_frac": recorded_mfma_busy(),
                     "sclk_ghz_observed": sclk,
                     "frac_at_observed_sclk": (achieved / (PEAK_BF16_TFLOPS * sclk / 2.4)) if sclk else None},
        "settle_ms": args.settle_ms,
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
