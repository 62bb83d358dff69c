#!/usr/bin/env python3
"""Throughput of sliding-window attention with sinks on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--only W]

One step = the chunked streaming prefill of 131072 tokens (B=1, H=32, d=128,
s=4 sinks + r=4092 recent, RoPE base 1e4, bf16) in 32 chunks of 4096: per
chunk the keys are rotated once at their positions (swa_rope_keys), the
chunk attends the rolling cache plus itself (swa_prefill, queries rotated in
the kernel) and is appended to the cache (swa_cache_append).  Inputs are
resident in HBM.  The JSON line's value is the step's algorithmic TFLOP/s:
only the (query, key) pairs of the sink + window key set count, 4*d flops
each; the rotations and appends are timed but not credited.

Alongside it every other workload is timed with its own roofline block
("rooflines"): the GQA Mistral-style prefill (B=1, Hq=32, Hkv=8, L=8192,
s=0, r=4096), the StreamingLLM 4+1020 prefill (B=4, H=32, L=16384), the
rolling-buffer decode loop (B=64, 32/8 heads, 4+4092 slots) and the
backward on the GQA prefill's shape; "extra" holds window sweeps, the
dilated window and the small fp32 case.  The "cpu_baseline" leg times the
fp64 oracle on a bounded sample of the main workload's rows.

Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
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

MAIN_WID = 5
CSRC = os.path.join(ROOT, "sliding_window_attention_sink_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# Sources each kernel family is built from: a counter note is valid only
# while they hash to the value recorded in it.
KERNEL_SOURCES = {
    "prefill_pp_kernel": ["prefill_bf16.hip", "prefill_common.h", "rope_common.h", "swa_internal.h"],
    "decode_split_kernel": ["decode.hip", "rope_common.h", "swa_internal.h"],
    "backward": ["backward.hip", "backward_internal.h"],
}


def _code_only(text: str) -> str:
    """A source's code with comments and blank space removed, so a note
    stays valid across edits of the comments alone."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_sources_sha256(family: str = "prefill_pp_kernel") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def note_path(family: str, workload: str, kind: str) -> str:
    """profiles/<kernel>_<workload>_<kind>.md (kind: traffic, mfma, sclk)."""
    return os.path.join(PROFILES, "%s_%s_%s.md" % (family, workload, kind))


def recorded(family: str, workload: str, kind: str, key: str):
    """A figure from a counter note (`key: value` line), or None if the note
    is absent or was taken on other kernel sources."""
    try:
        text = open(note_path(family, workload, kind)).read()
    except OSError:
        return None
    m_v = re.search(r"^%s:\s*([0-9.eE+-]+)\s*$" % re.escape(key), text, re.M)
    m_h = re.search(r"^kernel_sources_sha256:\s*([0-9a-f]{64})\s*$", text, re.M)
    if not (m_v and m_h) or m_h.group(1) != kernel_sources_sha256(family):
        return None
    return float(m_v.group(1))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def key_count_sum(L: int, s: int, r: int, pos0: int = 0) -> int:
    """sum over query rows t = pos0 .. pos0+L-1 of |U(t)| = min(t+1, s+r)."""
    t = np.arange(pos0, pos0 + L, dtype=np.int64)
    return int(np.minimum(t + 1, s + r).sum())


def prefill_flops(w) -> float:
    return 4.0 * w.d * key_count_sum(w.L, w.s, w.r) * w.B * w.Hq


def chunk_flops(w, p0: int, p1: int) -> float:
    return 4.0 * w.d * key_count_sum(p1 - p0, w.s, w.r, p0) * w.B * w.Hq


def mfma_roofline(kernel: str, family: str, workload: str, flops: float, ms: float) -> dict:
    """Roofline block of an MFMA-bound kernel: algorithmic flops per launch
    over its mean launch duration, against the dense bf16 peak, with the
    counter notes' traffic (bytes per launch) and MFMA busy fraction."""
    ach = flops / ms / 1e9
    return {"bound": "mfma", "kernel": kernel, "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS, "flops_per_launch": flops, "launch_ms": ms,
            "traffic": recorded(family, workload, "traffic", "traffic_bytes_per_launch"),
            "mfma_busy_frac": recorded(family, workload, "mfma", "mfma_busy_frac")}


SETTLE_MS = 150.0


class Settler:
    """Brings the GPU clock to its loaded level before a timed region.

    After an idle spell (here: staging each workload's inputs on the CPU) the
    graphics clock ramps up over the first ~20-50 ms of load.  Each timed
    region is therefore preceded by SETTLE_MS of back-to-back launches of the
    prefill kernel on random tensors of the GQA workload's shape (untimed;
    the steady-state rate is what the metric asks for, and a cold-start rate
    is reported beside it)."""

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


def events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_launches(torch, fn, n):
    """Mean duration (ms) of n back-to-back calls, from two HIP events on the
    current stream around all of them (an event between launches would add
    a cache flush and a stall to each)."""
    stream = torch.cuda.current_stream()
    t0, t1 = events(torch)
    t0.record(stream)
    for _ in range(n):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n


def bench_prefill(torch, swa, w, steps, warmup, settle=_no_settle):
    q, k, v = __import__("swa_inputs").prefill_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = to_dev(torch, q, dt), to_dev(torch, k, dt), to_dev(torch, v, dt)
    del q, k, v
    out = torch.empty_like(qd)
    settle()
    for _ in range(warmup):
        swa.prefill(qd, kd, vd, w.s, w.r, out=out)
    torch.cuda.synchronize()
    # one call is one launch of the kernel, so this is its mean launch duration
    ms = time_launches(torch, lambda: swa.prefill(qd, kd, vd, w.s, w.r, out=out), steps)
    flops = prefill_flops(w)
    return {"ms": ms, "flops": flops, "tflops": flops / ms / 1e9}


def bench_chunked(torch, swa, w, steps, warmup, settle=_no_settle, keep_host=False):
    """The main step: 32 chunks, each = key rotation + attention with the
    append fused in (swa_prefill_append: chunk i reads cache pair i % 2 and
    writes the cache after it to pair (i + 1) % 2; chunks are 4096 >= r
    tokens).  Also the same step with the separate append launch.

    Returns the step times and the launch durations on a chunk with a full
    cache (back-to-back launches of one chunk's call, the same inputs each
    time): the fused attention launch, the plain attention launch, the
    rotation and the separate append."""
    si = __import__("swa_inputs")
    q, k, v = si.chunk_inputs(w, 0, w.L)
    qd, kd, vd = (to_dev(torch, x, torch.bfloat16) for x in (q, k, v))
    host = (q, k, v) if keep_host else None
    del q, k, v
    C = w.chunk
    assert C >= w.r, "the fused append needs chunks of at least r tokens"
    chunks = [(p0, min(w.L, p0 + C)) for p0 in range(0, w.L, C)]
    parts = [tuple(x[:, :, a:b].contiguous() for x in (qd, kd, vd)) for a, b in chunks]
    del qd, kd, vd
    krot = torch.empty_like(parts[0][1])
    out = torch.empty_like(parts[0][0])
    base = w.rope_base
    pairs = [swa.new_cache(w.B, w.Hkv, w.d, w.s, w.r, torch.bfloat16, "cuda") for _ in range(2)]

    def run_chunk(i):
        (a, b), (qc, kk, vv) = chunks[i], parts[i]
        kr = krot[:, :, :b - a]
        kc, vc = pairs[i % 2]
        kx, vx = pairs[(i + 1) % 2]
        swa.rope_keys(kk, a, base, out=kr)
        swa.prefill_append(qc, kr, vv, w.s, w.r, kx, vx, rope_base=base, k_cache=kc if a else None,
                           v_cache=vc if a else None, pos0=a, out=out[:, :, :b - a])

    def run_chunk_separate(kc, vc, i):
        (a, b), (qc, kk, vv) = chunks[i], parts[i]
        kr = krot[:, :, :b - a]
        swa.rope_keys(kk, a, base, out=kr)
        swa.prefill(qc, kr, vv, w.s, w.r, rope_base=base, k_cache=kc if a else None, v_cache=vc if a else None,
                    pos0=a, out=out[:, :, :b - a])
        swa.cache_append(kr, vv, kc, vc, a, w.s, w.r)

    # chunk 0 reads no cache, and each later chunk reads only the pair its
    # predecessor in the same pass wrote
    def one_pass():
        for i in range(len(chunks)):
            run_chunk(i)

    kc0, vc0 = swa.new_cache(w.B, w.Hkv, w.d, w.s, w.r, torch.bfloat16, "cuda")

    def one_pass_separate():
        for i in range(len(chunks)):
            run_chunk_separate(kc0, vc0, i)

    for _ in range(max(1, warmup)):
        one_pass()
        one_pass_separate()
    torch.cuda.synchronize()
    settle()
    ms = time_launches(torch, one_pass, steps)
    settle()
    ms_sep = time_launches(torch, one_pass_separate, steps)
    flops = chunk_flops(w, 0, w.L)

    # each call on its own, on the chunk after a full cache: the cache state
    # after chunk m-1, then back-to-back launches of chunk m's calls
    m = len(chunks) // 2
    kc, vc = swa.new_cache(w.B, w.Hkv, w.d, w.s, w.r, torch.bfloat16, "cuda")
    for i in range(m):
        run_chunk_separate(kc, vc, i)
    (a, b), (qc, kk, vv) = chunks[m], parts[m]
    swa.rope_keys(kk, a, base, out=krot)
    kx, vx = pairs[0]
    torch.cuda.synchronize()
    settle()
    n = 20
    # (the fused launches last: the counter notes take the leg's last 20
    # launches of the attention kernel)
    attn_ms = time_launches(torch, lambda: swa.prefill(qc, krot, vv, w.s, w.r, rope_base=base, k_cache=kc,
                                                       v_cache=vc, pos0=a, out=out), n)
    fused_ms = time_launches(torch, lambda: swa.prefill_append(qc, krot, vv, w.s, w.r, kx, vx, rope_base=base,
                                                               k_cache=kc, v_cache=vc, pos0=a, out=out), n)
    rot_ms = time_launches(torch, lambda: swa.rope_keys(kk, a, base, out=krot), n)
    kc2, vc2 = kc.clone(), vc.clone()
    app_ms = time_launches(torch, lambda: swa.cache_append(krot, vv, kc2, vc2, a, w.s, w.r), n)
    del kc2, vc2
    cflops = chunk_flops(w, a, b)
    res = {"ms": ms, "flops": flops, "tflops": flops / ms / 1e9, "chunk_flops": cflops,
           "ms_separate_append": ms_sep, "tflops_separate_append": flops / ms_sep / 1e9,
           "fused_launch_ms": fused_ms, "attn_launch_ms": attn_ms, "rope_keys_ms": rot_ms, "append_ms": app_ms,
           "fused_tflops": cflops / fused_ms / 1e9, "attn_tflops": cflops / attn_ms / 1e9}
    # share of the step outside the attention launches, from the per-call times
    c0 = chunk_flops(w, *chunks[0])
    attn_total = fused_ms * (len(chunks) - 1 + c0 / cflops)
    res["non_attention_share"] = max(0.0, 1.0 - attn_total / ms)
    return res, host


def bench_window_sweep(torch, swa, w, windows, steps=10, settle=_no_settle):
    """Prefill of the GQA workload's tensors at several window sizes r (s as
    given), up to r >= L, i.e. full causal attention: time and cache size."""
    q, k, v = __import__("swa_inputs").prefill_inputs(w)
    qd, kd, vd = (to_dev(torch, x, torch.bfloat16) for x in (q, k, v))
    del q, k, v
    out = torch.empty_like(qd)
    res = {}
    settle()
    for r in windows:
        for _ in range(2):
            swa.prefill(qd, kd, vd, w.s, r, out=out)
        torch.cuda.synchronize()
        ms = time_launches(torch, lambda: swa.prefill(qd, kd, vd, w.s, r, out=out), steps)
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
    """Dilated-window prefill of a workload's tensors (read and written in
    place, no workspace), algorithmic TFLOP/s."""
    q, k, v = __import__("swa_inputs").prefill_inputs(w)
    qd, kd, vd = (to_dev(torch, x, torch.bfloat16) for x in (q, k, v))
    del q, k, v
    out = torch.empty_like(qd)
    desc = swa.make_desc(w.B, w.Hq, w.Hkv, w.d, w.s, w.r, torch.bfloat16)
    res = {}
    settle()
    for dil in dilations:
        assert swa._lib.swa_prefill_dilated_workspace_bytes(desc, w.L, dil) == 0
        for _ in range(2):
            swa.prefill_dilated(qd, kd, vd, w.s, w.r, dil, out=out)
        torch.cuda.synchronize()
        ms = time_launches(torch, lambda: swa.prefill_dilated(qd, kd, vd, w.s, w.r, dil, out=out), steps)
        flops = 4.0 * w.d * dilated_key_count_sum(w.L, w.s, w.r, dil) * w.B * w.Hq
        res["dilation%d" % dil] = {"ms": ms, "tflops": flops / ms / 1e9, "reach": w.s + dil * (w.r - 1) + 1}
    return res


def global_key_count_sum(L: int, s: int, r: int, G) -> int:
    """sum over rows of |U_G(t)|: a global row t has t + 1 keys, any other row
    min(t+1, s+r) plus the global positions in [s, t-r+1) that are <= t."""
    t = np.arange(L, dtype=np.int64)
    n = np.minimum(t + 1, s + r)
    gs = np.asarray(G, dtype=np.int64)
    lo = np.maximum(s, t - r + 1)
    extra = ((gs[None, :] >= s) & (gs[None, :] < lo[:, None]) & (gs[None, :] <= t[:, None])).sum(axis=1)
    n = n + extra
    n[gs] = gs + 1
    return int(n.sum())


def bench_global(torch, swa, w, G, steps=10, settle=_no_settle):
    """Prefill with task-bound global tokens at positions G on a prefill
    workload's tensors: the gather of the global keys, the banded pass with
    them as one more key tile, and the dense global rows; algorithmic TFLOP/s
    of the key sets."""
    q, k, v = __import__("swa_inputs").prefill_inputs(w)
    qd, kd, vd = (to_dev(torch, x, torch.bfloat16) for x in (q, k, v))
    del q, k, v
    out = torch.empty_like(qd)
    desc = swa.make_desc(w.B, w.Hq, w.Hkv, w.d, w.s, w.r, torch.bfloat16)
    ws = torch.empty(swa._lib.swa_prefill_global_workspace_bytes(desc, w.L, len(G)), dtype=torch.uint8,
                     device="cuda")
    call = lambda: swa.prefill_global(qd, kd, vd, w.s, w.r, G, out=out, workspace=ws)
    call()
    torch.cuda.synchronize()
    settle()
    ms = time_launches(torch, call, steps)
    flops = 4.0 * w.d * global_key_count_sum(w.L, w.s, w.r, G) * w.B * w.Hq
    plain = prefill_flops(w)
    return {"ms": ms, "tflops": flops / ms / 1e9, "globals": list(G), "flops": flops,
            "extra_flops_over_window": flops - plain}


def backward_flops(w) -> float:
    """Algorithmic flops of the backward: 10 d per (query, key) pair of the key
    set (the scores, dout . v, and the dq, dk and dv products, 2 d each)."""
    return 10.0 * w.d * key_count_sum(w.L, w.s, w.r) * w.B * w.Hq


def bench_backward(torch, swa, w, steps=5, settle=_no_settle):
    """Backward (dq, dk, dv) of a prefill workload's rows for a random upstream
    gradient, against the bf16 MFMA peak at 10 d flops per pair."""
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
    ws = torch.empty(max(16, swa._lib.swa_backward_workspace_bytes(desc, w.L)), dtype=torch.uint8, device="cuda")
    call = lambda: swa.backward(qd, kd, vd, od, dod, w.s, w.r, dq=dq, dk=dk, dv=dv, workspace=ws)
    call()
    torch.cuda.synchronize()
    settle()
    ms = time_launches(torch, call, steps)
    flops = backward_flops(w)
    return {"ms": ms, "flops": flops, "tflops": flops / ms / 1e9}


def decode_step_bytes(w) -> int:
    """Algorithmic bytes of one decode step: K/V of every valid slot (all s + r
    once the cache is full), q, o and the appended token's K/V."""
    S = w.s + w.r
    return w.B * w.Hkv * S * w.d * 2 * 2 + 2 * w.B * w.Hq * w.d * 2 + w.B * w.Hkv * w.d * 2 * 2


def bench_decode(torch, swa, w, steps=None, settle=_no_settle):
    si = __import__("swa_inputs")
    steps = w.steps if steps is None else steps
    hk, hv = si.decode_history(w)
    kc, vc = swa.new_cache(w.B, w.Hkv, w.d, w.s, w.r, torch.bfloat16, "cuda")
    hkd, hvd = to_dev(torch, hk, torch.bfloat16), to_dev(torch, hv, torch.bfloat16)
    del hk, hv
    swa.cache_append(hkd, hvd, kc, vc, 0, w.s, w.r)
    # the RoPE cache: the same history with every key rotated at its position
    kcr, vcr = swa.new_cache(w.B, w.Hkv, w.d, w.s, w.r, torch.bfloat16, "cuda")
    swa.cache_append(swa.rope_keys(hkd, 0, 1e4), hvd, kcr, vcr, 0, w.s, w.r)
    torch.cuda.synchronize()
    del hkd, hvd
    qs, ks, vs = si.decode_steps(w, steps=steps)
    qd, kd, vd = (to_dev(torch, x, torch.bfloat16) for x in (qs, ks, vs))
    del qs, ks, vs
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    desc = swa.make_desc(w.B, w.Hq, w.Hkv, w.d, w.s, w.r, torch.bfloat16)
    ws = torch.empty(max(16, swa.decode_workspace_bytes(desc)), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    kn = [kd[i].unsqueeze(2) for i in range(steps)]
    vn = [vd[i].unsqueeze(2) for i in range(steps)]
    # warm-up on a scratch copy of the cache (8 steps)
    kc2, vc2 = kc.clone(), vc.clone()
    for i in range(8):
        swa.cache_append(kn[i], vn[i], kc2, vc2, w.L + i, w.s, w.r)
        swa.decode(qd[i], kc2, vc2, w.L + i + 1, w.s, w.r, out=out, workspace=ws)
    torch.cuda.synchronize()
    del kc2, vc2
    settle()
    t0, t1 = events(torch)
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
    # the streaming generation step with RoPE re-positioning, rope_base 1e4,
    # on the RoPE cache: step keys rotated at their positions beforehand (the
    # form the library takes keys in), then fused steps
    nr = min(256, steps)
    knr = [swa.rope_keys(kd[i].unsqueeze(2), w.L + i, 1e4)[:, :, 0] for i in range(nr)]
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(nr):
        swa.decode_step(qd[i], knr[i], vnd[i], kcr, vcr, w.L + i + 1, w.s, w.r, rope_base=1e4, out=out,
                        workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_rope = t0.elapsed_time(t1) / nr
    # the decode launch alone: back-to-back launches at the last step's T
    decode_ms = time_launches(torch, lambda: swa.decode(qd[steps - 1], kc, vc, w.L + steps, w.s, w.r, out=out,
                                                        workspace=ws), min(64, steps))
    step_bytes = decode_step_bytes(w)
    kernel_bytes = step_bytes - w.B * w.Hkv * w.d * 2 * 2
    return {"ms": ms, "ms_separate": ms_separate, "ms_rope": ms_rope, "rope_steps": nr, "decode_ms": decode_ms,
            "bytes_per_step": step_bytes, "steps": steps, "gbs": step_bytes / ms / 1e6,
            "decode_kernel_bytes": kernel_bytes}


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
        ms = time_launches(torch, lambda: swa.decode(q, kc, vc, T, w.s, r, out=out, workspace=ws), 32)
        kv = w.B * w.Hkv * S * w.d * 2 * 2
        out_res["slots%d" % S] = {"us": ms * 1e3, "kv_bytes": kv, "GB/s": (kv + 2 * w.B * w.Hq * w.d * 2) / ms / 1e6,
                                  "full_attention_32k": S == 32768}
        del kc, vc, ws
        torch.cuda.empty_cache()
    return out_res


def cpu_baseline(w, budget_s: float, host=None):
    """The fp64 oracle, as it stands, on random query rows of the main
    (chunked, RoPE) workload, over the whole token history."""
    import oracle
    import swa_inputs as si
    q, k, v = host if host is not None else si.chunk_inputs(w, 0, w.L)
    g = np.random.default_rng(99)
    done_rows, done_keys, elapsed = 0, 0, 0.0
    batch = 64
    while elapsed < budget_s:
        rows = np.stack([g.integers(0, w.B, batch), g.integers(0, w.Hq, batch), g.integers(0, w.L, batch)], axis=1)
        t0 = time.perf_counter()
        _, nk = oracle.prefill_rows(q, k, v, w.s, w.r, rope_base=w.rope_base, rows=rows, return_nkeys=True)
        elapsed += time.perf_counter() - t0
        done_rows += batch
        done_keys += int(nk.sum())
        batch = min(batch * 2, 4096)
    flops = 4.0 * w.d * done_keys
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "%d random query rows of %s (%d keys, RoPE by rank), fp64, %.1f s"
                      % (done_rows, w.name, done_keys, elapsed),
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
    ap.add_argument("--steps", type=int, default=10, help="timed passes of the main step")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="time only these legs (comma list: 5 = the main chunked step, 2, 3 = prefill "
                         "workloads, 4 = decode, 9 = backward, 10 = global tokens, 6, 7, 8, 1 = sweeps / "
                         "dilated / fp32)")
    ap.add_argument("--decode-steps", type=int, default=None, help="decode steps (default: the workload's 1024)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed back-to-back prefill launches before each timed region, in ms (0: none)")
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

    todo = {5, 2, 3, 4, 9, 10, 6, 7, 8, 1} if args.only is None else {int(x) for x in args.only.split(",") if x}
    w2 = si.WORKLOADS[2]
    settle = Settler(torch, swa, w2, args.settle_ms) if args.settle_ms > 0 else _no_settle
    rooflines, extra = {}, {}
    w = si.WORKLOADS[MAIN_WID]
    main_res, host = None, None
    if 5 in todo:
        log("main workload", w.name)
        want_host = not args.no_cpu_baseline
        main_res, host = bench_chunked(torch, swa, w, args.steps, args.warmup, settle, keep_host=want_host)
        # the dominant kernel of the step: the attention launch with the
        # append fused in
        rooflines[w.name] = mfma_roofline("prefill_pp_kernel<128, false, true>", "prefill_pp_kernel", w.name,
                                          main_res["chunk_flops"], main_res["fused_launch_ms"])
        log("main", main_res)
        torch.cuda.empty_cache()
    for wid in (2, 3):
        if wid in todo:
            wk = si.WORKLOADS[wid]
            rk = bench_prefill(torch, swa, wk, max(10, args.steps), 3, settle)
            rooflines[wk.name] = mfma_roofline("prefill_pp_kernel<128, false, false>", "prefill_pp_kernel", wk.name,
                                               rk["flops"], rk["ms"])
            log("w%d" % wid, rk)
            torch.cuda.empty_cache()
    if 4 in todo:
        w4 = si.WORKLOADS[4]
        r4 = bench_decode(torch, swa, w4, args.decode_steps, settle)
        dec_gbs = r4["decode_kernel_bytes"] / r4["decode_ms"] / 1e6
        rooflines[w4.name] = {"bound": "hbm", "kernel": "decode_split_kernel<128, false, false>", "achieved": dec_gbs,
                              "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": dec_gbs / PEAK_HBM_GBS,
                              "bytes_per_launch": r4["decode_kernel_bytes"], "launch_ms": r4["decode_ms"],
                              "traffic": recorded("decode_split_kernel", w4.name, "traffic",
                                                  "traffic_bytes_per_launch")}
        extra[w4.name] = {"GB/s": r4["gbs"], "us_per_step": r4["ms"] * 1e3, "steps": r4["steps"],
                          "frac_hbm_peak": r4["gbs"] / PEAK_HBM_GBS, "bytes_per_step": r4["bytes_per_step"],
                          "us_per_step_separate_append_decode": r4["ms_separate"] * 1e3,
                          "rope1e4_us_per_step": r4["ms_rope"] * 1e3, "rope1e4_steps": r4["rope_steps"],
                          "rope1e4_GB/s": r4["bytes_per_step"] / r4["ms_rope"] / 1e6}
        log("w4", r4)
        torch.cuda.empty_cache()
    if 9 in todo:
        # the backward on the GQA prefill's shape (no sinks) and on the 4+1020
        # shape (sink keys seen by every later query)
        for wb in (w2, si.WORKLOADS[3]):
            rb = bench_backward(torch, swa, wb, settle=settle)
            rooflines["backward_" + wb.name] = {
                "bound": "mfma", "kernel": "swa_backward (bwd_dq + bwd_dkdv + bwd_reduce kernels)",
                "achieved": rb["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": rb["tflops"] / PEAK_BF16_TFLOPS, "flops_per_call": rb["flops"], "call_ms": rb["ms"],
                "traffic": recorded("backward", wb.name, "traffic", "traffic_bytes_per_launch"),
                "mfma_busy_frac": recorded("backward", wb.name, "mfma", "mfma_busy_frac")}
            log("backward", wb.name, rb)
            torch.cuda.empty_cache()
    if 10 in todo:
        # task-bound global tokens on the 4+1020 workload's tensors
        w3 = si.WORKLOADS[3]
        extra["global_tokens_" + w3.name] = bench_global(torch, swa, w3, [2, 100, 2000, 2001, 7777, 12000, 12500,
                                                                          16383], settle=settle)
        log("global", extra["global_tokens_" + w3.name])
        torch.cuda.empty_cache()
    if 6 in todo:
        # window sweep on the GQA workload's tensors, to the full-attention limit
        extra["window_sweep_" + w2.name] = bench_window_sweep(torch, swa, w2, [512, 1024, 2048, 4096, 8192],
                                                              settle=settle)
        torch.cuda.empty_cache()
    if 7 in todo:
        extra["dilated_" + w2.name] = bench_dilated(torch, swa, w2, [2, 4], settle=settle)
        log("dilated", w2.name, extra["dilated_" + w2.name])
        w3 = si.WORKLOADS[3]
        extra["dilated_" + w3.name] = bench_dilated(torch, swa, w3, [2, 8], settle=settle)
        log("dilated", w3.name, extra["dilated_" + w3.name])
        torch.cuda.empty_cache()
    if 8 in todo:
        w4 = si.WORKLOADS[4]
        extra["decode_window_sweep_" + w4.name] = bench_decode_window_sweep(torch, swa, w4, settle=settle)
        torch.cuda.empty_cache()
    if 1 in todo:
        w1 = si.WORKLOADS[1]
        r1 = bench_prefill(torch, swa, w1, 20, 3, settle)
        extra[w1.name] = {"tflops": r1["tflops"], "ms": r1["ms"], "frac_f32_peak": r1["tflops"] / PEAK_F32_TFLOPS}
    if 2 in todo and 5 in todo:
        # the GQA prefill from a cold start: after an idle second, no settle
        # phase (the clock is still ramping during these launches)
        time.sleep(1.0)
        rc = bench_prefill(torch, swa, w2, max(10, args.steps), 3)
        extra["cold_start_" + w2.name] = {"ms": rc["ms"], "tflops": rc["tflops"],
                                          "frac_bf16_peak": rc["tflops"] / PEAK_BF16_TFLOPS}

    if main_res is not None:
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
            "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "L": w.L, "s": w.s,
                       "r": w.r, "chunk": w.chunk, "rope_base": w.rope_base, "global_batch": w.B,
                       "seq_len": w.L, "parallelism": "none (1 GPU)"},
            "roofline": rooflines[w.name],
            "step_breakdown": {"fused_attention_append_launch_ms": main_res["fused_launch_ms"],
                               "rope_keys_ms": main_res["rope_keys_ms"],
                               "non_attention_share": main_res["non_attention_share"],
                               "attention_only_launch_ms": main_res["attn_launch_ms"],
                               "separate_append_ms": main_res["append_ms"],
                               "step_ms_with_separate_append": main_res["ms_separate_append"],
                               "tflops_with_separate_append": main_res["tflops_separate_append"]},
            "rooflines": rooflines,
            "settle_ms": args.settle_ms,
            "extra": extra,
        }
    else:
        # a partial run (profiling some legs): their roofline blocks only
        line = {"metric": "partial run", "legs": sorted(todo), "rooflines": rooflines, "extra": extra}
    if not args.no_cpu_baseline and main_res is not None:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
