"""Seeded synthetic inputs for sliding-window attention with sinks.

This module is the one place that both the fp64 CPU oracle (``oracle/``) and
the HIP path (``sliding_window_attention_sink_amd``) draw their inputs from.
It holds workload shapes, random draws and the bf16 rounding of inputs; it
holds none of the attention arithmetic.

Recipe (every tensor, every workload):
  * one numpy ``Generator`` per slab, seeded with
    ``SeedSequence([1234, workload_id, tensor_id, b, h, block])``,
    tensor_id 0 = Q, 1 = K, 2 = V;
  * ``block`` is 0 for a plain prefill, the chunk index for chunked prefill,
    0 for the decode pre-fill history and 1 for the decode step tokens;
  * values are ``standard_normal(float32)`` times the workload's value scale,
    then rounded to bf16 with round-to-nearest-even for bf16 workloads (fp32
    workloads keep the fp32 draw).

Arrays are returned as float32 numpy arrays whose values are exactly what the
device receives (bf16-representable for bf16 workloads).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np

SEED_ROOT = 1234
TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


# --------------------------------------------------------------------------
# bf16 round-to-nearest-even (input preparation only)
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bf16 bit patterns, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    # NaN stays NaN (quiet it); the draws never produce one.
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16, returned as float32."""
    return bf16_bits_to_f32(bf16_bits(x))


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic workload.

    kind: "prefill", "decode" or "chunked".
    For "decode": L = tokens of pre-fill history, steps = decode steps.
    For "chunked": L = total tokens, chunk = tokens per chunk.
    """
    wid: int
    name: str
    kind: str
    dtype: str          # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    d: int
    L: int
    s: int
    r: int
    value_scale: float = 1.0
    sink_from_mean_q: float = 0.0   # K rows 0..s-1 := c * mean_t(Q) per head when c != 0
    rope_base: float = 0.0
    chunk: int = 0
    steps: int = 0
    check_every: int = 1            # rows checked against the oracle (chunked)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


# The five workloads: a small fp32 prefill, GQA Mistral-style window, the
# StreamingLLM 4+1020 split, rolling-buffer decode and chunked streaming
# prefill with RoPE re-positioning inside the cache.
WORKLOADS = {
    1: Workload(1, "prefill_f32_L256_s4_r28", "prefill", "f32", 1, 1, 1, 64, 256, 4, 28),
    2: Workload(2, "prefill_bf16_gqa32x8_L8192_s0_r4096", "prefill", "bf16", 1, 32, 8, 128, 8192, 0, 4096,
                value_scale=float(np.float32(1.0 / np.sqrt(2.0)))),
    3: Workload(3, "prefill_bf16_B4_H32_L16384_s4_r1020", "prefill", "bf16", 4, 32, 32, 128, 16384, 4, 1020,
                sink_from_mean_q=3.0),
    4: Workload(4, "decode_bf16_B64_gqa32x8_s4_r4092_hist8192_steps1024", "decode", "bf16", 64, 32, 8, 128,
                8192, 4, 4092, steps=1024),
    5: Workload(5, "chunked_bf16_H32_L131072_chunk4096_s4_r4092_rope1e4", "chunked", "bf16", 1, 32, 32, 128,
                131072, 4, 4092, rope_base=10000.0, chunk=4096, check_every=64),
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_slab(wid: int, tensor: int, b: int, h: int, block: int, shape, scale: float = 1.0) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence([SEED_ROOT, wid, tensor, b, h, block]))
    x = g.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def draw(wid: int, tensor: int, B: int, H: int, rows: int, d: int, *, block: int = 0,
         scale: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """[B, H, rows, d] float32 array of the workload's values for one tensor."""
    out = np.empty((B, H, rows, d), dtype=np.float32)

    def fill(bh):
        b, h = divmod(bh, H)
        x = normal_slab(wid, tensor, b, h, block, (rows, d), scale)
        out[b, h] = round_bf16(x) if dtype == "bf16" else x

    if B * H * rows * d >= (1 << 22):
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(B * H)))
    else:
        for bh in range(B * H):
            fill(bh)
    return out


def prefill_inputs(w: Workload, *, L: int | None = None, B: int | None = None):
    """Q [B,Hq,L,d], K and V [B,Hkv,L,d] for a prefill workload.

    ``L``/``B`` may shrink the workload (same seeds, leading rows/batches).
    For the sink construction the per-head mean of Q over the L rows is taken
    in fp64 on the rounded Q; with GQA the mean is over the q-heads of the
    group as well (for Hq == Hkv that is just the head).
    """
    L = w.L if L is None else L
    B = w.B if B is None else B
    q = draw(w.wid, TENSOR_Q, B, w.Hq, L, w.d, scale=w.value_scale, dtype=w.dtype)
    k = draw(w.wid, TENSOR_K, B, w.Hkv, L, w.d, scale=w.value_scale, dtype=w.dtype)
    v = draw(w.wid, TENSOR_V, B, w.Hkv, L, w.d, scale=w.value_scale, dtype=w.dtype)
    if w.sink_from_mean_q != 0.0 and w.s > 0:
        g = w.Hq // w.Hkv
        qm = q.astype(np.float64).reshape(B, w.Hkv, g, L, w.d).mean(axis=(2, 3))
        sink = (w.sink_from_mean_q * qm).astype(np.float32)
        if w.dtype == "bf16":
            sink = round_bf16(sink)
        ns = min(w.s, L)
        k[:, :, :ns, :] = sink[:, :, None, :]
    return q, k, v


def decode_history(w: Workload, *, B: int | None = None, hist: int | None = None):
    """K, V [B,Hkv,hist,d] for the tokens written before the first decode step."""
    B = w.B if B is None else B
    hist = w.L if hist is None else hist
    k = draw(w.wid, TENSOR_K, B, w.Hkv, hist, w.d, block=0, scale=w.value_scale, dtype=w.dtype)
    v = draw(w.wid, TENSOR_V, B, w.Hkv, hist, w.d, block=0, scale=w.value_scale, dtype=w.dtype)
    return k, v


def decode_steps(w: Workload, *, B: int | None = None, steps: int | None = None):
    """Step tokens: q [steps,B,Hq,d], k_new and v_new [steps,B,Hkv,d].

    Step i appends the token at position hist + i and then queries with it.
    """
    B = w.B if B is None else B
    steps = w.steps if steps is None else steps
    q = draw(w.wid, TENSOR_Q, B, w.Hq, steps, w.d, block=1, scale=w.value_scale, dtype=w.dtype)
    k = draw(w.wid, TENSOR_K, B, w.Hkv, steps, w.d, block=1, scale=w.value_scale, dtype=w.dtype)
    v = draw(w.wid, TENSOR_V, B, w.Hkv, steps, w.d, block=1, scale=w.value_scale, dtype=w.dtype)
    tr = lambda x: np.ascontiguousarray(x.transpose(2, 0, 1, 3))
    return tr(q), tr(k), tr(v)


def sequence_rows(w: Workload, tensor: int, H: int, p0: int, p1: int, *, B: int | None = None) -> np.ndarray:
    """Rows for positions p0..p1-1 of a chunked workload's token sequence.

    The sequence is drawn in blocks of ``w.chunk`` positions (block index =
    position // w.chunk), so any split of it into chunks of another size sees
    the same tokens.
    """
    B = w.B if B is None else B
    C = w.chunk
    out = np.empty((B, H, p1 - p0, w.d), dtype=np.float32)
    c0, c1 = p0 // C, (p1 - 1) // C
    for c in range(c0, c1 + 1):
        blk = draw(w.wid, tensor, B, H, C, w.d, block=c, scale=w.value_scale, dtype=w.dtype)
        a, b = max(p0, c * C), min(p1, (c + 1) * C)
        out[:, :, a - p0:b - p0] = blk[:, :, a - c * C:b - c * C]
    return out


def chunk_inputs(w: Workload, p0: int, p1: int, *, B: int | None = None):
    """Q [B,Hq,p1-p0,d], K and V [B,Hkv,p1-p0,d] for positions p0..p1-1."""
    return (sequence_rows(w, TENSOR_Q, w.Hq, p0, p1, B=B),
            sequence_rows(w, TENSOR_K, w.Hkv, p0, p1, B=B),
            sequence_rows(w, TENSOR_V, w.Hkv, p0, p1, B=B))
