"""Python side of the fp64 CPU oracle (test infrastructure only).

``swa_oracle.c`` holds the per-row attention in fp64; this module builds it
with gcc, wraps it with ctypes and adds the rolling-buffer cache simulator.

Parity unpinned: nothing here; every function has a pin in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "swa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def library_path() -> str:
    return _LIB


def build(force: bool = False) -> str:
    """Compile liboracle.so (gcc, fp64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i64, f64 = ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.swa_oracle_rows.restype = ctypes.c_int
        lib.swa_oracle_rows.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, f64, f64, i64,
                                        i64, vp, vp, vp, i64, vp, i64]
        lib.swa_oracle_attend_set.restype = ctypes.c_int
        lib.swa_oracle_attend_set.argtypes = [vp, vp, vp, i64, i64, f64, vp]
        lib.swa_oracle_rope.restype = ctypes.c_int
        lib.swa_oracle_rope.argtypes = [vp, vp, i64, i64, f64]
        lib.swa_oracle_key_set.restype = i64
        lib.swa_oracle_key_set.argtypes = [i64, i64, i64, i64, vp, i64, vp]
        lib.swa_oracle_threads.restype = ctypes.c_int
        lib.swa_oracle_threads.argtypes = []
        _lib = lib
    return _lib


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    """OpenMP threads the oracle's row loop runs on."""
    return int(_load().swa_oracle_threads())


def _globals(globals_):
    g = np.ascontiguousarray(np.zeros(0) if globals_ is None else globals_, dtype=np.int64)
    return g, (_ptr(g) if g.size else None), int(g.size)


def key_set(t: int, s: int, r: int, dilation: int = 1, globals_=None) -> np.ndarray:
    """U(t) as the oracle enumerates it (sinks, then the window; with a
    dilation the window takes every dilation-th position back from t; with
    global positions, a global row takes 0..t and other rows add the global
    positions <= t)."""
    g, gp, ng = _globals(globals_)
    buf = np.empty(max(s + r + ng, t + 1), dtype=np.int64)
    n = _load().swa_oracle_key_set(t, s, r, dilation, gp, ng, _ptr(buf))
    if n < 0:
        raise ValueError("invalid key-set arguments")
    return buf[:n].copy()


def rope(x, pos: int, base: float) -> np.ndarray:
    """Rotate vector x (fp64) to position ``pos``: pairs (j, j + d/2)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    if _load().swa_oracle_rope(_ptr(x), _ptr(y), x.shape[0], int(pos), float(base)) != 0:
        raise ValueError("invalid rope arguments")
    return y


def prefill_rows(q, k, v, s: int, r: int, *, scale: float | None = None, rope_base: float = 0.0,
                 qpos0: int = 0, rows=None, return_nkeys: bool = False, dilation: int = 1, globals_=None):
    """Attention rows over the sink + recent key set, fp64.

    ``globals_``: sorted, distinct global-token positions (plain window only):
    a row in it attends keys 0..t, any other row adds the global positions
    up to itself to U(t).

    q: [B, Hq, Lq, d] (row i at position qpos0 + i); k, v: [B, Hkv, Lk, d]
    (row p at position p).  ``rows``: int array [n, 3] of (b, h, i); None means
    every row.  Returns [n, d] fp64 (and |U(t)| per row when asked).
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, Hq, Lq, d = q.shape
    Bk, Hkv, Lk, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d:
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if rows is None:
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(Lq), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], d), dtype=np.float64)
    nk = np.empty(rows.shape[0], dtype=np.int64)
    g, gp, ng = _globals(globals_)
    rc = _load().swa_oracle_rows(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Lq, Lk, d, s, r, float(scale),
                                 float(rope_base), qpos0, rows.shape[0], _ptr(rows), _ptr(out), _ptr(nk),
                                 int(dilation), gp, ng)
    if rc != 0:
        raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
    return (out, nk) if return_nkeys else out


def chunked_rows(q, k, v, s: int, r: int, *, rope_base: float, rows, scale: float | None = None):
    """Rows of a chunked streaming prefill.  Chunking is only an execution
    schedule, so the oracle is the row definition over the whole history."""
    return prefill_rows(q, k, v, s, r, scale=scale, rope_base=rope_base, qpos0=0, rows=rows)


def attend_set(q, keys, vals, *, scale: float | None = None) -> np.ndarray:
    """Softmax attention of one query [d] over explicit rows [n, d], fp64."""
    q, keys, vals = _f32(q), _f32(keys), _f32(vals)
    n, d = keys.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty(d, dtype=np.float64)
    if _load().swa_oracle_attend_set(_ptr(q), _ptr(keys), _ptr(vals), n, d, float(scale), _ptr(out)) != 0:
        raise ValueError("invalid attend_set arguments")
    return out


class RollingCacheSim:
    """Token-by-token simulator of the sink + rolling-buffer KV cache.

    s sink slots hold tokens 0..s-1 (t6page eq:attn-fixed-streaming: the
    cache is the first k tokens plus the m most recent).  The recent tokens go
    to a rolling buffer of r slots written at slot (p mod r), overwriting the
    oldest (t6page eq:attn-fixed-rolling); with the sink slots in front that
    is slot s + (p mod r).  Tokens below s go only to their sink slot.
    """

    def __init__(self, B: int, Hkv: int, d: int, s: int, r: int):
        self.s, self.r = s, r
        self.k = np.full((B, Hkv, s + r, d), np.nan, dtype=np.float32)
        self.v = np.full((B, Hkv, s + r, d), np.nan, dtype=np.float32)
        self.pos = np.full(s + r, -1, dtype=np.int64)   # token held by each slot, -1 = never written
        self.T = 0

    def slot_of(self, p: int) -> int:
        return p if p < self.s else self.s + (p % self.r)

    def append(self, k_new, v_new, pos0: int):
        """Write tokens pos0 .. pos0+n-1 in order; k_new, v_new: [B, Hkv, n, d]."""
        n = k_new.shape[2]
        for j in range(n):
            p = pos0 + j
            sl = self.slot_of(p)
            self.k[:, :, sl] = k_new[:, :, j]
            self.v[:, :, sl] = v_new[:, :, j]
            self.pos[sl] = p
        self.T = max(self.T, pos0 + n)

    def valid_slots(self) -> np.ndarray:
        return np.nonzero(self.pos >= 0)[0]


def decode_row(cache: RollingCacheSim, q, b: int, h: int, Hq: int, *, scale: float | None = None):
    """One decode query (q-head h of batch b) over every written slot."""
    Hkv = cache.k.shape[1]
    kvh = h // (Hq // Hkv)
    sl = cache.valid_slots()
    return attend_set(q, cache.k[b, kvh, sl], cache.v[b, kvh, sl], scale=scale)


def backward(q, k, v, o, do, s: int, r: int, *, scale: float | None = None):
    """Gradients of the prefill rows with respect to q, k and v, fp64.

    The forward is row t = softmax over U(t) of scale * q_t . k_i, weighting
    v_i (hyper.ai summary, section on sliding-window attention with sinks;
    t6page eq:attn-fixed-streaming for the key set).  For an upstream
    gradient dO its derivative, written out per (batch, q-head) with the key
    set as a 0/1 mask M[t, i] = [i in U(t)]:

        P  = softmax_rows(scale * Q K^T restricted to M)
        dV = P^T dO                      (summed over the q-heads of a kv-head)
        dP = dO V^T
        D_t = sum_j dO[t, j] * O[t, j]   (O as the caller passes it)
        dS = P * (dP - D)
        dQ = scale * dS K,   dK = scale * dS^T Q   (dK summed over the group)

    ``o`` is the forward output the caller holds (the same O enters D on
    both sides); q, k, v, o, do: [B, Hq|Hkv, L, d].  Returns (dq, dk, dv) in
    fp64 with the shapes of q, k, v.
    """
    q, k, v, o, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, o, do))
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, L, d) or v.shape != k.shape or o.shape != q.shape or do.shape != q.shape:
        raise ValueError("shape mismatch")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    mask = np.zeros((L, L), dtype=bool)
    for t in range(L):
        mask[t, key_set(t, s, r)] = True
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kvh = h // G
            S = scale * (q[b, h] @ k[b, kvh].T)
            S = np.where(mask, S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dv[b, kvh] += P.T @ do[b, h]
            dP = do[b, h] @ v[b, kvh].T
            D = (do[b, h] * o[b, h]).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dq[b, h] = scale * (dS @ k[b, kvh])
            dk[b, kvh] += scale * (dS.T @ q[b, h])
    return dq, dk, dv
