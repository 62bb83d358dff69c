"""Torch-facing calls into libswa.so.

PyTorch supplies device memory and the current stream; every step of the
computation runs in the library's HIP kernels.  These helpers only check
tensor shapes/dtypes, allocate outputs and workspaces, and raise SwaError
when the library rejects a call.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import SwaDesc, check

_DTYPES = {torch.float32: _lib.SWA_F32, torch.bfloat16: _lib.SWA_BF16}


def make_desc(B, Hq, Hkv, d, s, r, dtype, scale=None, rope_base=0.0) -> SwaDesc:
    if dtype not in _DTYPES:
        raise TypeError("dtype must be float32 or bfloat16, got %s" % dtype)
    return SwaDesc(B, Hq, Hkv, d, s, r, _DTYPES[dtype], float(1.0 / math.sqrt(d) if scale is None else scale),
                   float(rope_base))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev, stream):
    s = torch.cuda.current_stream(dev) if stream is None else stream
    return s.cuda_stream


def _need(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def prefill_workspace_bytes(desc: SwaDesc, L: int) -> int:
    return _lib.swa_prefill_workspace_bytes(desc, L)


def rope_keys(k, pos0, base, *, out=None, stream=None):
    """Keys k [B,Hkv,n,d] (bf16; row i = position pos0 + i) rotated at their
    positions: the form prefill, cache_append and decode take with RoPE."""
    B, Hkv, n, d = k.shape
    dev = k.device
    desc = make_desc(B, Hkv, Hkv, d, 0, 1, k.dtype, rope_base=base)
    if out is None:
        out = torch.empty_like(k)
    _need(out, "out", k.shape, k.dtype, dev)
    check(_lib.swa_rope_keys(desc, _ptr(k), n, pos0, _ptr(out), _stream(dev, stream)))
    return out


def prefill(q, k, v, s, r, *, scale=None, rope_base=0.0, k_cache=None, v_cache=None, pos0=0, out=None,
            workspace=None, stream=None):
    """O = sliding-window attention with sinks over q [B,Hq,L,d], k/v [B,Hkv,L,d].

    With k_cache/v_cache ([B,Hkv,s+r,d]) rows are positions pos0.. and keys
    before pos0 come from the cache (chunked prefill).  With rope_base > 0 the
    keys (k and the cache's) are rotated at their positions (rope_keys) and q
    is not.
    """
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    desc = make_desc(B, Hq, Hkv, d, s, r, q.dtype, scale, rope_base)
    _need(k, "k", (B, Hkv, L, d), q.dtype, dev)
    _need(v, "v", (B, Hkv, L, d), q.dtype, dev)
    if k_cache is not None or v_cache is not None:
        _need(k_cache, "k_cache", (B, Hkv, s + r, d), q.dtype, dev)
        _need(v_cache, "v_cache", (B, Hkv, s + r, d), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.shape, q.dtype, dev)
    wsb = _lib.swa_prefill_workspace_bytes(desc, L)
    if wsb and workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    check(_lib.swa_prefill(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(out), L, _ptr(k_cache), _ptr(v_cache), pos0,
                           _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(dev, stream)))
    return out


def prefill_append(q, k, v, s, r, k_next, v_next, *, scale=None, rope_base=0.0, k_cache=None, v_cache=None,
                   pos0=0, out=None, stream=None):
    """prefill's rows over (k_cache, v_cache) + the chunk, and the cache after
    appending the chunk written to (k_next, v_next) in the same launch (bf16;
    needs L >= r or pos0 <= s; the current cache is only read)."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    desc = make_desc(B, Hq, Hkv, d, s, r, q.dtype, scale, rope_base)
    _need(k, "k", (B, Hkv, L, d), q.dtype, dev)
    _need(v, "v", (B, Hkv, L, d), q.dtype, dev)
    if k_cache is not None or v_cache is not None:
        _need(k_cache, "k_cache", (B, Hkv, s + r, d), q.dtype, dev)
        _need(v_cache, "v_cache", (B, Hkv, s + r, d), q.dtype, dev)
    _need(k_next, "k_next", (B, Hkv, s + r, d), q.dtype, dev)
    _need(v_next, "v_next", (B, Hkv, s + r, d), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.shape, q.dtype, dev)
    check(_lib.swa_prefill_append(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(out), L, _ptr(k_cache), _ptr(v_cache),
                                  pos0, _ptr(k_next), _ptr(v_next), _stream(dev, stream)))
    return out


def new_cache(B, Hkv, d, s, r, dtype, device, fill=0.0):
    """Caller-owned rolling cache pair [B, Hkv, s+r, d] (fill e.g. NaN to poison unwritten slots)."""
    kc = torch.full((B, Hkv, s + r, d), fill, dtype=dtype, device=device)
    vc = torch.full((B, Hkv, s + r, d), fill, dtype=dtype, device=device)
    return kc, vc


def prefill_dilated(q, k, v, s, r, dilation, *, scale=None, out=None, workspace=None, stream=None):
    """Prefill with a dilated window: row t attends the sinks and t, t-dilation, ..., t-(r-1)dilation."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    desc = make_desc(B, Hq, Hkv, d, s, r, q.dtype, scale)
    _need(k, "k", (B, Hkv, L, d), q.dtype, dev)
    _need(v, "v", (B, Hkv, L, d), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.shape, q.dtype, dev)
    wsb = _lib.swa_prefill_dilated_workspace_bytes(desc, L, dilation)
    if workspace is None and wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    check(_lib.swa_prefill_dilated(desc, dilation, _ptr(q), _ptr(k), _ptr(v), _ptr(out), L, _ptr(workspace),
                                   0 if workspace is None else workspace.numel(), _stream(dev, stream)))
    return out


def prefill_global(q, k, v, s, r, globals_, *, scale=None, out=None, workspace=None, stream=None):
    """Prefill with task-bound global tokens at the given positions (host ints,
    strictly increasing): those rows attend every earlier key, every other
    row also attends the global positions up to itself."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    desc = make_desc(B, Hq, Hkv, d, s, r, q.dtype, scale)
    _need(k, "k", (B, Hkv, L, d), q.dtype, dev)
    _need(v, "v", (B, Hkv, L, d), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.shape, q.dtype, dev)
    g = [int(x) for x in globals_]
    wsb = _lib.swa_prefill_global_workspace_bytes(desc, L, len(g)) if g else 0
    if workspace is None and wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    check(_lib.swa_prefill_global(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(out), L, g, len(g), _ptr(workspace),
                                  0 if workspace is None else workspace.numel(), _stream(dev, stream)))
    return out


def backward(q, k, v, o, dout, s, r, *, scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv; fp32) of prefill's rows for the upstream dout.

    q, o, dout [B,Hq,L,d] and k, v [B,Hkv,L,d] are bf16; o is prefill's output.
    """
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    desc = make_desc(B, Hq, Hkv, d, s, r, q.dtype, scale)
    _need(k, "k", (B, Hkv, L, d), q.dtype, dev)
    _need(v, "v", (B, Hkv, L, d), q.dtype, dev)
    _need(o, "o", q.shape, q.dtype, dev)
    _need(dout, "dout", q.shape, q.dtype, dev)
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty(k.shape, dtype=torch.float32, device=dev)
    _need(dq, "dq", q.shape, torch.float32, dev)
    _need(dk, "dk", k.shape, torch.float32, dev)
    _need(dv, "dv", k.shape, torch.float32, dev)
    wsb = _lib.swa_backward_workspace_bytes(desc, L)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    check(_lib.swa_backward(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), L,
                            _ptr(workspace), workspace.numel(), _stream(dev, stream)))
    return dq, dk, dv


def cache_append(k_new, v_new, k_cache, v_cache, pos0, s, r, *, stream=None):
    """Write tokens pos0 .. pos0+n-1 (k_new/v_new [B,Hkv,n,d]) into the rolling cache."""
    B, Hkv, n, d = k_new.shape
    dev = k_new.device
    desc = make_desc(B, Hkv, Hkv, d, s, r, k_new.dtype)
    _need(v_new, "v_new", k_new.shape, k_new.dtype, dev)
    _need(k_cache, "k_cache", (B, Hkv, s + r, d), k_new.dtype, dev)
    _need(v_cache, "v_cache", (B, Hkv, s + r, d), k_new.dtype, dev)
    check(_lib.swa_cache_append(desc, _ptr(k_new), _ptr(v_new), n, pos0, _ptr(k_cache), _ptr(v_cache),
                                _stream(dev, stream)))


def decode_workspace_bytes(desc: SwaDesc, n_split: int = 0) -> int:
    return _lib.swa_decode_workspace_bytes(desc, n_split)


def decode(q, k_cache, v_cache, T, s, r, *, scale=None, rope_base=0.0, n_split=0, out=None, workspace=None,
           stream=None):
    """Decode step: q [B,Hq,d] of token T-1 over the cache holding tokens 0..T-1
    (rope_base > 0: pre-rotation q and keys, StreamingLLM re-positioning)."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    dev = q.device
    desc = make_desc(B, Hq, Hkv, d, s, r, q.dtype, scale, rope_base=rope_base)
    _need(k_cache, "k_cache", (B, Hkv, s + r, d), q.dtype, dev)
    _need(v_cache, "v_cache", (B, Hkv, s + r, d), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.shape, q.dtype, dev)
    wsb = _lib.swa_decode_workspace_bytes(desc, n_split)
    if workspace is None and wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    check(_lib.swa_decode(desc, _ptr(q), _ptr(k_cache), _ptr(v_cache), T, _ptr(out), n_split, _ptr(workspace),
                          0 if workspace is None else workspace.numel(), _stream(dev, stream)))
    return out


def decode_step(q, k_new, v_new, k_cache, v_cache, T, s, r, *, scale=None, rope_base=0.0, n_split=0, out=None,
                workspace=None, stream=None):
    """Append token T-1 (k_new/v_new [B,Hkv,d]) and decode its query q [B,Hq,d], in one launch."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    dev = q.device
    desc = make_desc(B, Hq, Hkv, d, s, r, q.dtype, scale, rope_base=rope_base)
    _need(k_new, "k_new", (B, Hkv, d), q.dtype, dev)
    _need(v_new, "v_new", (B, Hkv, d), q.dtype, dev)
    _need(k_cache, "k_cache", (B, Hkv, s + r, d), q.dtype, dev)
    _need(v_cache, "v_cache", (B, Hkv, s + r, d), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.shape, q.dtype, dev)
    wsb = _lib.swa_decode_workspace_bytes(desc, n_split)
    if workspace is None and wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    check(_lib.swa_decode_step(desc, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), T, _ptr(out),
                               n_split, _ptr(workspace), 0 if workspace is None else workspace.numel(),
                               _stream(dev, stream)))
    return out


def decode_step_noalloc(q, k_new, v_new, k_cache, v_cache, T, s, r, *, out, scale=None, rope_base=0.0, n_split=0,
                        stream=None):
    """decode_step without a workspace: the split partials go to the library's
    static per-GPU scratch (calls on one GPU must not overlap).  `out` is
    required, so the call allocates nothing."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    dev = q.device
    desc = make_desc(B, Hq, Hkv, d, s, r, q.dtype, scale, rope_base=rope_base)
    _need(k_new, "k_new", (B, Hkv, d), q.dtype, dev)
    _need(v_new, "v_new", (B, Hkv, d), q.dtype, dev)
    _need(k_cache, "k_cache", (B, Hkv, s + r, d), q.dtype, dev)
    _need(v_cache, "v_cache", (B, Hkv, s + r, d), q.dtype, dev)
    _need(out, "out", q.shape, q.dtype, dev)
    check(_lib.swa_decode_step_noalloc(desc, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), T,
                                       _ptr(out), n_split, _stream(dev, stream)))
    return out
