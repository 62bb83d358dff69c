"""Sliding-window softmax attention with attention sinks on MI355X (gfx950).

The computation lives in libswa.so (hand-written HIP kernels behind the C ABI
of include/swa.h); this package binds it for PyTorch callers:

  * prefill(q, k, v, s, r, ...)        banded flash-style prefill, optional
                                       rolling cache (chunked) and RoPE
  * prefill_dilated(q, k, v, s, r, dilation) the same with a dilated window
  * rope_keys(k, pos0, base)           keys rotated at their positions (the
                                       form every RoPE call takes)
  * prefill_global(q, k, v, s, r, globals) the same with task-bound global
                                       tokens
  * cache_append(k, v, kc, vc, pos0, ...) write tokens into the rolling cache
  * prefill_append(q, k, v, s, r, kc_next, vc_next, ...) a chunk's rows and
                                       the cache after it, into a second
                                       cache pair, in one launch
  * decode(q, kc, vc, T, s, r, ...)    split-K single-query decode
  * decode_step(q, k, v, kc, vc, T, s, r, ...) append token T-1 and decode
                                       it in one launch
  * decode_step_noalloc(...)           the same without a workspace or any
                                       allocation (static per-GPU scratch)
  * backward(q, k, v, o, dout, s, r)   gradients of prefill's rows (training)

The low-level same-name wrappers of the C functions are in ``_lib``.
"""
from ._lib import EXPORTS, LIB_PATH, SwaDesc, SwaError, load  # noqa: F401
from .ops import (  # noqa: F401
    backward,
    cache_append,
    decode,
    decode_step,
    decode_step_noalloc,
    decode_workspace_bytes,
    make_desc,
    new_cache,
    prefill,
    prefill_append,
    prefill_dilated,
    prefill_global,
    prefill_workspace_bytes,
    rope_keys,
)
