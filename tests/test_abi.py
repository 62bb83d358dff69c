"""The C ABI on the CPU: the library loads, exports every function that
include/swa.h declares, and rejects bad arguments on the host (status code
and message) before touching the GPU.  No call here reaches a kernel."""
import ctypes
import os
import re

import pytest

from sliding_window_attention_sink_amd import _lib
from sliding_window_attention_sink_amd._lib import SwaDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swa.h")

# distinct, 16-byte aligned fake device addresses: validation never dereferences them
A, B_, C, D, E, F, W = (0x10000 * (i + 1) for i in range(7))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(swa_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def desc(**kw):
    base = dict(B=1, Hq=4, Hkv=2, d=128, s=4, r=28, dtype=_lib.SWA_BF16, scale=0.125, rope_base=0.0)
    base.update(kw)
    return SwaDesc(**base)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_match_header(lib):
    decl = declared_functions()
    assert decl == sorted(_lib.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name
    assert lib.swa_abi_version() == 1


def test_status_strings(lib):
    assert _lib.swa_status_str(0) == "ok"
    assert _lib.swa_status_str(-1) == "invalid argument"
    assert _lib.swa_status_str(-2) == "unsupported configuration"
    assert _lib.swa_status_str(-3) == "HIP error"


def prefill(d_, q=A, k=B_, v=C, o=D, L=100, kc=None, vc=None, pos0=0, ws=None, wsb=0):
    return _lib.swa_prefill(d_, q, k, v, o, L, kc, vc, pos0, ws, wsb, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(B=0), -1, "B, Hq, Hkv"),
    (dict(Hq=6, Hkv=4), -1, "multiple of Hkv"),
    (dict(s=-1), -1, "s must be"),
    (dict(r=0), -1, "r must be"),
    (dict(scale=0.0), -1, "scale"),
    (dict(scale=float("nan")), -1, "scale"),
    (dict(rope_base=-1.0), -1, "rope_base"),
    (dict(d=96), -2, "head dim"),
    (dict(dtype=5), -2, "dtype"),
    (dict(dtype=_lib.SWA_F32, rope_base=10000.0), -2, "RoPE"),
])
def test_prefill_rejects_desc(kw, status, msg):
    assert prefill(desc(**kw)) == status
    assert msg in _lib.swa_last_error()


def test_prefill_rejects_args(lib):
    d_ = desc()
    assert prefill(d_, q=None) == -1 and "q is NULL" in _lib.swa_last_error()
    assert prefill(d_, o=D + 8) == -1 and "aligned" in _lib.swa_last_error()
    assert prefill(d_, L=0) == -1 and "L must be" in _lib.swa_last_error()
    assert prefill(d_, pos0=-1) == -1
    assert prefill(d_, pos0=5) == -1 and "cache" in _lib.swa_last_error()
    assert prefill(d_, kc=E, vc=None) == -1 and "v_cache is NULL" in _lib.swa_last_error()
    assert prefill(d_, L=(1 << 30) + 1) == -1 and "2^30" in _lib.swa_last_error()
    assert lib.swa_prefill(None, A, B_, C, D, 10, None, None, 0, None, 0, None) == -1
    assert "desc is NULL" in _lib.swa_last_error()


def test_prefill_needs_no_workspace():
    # keys come rotated (swa_rope_keys), so no call needs a workspace
    assert _lib.swa_prefill_workspace_bytes(desc(rope_base=10000.0), 100) == 0
    assert _lib.swa_prefill_workspace_bytes(desc(), 100) == 0
    assert _lib.swa_prefill_workspace_bytes(desc(r=0), 100) == 0


def test_rope_keys_rejects():
    d_ = desc(rope_base=10000.0)
    assert _lib.swa_rope_keys(desc(), A, 4, 0, B_, None) == -1 and "rope_base" in _lib.swa_last_error()
    assert _lib.swa_rope_keys(d_, None, 4, 0, B_, None) == -1 and "k is NULL" in _lib.swa_last_error()
    assert _lib.swa_rope_keys(d_, A, 4, 0, B_ + 8, None) == -1 and "aligned" in _lib.swa_last_error()
    assert _lib.swa_rope_keys(d_, A, 0, 0, B_, None) == -1 and "n must be" in _lib.swa_last_error()
    assert _lib.swa_rope_keys(d_, A, 4, -1, B_, None) == -1 and "pos0" in _lib.swa_last_error()
    assert _lib.swa_rope_keys(d_, A, 4, (1 << 30) - 2, B_, None) == -1
    assert _lib.swa_rope_keys(desc(rope_base=1e4, d=80), A, 4, 0, B_, None) == -2
    assert _lib.swa_rope_keys(desc(rope_base=1e4, dtype=_lib.SWA_F32), A, 4, 0, B_, None) == -2


def test_rope_decode_group_limit():
    # the band and sink copies of a kv-head's q-heads share 16 MFMA columns
    d_ = desc(Hq=16, Hkv=1, rope_base=1e4)
    assert _lib.swa_decode(d_, A, B_, C, 100, D, 1, None, 0, None) == -2
    assert "8 q-heads" in _lib.swa_last_error()


def test_prefill_append_rejects():
    d_ = desc()          # s = 4, r = 28
    G, H = 0x90000, 0xA0000
    call = lambda dd, L=40, kc=E, vc=F, pos0=64, kn=G, vn=H: _lib.swa_prefill_append(
        dd, A, B_, C, D, L, kc, vc, pos0, kn, vn, None)
    assert call(d_, kn=None) == -1 and "k_next is NULL" in _lib.swa_last_error()
    assert call(d_, vn=H + 8) == -1 and "aligned" in _lib.swa_last_error()
    assert call(d_, kn=E) == -1 and "another buffer" in _lib.swa_last_error()
    assert call(d_, vn=G) == -1 and "another buffer" in _lib.swa_last_error()
    # a chunk shorter than r past the sinks leaves cached tokens in rolling slots
    assert call(d_, L=27) == -1 and "L >= r or pos0 <= s" in _lib.swa_last_error()
    assert call(desc(dtype=_lib.SWA_F32)) == -2 and "bf16" in _lib.swa_last_error()
    # the checks of swa_prefill come first
    assert call(d_, L=0) == -1 and "L must be" in _lib.swa_last_error()
    assert call(d_, kc=None, vc=None) == -1 and "cache" in _lib.swa_last_error()


def test_append_rejects():
    d_ = desc()
    assert _lib.swa_cache_append(d_, A, B_, 0, 0, C, D, None) == -1 and "n must be" in _lib.swa_last_error()
    assert _lib.swa_cache_append(d_, A, B_, 4, -2, C, D, None) == -1
    assert _lib.swa_cache_append(d_, A, None, 4, 0, C, D, None) == -1 and "v_new" in _lib.swa_last_error()
    assert _lib.swa_cache_append(d_, A, B_, 4, 0, C + 4, D, None) == -1 and "aligned" in _lib.swa_last_error()
    assert _lib.swa_cache_append(desc(d=80), A, B_, 4, 0, C, D, None) == -2


def test_decode_rejects():
    d_ = desc()
    ws = _lib.swa_decode_workspace_bytes(d_, 3)
    assert ws == 1 * 4 * 3 * (128 + 2) * 4
    dflt = _lib.swa_decode_default_splits(d_)
    assert 1 <= dflt <= 64
    assert _lib.swa_decode_workspace_bytes(d_, 0) == (0 if dflt == 1 else 1 * 4 * dflt * 130 * 4)
    assert _lib.swa_decode_workspace_bytes(d_, 65) == 0
    # one split needs no workspace
    assert _lib.swa_decode_workspace_bytes(d_, 1) == 0

    def dec(dd=d_, T=10, n_split=3, wsb=ws, q=A):
        return _lib.swa_decode(dd, q, B_, C, T, D, n_split, W, wsb, None)

    assert dec(T=0) == -1 and "T must be" in _lib.swa_last_error()
    assert dec(n_split=65) == -1 and "n_split" in _lib.swa_last_error()
    assert dec(wsb=ws - 4) == -1 and "workspace" in _lib.swa_last_error()
    assert dec(q=None) == -1
    assert dec(dd=desc(dtype=_lib.SWA_F32)) == -2
    assert dec(dd=desc(Hq=34, Hkv=2)) == -2 and "16 q-heads" in _lib.swa_last_error()


def test_decode_step_rejects():
    d_ = desc()
    ws = _lib.swa_decode_workspace_bytes(d_, 3)

    def step(kn=A, vn=B_, T=10, wsb=ws):
        return _lib.swa_decode_step(d_, A, kn, vn, C, D, T, W, 3, W, wsb, None)

    assert step(kn=None) == -1 and "k_new" in _lib.swa_last_error()
    assert step(vn=None) == -1 and "v_new" in _lib.swa_last_error()
    assert step(kn=A + 4) == -1 and "aligned" in _lib.swa_last_error()
    assert step(T=0) == -1 and "T must be" in _lib.swa_last_error()
    assert step(wsb=ws - 4) == -1 and "workspace" in _lib.swa_last_error()


def test_prefill_dilated_rejects():
    d_ = desc()
    # the classes are read and written in place: no workspace at any dilation
    assert _lib.swa_prefill_dilated_workspace_bytes(d_, 100, 3) == 0
    assert _lib.swa_prefill_dilated_workspace_bytes(d_, 100, 1) == 0

    def dil(dd=d_, dl=3, L=100):
        return _lib.swa_prefill_dilated(dd, dl, A, B_, C, D, L, None, 0, None)

    assert dil(dl=0) == -1 and "dilation" in _lib.swa_last_error()
    assert dil(dl=65537) == -1 and "dilation" in _lib.swa_last_error()
    assert dil(dd=desc(rope_base=1e4)) == -2
    assert dil(L=0) == -1
    assert _lib.swa_prefill_dilated(d_, 3, None, B_, C, D, 100, None, 0, None) == -1
    assert "q" in _lib.swa_last_error()


def test_backward_rejects():
    d_ = desc()
    wsb = _lib.swa_backward_workspace_bytes(d_, 100)
    # two floats a row (log-sum-exp and D), each array padded by 64 rows and
    # rounded to 256 bytes; no split key tile at L = 100
    per = (1 * 4 * 100 + 64) * 4
    assert wsb == 2 * ((per + 255) // 256 * 256)
    # split tiles add partial slots of 2 * 128 * d floats: GQA 4/2 (256 / 2 =
    # 128 query blocks a segment), L = 8192, r = 4096 -> band tiles of
    # (126 + 4096) // 32 + 1 = 132 blocks in 2 segments, 64 tiles, 2 kv-heads
    big = desc(s=0, r=4096)
    per = (1 * 4 * 8192 + 64) * 4
    assert _lib.swa_backward_workspace_bytes(big, 8192) == 2 * ((per + 255) // 256 * 256) + 2 * 64 * 1 * 2 * 128 * 128 * 4
    G1, G2, G3 = 0x80000, 0x90000, 0xA0000

    def bwd(dd=d_, q=A, dq=G1, ws=W, n=wsb, L=100):
        return _lib.swa_backward(dd, q, B_, C, D, E, dq, G2, G3, L, ws, n, None)

    assert bwd(q=None) == -1 and "q is NULL" in _lib.swa_last_error()
    assert bwd(dq=G1 + 8) == -1 and "aligned" in _lib.swa_last_error()
    assert bwd(ws=None) == -1 and "workspace" in _lib.swa_last_error()
    assert bwd(n=wsb - 16) == -1 and "workspace" in _lib.swa_last_error()
    assert bwd(L=0) == -1 and "L must be" in _lib.swa_last_error()
    assert bwd(dd=desc(dtype=_lib.SWA_F32)) == -2 and "bf16" in _lib.swa_last_error()
    assert bwd(dd=desc(rope_base=1e4)) == -2 and "RoPE" in _lib.swa_last_error()
    assert bwd(dd=desc(d=96)) == -2


def test_last_error_is_per_call():
    assert prefill(desc(r=0)) == -1
    assert _lib.swa_last_error() != ""
    # a later rejected call replaces the message
    assert prefill(desc(s=-3)) == -1
    assert "s must be" in _lib.swa_last_error()


def test_ctypes_desc_layout():
    assert ctypes.sizeof(SwaDesc) == 9 * 4
    assert SwaDesc.scale.offset == 28 and SwaDesc.rope_base.offset == 32


def test_decode_step_noalloc_rejects_on_host(lib):
    # partials beyond the static scratch: 64 x 32 heads x 64 splits x 130 floats
    big = desc(B=64, Hq=32, Hkv=8, s=4, r=4092)
    st = _lib.swa_decode_step_noalloc(big, A, B_, C, D, E, 100, F, 64, None)
    assert st == _lib.SWA_ERR_INVALID_ARG and "scratch" in _lib.swa_last_error()
    assert str(_lib.NOALLOC_SCRATCH_BYTES) in _lib.swa_last_error()
    # argument errors of swa_decode_step come before any HIP call
    assert _lib.swa_decode_step_noalloc(desc(), A, None, C, D, E, 100, F, 2, None) == _lib.SWA_ERR_INVALID_ARG
    assert _lib.swa_decode_step_noalloc(desc(), A, B_, C, D, E, 0, F, 2, None) == _lib.SWA_ERR_INVALID_ARG
    assert _lib.swa_decode_step_noalloc(desc(), A + 8, B_, C, D, E, 100, F, 2, None) == _lib.SWA_ERR_INVALID_ARG
    assert _lib.swa_decode_step_noalloc(desc(), A, B_, C, D, E, 100, F, 65, None) == _lib.SWA_ERR_INVALID_ARG
    assert _lib.swa_decode_step_noalloc(desc(dtype=_lib.SWA_F32), A, B_, C, D, E, 100, F, 2, None) == \
        _lib.SWA_ERR_UNSUPPORTED


def test_prefill_global_rejects():
    d_ = desc()
    wsb = _lib.swa_prefill_global_workspace_bytes(d_, 100, 3)
    assert wsb > 0 and _lib.swa_prefill_global_workspace_bytes(d_, 100, 0) == 0
    assert _lib.swa_prefill_global_workspace_bytes(d_, 100, 65) == 0

    def glob(dd=d_, G=(5, 9, 40), ng=None, ws=W, n=wsb, L=100):
        return _lib.swa_prefill_global(dd, A, B_, C, D, L, G, len(G) if ng is None else ng, ws, n, None)

    assert glob(G=(5, 5)) == -1 and "increase" in _lib.swa_last_error()
    assert glob(G=(9, 5)) == -1 and "increase" in _lib.swa_last_error()
    assert glob(G=(5, 100)) == -1 and "outside" in _lib.swa_last_error()
    assert glob(G=(-1, 5)) == -1 and "outside" in _lib.swa_last_error()
    assert glob(G=None, ng=2) == -1 and "globals is NULL" in _lib.swa_last_error()
    assert glob(G=tuple(range(65)), L=200) == -1 and "global tokens" in _lib.swa_last_error()
    assert glob(ws=None) == -1 and "workspace" in _lib.swa_last_error()
    assert glob(n=wsb - 16) == -1 and "workspace" in _lib.swa_last_error()
    assert glob(dd=desc(dtype=_lib.SWA_F32)) == -2
    assert glob(dd=desc(rope_base=1e4)) == -2
    assert glob(dd=desc(Hq=34, Hkv=2)) == -2
