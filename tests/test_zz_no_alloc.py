"""swa_decode_step_noalloc (no workspace, no allocation) against
swa_decode_step with a caller workspace: same cache bytes and outputs, bit
for bit, through the C ABI, on two calls in a row (the second smaller, so it
runs on what the first left in the static scratch)."""
import numpy as np
import pytest
import torch

import swa_inputs as si
from sliding_window_attention_sink_amd import _lib
from sliding_window_attention_sink_amd._lib import SwaDesc

from gpu_common import bits, dev, say

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, d, s, r, T, n_split, seed, rope_base=0.0):
    hist = T - 1
    k = dev(si.draw(seed, 1, B, Hkv, hist, d), "bf16")
    v = dev(si.draw(seed, 2, B, Hkv, hist, d), "bf16")
    q = dev(si.draw(seed, 0, B, Hq, 1, d, block=1)[:, :, 0], "bf16")
    kn = dev(si.draw(seed, 1, B, Hkv, 1, d, block=1)[:, :, 0], "bf16")
    vn = dev(si.draw(seed, 2, B, Hkv, 1, d, block=1)[:, :, 0], "bf16")
    desc = SwaDesc(B, Hq, Hkv, d, s, r, _lib.SWA_BF16, float(1 / np.sqrt(d)), float(rope_base))
    kc = torch.full((B, Hkv, s + r, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    _lib.check(_lib.swa_cache_append(desc, k.data_ptr(), v.data_ptr(), hist, 0, kc.data_ptr(), vc.data_ptr(), None))
    return desc, q, kn, vn, kc, vc


@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
def test_noalloc_matches_workspace_call(gpu, rope_base):
    # first call: 4 sequences, 8 splits; second: 2 sequences, 3 splits (a
    # smaller partial block on top of the first call's leftovers)
    for (B, Hq, Hkv, d, s, r, T, ns, seed) in [(4, 8, 2, 128, 4, 1000, 1500, 8, 71),
                                               (2, 4, 2, 64, 2, 300, 250, 3, 72)]:
        say("noalloc", B, Hq, Hkv, d, s, r, T, ns, rope_base)
        desc, q, kn, vn, kc, vc = _case(B, Hq, Hkv, d, s, r, T, ns, seed, rope_base)
        kc2, vc2 = kc.clone(), vc.clone()
        wsb = _lib.swa_decode_workspace_bytes(desc, ns)
        assert 0 < wsb <= _lib.NOALLOC_SCRATCH_BYTES
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        o_ref = torch.empty_like(q)
        o_na = torch.full_like(q, float("nan"))
        _lib.check(_lib.swa_decode_step(desc, q.data_ptr(), kn.data_ptr(), vn.data_ptr(), kc.data_ptr(),
                                        vc.data_ptr(), T, o_ref.data_ptr(), ns, ws.data_ptr(), wsb, None))
        _lib.check(_lib.swa_decode_step_noalloc(desc, q.data_ptr(), kn.data_ptr(), vn.data_ptr(), kc2.data_ptr(),
                                                vc2.data_ptr(), T, o_na.data_ptr(), ns, None))
        torch.cuda.synchronize()
        assert np.array_equal(bits(o_na), bits(o_ref))
        assert np.array_equal(bits(kc2), bits(kc)) and np.array_equal(bits(vc2), bits(vc))


def test_noalloc_default_and_one_split(gpu):
    # the library's split choice (16 splits for one sequence of 8 kv-heads)
    # and one split (no scratch used), against the workspace call
    B, Hq, Hkv, d, s, r, T = 1, 32, 8, 128, 4, 4092, 9000
    desc, q, kn, vn, kc, vc = _case(B, Hq, Hkv, d, s, r, T, 0, 73)
    for ns in (0, 1):
        say("noalloc splits", ns)
        kc1, vc1, kc2, vc2 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
        wsb = _lib.swa_decode_workspace_bytes(desc, ns)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        o_ref = torch.empty_like(q)
        o_na = torch.full_like(q, float("nan"))
        _lib.check(_lib.swa_decode_step(desc, q.data_ptr(), kn.data_ptr(), vn.data_ptr(), kc1.data_ptr(),
                                        vc1.data_ptr(), T, o_ref.data_ptr(), ns, ws.data_ptr(), wsb, None))
        _lib.check(_lib.swa_decode_step_noalloc(desc, q.data_ptr(), kn.data_ptr(), vn.data_ptr(), kc2.data_ptr(),
                                                vc2.data_ptr(), T, o_na.data_ptr(), ns, None))
        torch.cuda.synchronize()
        assert np.array_equal(bits(o_na), bits(o_ref))
        assert np.array_equal(bits(kc2), bits(kc1)) and np.array_equal(bits(vc2), bits(vc1))


def test_noalloc_rejects_oversize(gpu):
    # 64 sequences x 32 heads x 64 splits x 130 floats = 68 MB > 8 MiB: rejected,
    # nothing enqueued, the message names the limit
    desc = SwaDesc(64, 32, 8, 128, 4, 4092, _lib.SWA_BF16, 0.088, 0.0)
    x = torch.empty(64 * 32 * 128, dtype=torch.bfloat16, device="cuda")
    st = _lib.swa_decode_step_noalloc(desc, x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(),
                                      100, x.data_ptr(), 64, None)
    assert st == _lib.SWA_ERR_INVALID_ARG
    assert "scratch" in _lib.swa_last_error()
