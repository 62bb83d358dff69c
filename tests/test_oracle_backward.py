"""Pins of the oracle's backward (CPU): the gradient of the forward
definition by central differences, the dense limit against torch's
autograd on the CPU in fp64, the r = 1 special case and two sum rules."""
import numpy as np
import pytest
import torch

import oracle


def fwd64(q, k, v, s, r, scale):
    """The forward rows in fp64 straight from the key sets (the definition
    the forward pins fix), for the finite differences."""
    B, Hq, L, d = q.shape
    G = Hq // k.shape[1]
    o = np.empty_like(q)
    for b in range(B):
        for h in range(Hq):
            for t in range(L):
                ks = oracle.key_set(t, s, r)
                x = scale * (k[b, h // G, ks] @ q[b, h, t])
                w = np.exp(x - x.max())
                o[b, h, t] = (w / w.sum()) @ v[b, h // G, ks]
    return o


@pytest.mark.parametrize("Hq,Hkv,L,d,s,r", [(2, 1, 9, 4, 2, 3), (1, 1, 7, 3, 0, 2), (3, 3, 6, 2, 1, 1)])
def test_backward_is_the_gradient_of_the_forward(Hq, Hkv, L, d, s, r):
    """Central differences of sum(G * O) against the oracle's gradients."""
    g = np.random.default_rng(L * 10 + d)
    q, k, v = (g.standard_normal((1, H, L, d)) for H in (Hq, Hkv, Hkv))
    G = g.standard_normal((1, Hq, L, d))
    scale = 0.7
    o = fwd64(q, k, v, s, r, scale)
    dq, dk, dv = oracle.backward(q, k, v, o, G, s, r, scale=scale)
    eps = 1e-6
    for x, grad in ((q, dq), (k, dk), (v, dv)):
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            fp = (G * fwd64(q, k, v, s, r, scale)).sum()
            x[idx] = keep - eps
            fm = (G * fwd64(q, k, v, s, r, scale)).sum()
            x[idx] = keep
            num[idx] = (fp - fm) / (2 * eps)
        assert np.abs(num - grad).max() < 1e-7, np.abs(num - grad).max()


@pytest.mark.parametrize("B,Hq,Hkv,L,d,s,r", [(2, 4, 2, 40, 8, 0, 40), (1, 2, 1, 33, 16, 30, 5)])
def test_backward_dense_limit_matches_autograd(B, Hq, Hkv, L, d, s, r):
    """With s + r >= L the key set is every earlier position: torch's
    autograd (CPU, fp64) of plain causal softmax attention."""
    g = np.random.default_rng(B + L)
    q, k, v = (g.standard_normal((B, H, L, d)) for H in (Hq, Hkv, Hkv))
    dO = g.standard_normal((B, Hq, L, d))
    scale = 1.0 / np.sqrt(d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    G = Hq // Hkv
    ke = tk.repeat_interleave(G, dim=1)
    ve = tv.repeat_interleave(G, dim=1)
    sc = torch.matmul(tq, ke.transpose(-1, -2)) * scale
    causal = torch.ones(L, L, dtype=torch.bool).tril()
    sc = sc.masked_fill(~causal, float("-inf"))
    out = torch.matmul(torch.softmax(sc, dim=-1), ve)
    out.backward(torch.tensor(dO))
    dq, dk, dv = oracle.backward(q, k, v, out.detach().numpy(), dO, s, r)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() < 1e-10


def test_backward_r1_s0_passes_dO_to_v_only():
    """r = 1, s = 0: O_t = V_t, so dV_i = sum over the group of dO_i and the
    scores get no gradient."""
    g = np.random.default_rng(3)
    q, k, v = (g.standard_normal((1, H, 12, 8)) for H in (4, 2, 2))
    dO = g.standard_normal((1, 4, 12, 8))
    o = np.repeat(v, 2, axis=1)
    dq, dk, dv = oracle.backward(q, k, v, o, dO, 0, 1)
    # dS = P (dP - D) with P = 1 and dP = D up to the rounding of two dot orders
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    np.testing.assert_allclose(dv, dO.reshape(1, 2, 2, 12, 8).sum(axis=2), rtol=0, atol=1e-14)


def test_backward_sum_rules():
    """Each softmax row sums to one: the key gradients of a kv-head sum to
    zero, and the value gradients sum to the group's summed dO."""
    g = np.random.default_rng(4)
    B, Hq, Hkv, L, d, s, r = 2, 4, 2, 50, 8, 3, 11
    q, k, v = (g.standard_normal((B, H, L, d)) for H in (Hq, Hkv, Hkv))
    dO = g.standard_normal((B, Hq, L, d))
    o = oracle.prefill_rows(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), s, r)
    o = o.reshape(B, Hq, L, d)
    q, k, v = (x.astype(np.float32).astype(np.float64) for x in (q, k, v))
    dq, dk, dv = oracle.backward(q, k, v, o, dO, s, r)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
    want = dO.reshape(B, Hkv, Hq // Hkv, L, d).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(axis=2), want, rtol=0, atol=1e-11)
