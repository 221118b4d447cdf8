"""Pins of the fp64 backward oracle (analytic gradient of exact attention).

The pages give no backward formulas ("FlashAttention: GPUメモリ階層を活用した
アテンション最適化の分析", sec. 7.2: S and P are recomputed from Q, K, V and the
saved row statistics), so the oracle is the derivative of the forward
definition.  It is pinned by central finite differences of the (separately
pinned) forward oracle, by torch.autograd in fp64, and by two invariants:
softmax shift invariance gives sum_j dK_j = 0, and rows of P summing to one give
sum_j dV_j = sum_i dO_i.
"""
import numpy as np
import pytest

import oracle


def _rand(seed, shape):
    g = np.random.default_rng(seed)
    return [g.standard_normal(shape) for _ in range(4)]


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    q, k, v, do = _rand(1, (1, 2, 6, 3))
    scale = 0.8
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal=causal, scale=scale)

    def loss(q_, k_, v_):
        o, _ = oracle.attn_fwd(q_, k_, v_, causal=causal, scale=scale)
        return float(np.sum(o * do))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}; args_p[name] = xp
            args_m = {"q": q, "k": k, "v": v}; args_m[name] = xm
            num[idx] = (loss(**{a + "_": b for a, b in args_p.items()})
                        - loss(**{a + "_": b for a, b in args_m.items()})) / (2 * h)
        err = np.max(np.abs(num - g)) / max(1.0, np.max(np.abs(g)))
        assert err <= 1e-6, (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd(causal):
    import torch
    q, k, v, do = _rand(2, (2, 2, 17, 8))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = (tq @ tk.transpose(-1, -2)) / np.sqrt(8)
    if causal:
        mask = torch.ones(17, 17, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    o.backward(torch.tensor(do))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal=causal)
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(a - b.numpy())) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    q, k, v, do = _rand(3, (1, 2, 23, 8))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal=causal)
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12
    assert np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_row_subset_matches_full(causal):
    q, k, v, do = _rand(4, (1, 3, 19, 8))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal=causal)
    qr = np.array([0, 5, 18, 19, 40, 56])
    kr = np.array([1, 18, 20, 37, 38])
    sq, sk, sv = oracle.attn_bwd(q, k, v, do, causal=causal, qrows=qr, krows=kr)
    assert np.max(np.abs(sq - dq.reshape(-1, 8)[qr])) <= 1e-14
    assert np.max(np.abs(sk - dk.reshape(-1, 8)[kr])) <= 1e-14
    assert np.max(np.abs(sv - dv.reshape(-1, 8)[kr])) <= 1e-14
