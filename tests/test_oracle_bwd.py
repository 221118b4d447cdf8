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
from synth_inputs import normal_qkv


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


# ---- bf16 rounding and the bf16 standard-attention backward baseline ----

def test_bf16_round_matches_torch():
    import torch
    g = np.random.default_rng(40)
    x = (g.standard_normal(50000) * 10.0 ** g.integers(-20, 20, 50000)).astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_round(x), want)
    # exact midpoints between neighbouring bf16 values go to the even one
    lo = torch.from_numpy(x[:2000].astype(np.float32)).to(torch.bfloat16)
    lo_bits = lo.view(torch.int16).numpy().astype(np.int64)
    hi = torch.from_numpy((lo_bits + 1).astype(np.int16)).view(torch.bfloat16)
    a, b = lo.to(torch.float64).numpy(), hi.to(torch.float64).numpy()
    fin = np.isfinite(a) & np.isfinite(b) & (np.sign(a) == np.sign(b)) & (a != 0)
    mid = 0.5 * (a + b)[fin]
    got = oracle.bf16_round(mid)
    even = np.where(lo_bits[fin] % 2 == 0, a[fin], b[fin])
    assert np.array_equal(got, even)


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_baseline_single_key_is_exact(causal):
    # one key: P = 1, O = v_0, dS = dO . (v_0 - O) = 0 for bf16 inputs, so
    # dQ = dK = 0 and dV = dO exactly
    import torch
    g = np.random.default_rng(41)
    x = [torch.from_numpy(g.standard_normal((2, 3, 1, 8)).astype(np.float32)).to(torch.bfloat16)
         .to(torch.float64).numpy() for _ in range(4)]
    dq, dk, dv = oracle.attn_bwd_bf16_baseline(*x, causal=causal)
    assert np.all(dq == 0) and np.all(dk == 0) and np.array_equal(dv, x[3])


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_baseline_is_near_the_exact_gradient(causal):
    """Its error against the exact gradient is that of a few bf16 roundings:
    relative RMS between 1e-4 (some rounding happened) and 1e-2."""
    q, k, v, do = (x.astype(np.float64) for x in normal_qkv(1, 2, 70, 16, 42, with_dout=True))
    exact = oracle.attn_bwd(q, k, v, do, causal=causal)
    base = oracle.attn_bwd_bf16_baseline(q, k, v, do, causal=causal)
    for e, b in zip(exact, base):
        rel = np.sqrt(np.mean((b - e) ** 2)) / np.sqrt(np.mean(e ** 2))
        assert 1e-4 < rel < 1e-2, rel
