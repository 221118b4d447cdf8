"""Pins of the fp64 forward oracle against facts other than itself.

Each test fixes a property that the exact-attention definition implies
("FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析", sec. 2.1 and
6.1; causal = lower triangle, sec. 11.3):
  * probability rows are non-negative, sum to 1 and vanish on masked keys;
  * constant V returns that constant;
  * equal scores return the (prefix) mean of V and LSE = ln(#allowed keys);
  * causal row 0 returns v_0 with LSE_0 = scale * q_0 . k_0;
  * brute force in 50-digit arithmetic (mpmath) on tiny shapes;
  * torch's fp64 CPU scaled_dot_product_attention (a library routine);
  * metamorphic relations: joint K/V row permutation (non-causal) and adding
    one vector to every key row (O unchanged, LSE shifted by scale * q . c).
A dropped term, a wrong sign, a transposed operand or an off-by-one in the
mask fails at least one of them (see test_oracle_mutants.py).
"""
import numpy as np
import pytest

import oracle
from synth_inputs import normal_qkv, sample_rows


def _qkv(B, H, N, d, seed):
    q, k, v = normal_qkv(B, H, N, d, seed)
    return q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    q, k, _ = _qkv(2, 3, 37, 16, 11)
    B, H, N, d = q.shape
    for flat in [0, 1, 17, N - 1, N + 5, B * H * N - 1]:
        p = oracle.attn_probs_row(q, k, flat, causal=causal)
        i = flat % N
        assert np.all(p >= 0)
        assert abs(p.sum() - 1.0) <= 1e-15 * N
        if causal:
            assert np.all(p[i + 1:] == 0.0)
            assert np.all(p[: i + 1] > 0)


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_reproduce_the_forward(causal):
    """A probability row times V is the output row of the forward oracle (whose
    pins are below), and its log-normaliser is the forward's LSE: the row
    P[i, :] = exp(s_i - LSE_i) is what O = P V and LSE summarise."""
    q, k, v = _qkv(2, 3, 37, 16, 21)
    B, H, N, d = q.shape
    o, lse = oracle.attn_fwd(q, k, v, causal=causal)
    for flat in [0, 1, 17, N - 1, N + 5, 2 * N + 30, B * H * N - 1]:
        bh, i = divmod(flat, N)
        b, h = divmod(bh, H)
        p = oracle.attn_probs_row(q, k, flat, causal=causal)
        assert np.max(np.abs(p @ v[b, h] - o[b, h, i])) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_brute_force_mpmath(causal):
    import mpmath as mp
    mp.mp.dps = 50
    g = np.random.default_rng(31)
    q, k = (g.standard_normal((1, 2, 5, 3)) * 2 for _ in range(2))
    scale = 0.9
    for flat in range(10):
        h, i = divmod(flat, 5)
        js = range(i + 1) if causal else range(5)
        s = {j: mp.mpf(scale) * mp.fsum(mp.mpf(q[0, h, i, c]) * mp.mpf(k[0, h, j, c]) for c in range(3))
             for j in js}
        z = mp.fsum(mp.e ** s[j] for j in js)
        want = np.array([float(mp.e ** s[j] / z) if j in s else 0.0 for j in range(5)])
        got = oracle.attn_probs_row(q, k, flat, causal=causal, scale=scale)
        assert np.max(np.abs(got - want)) <= 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_returns_constant(causal):
    q, k, _ = _qkv(1, 2, 50, 8, 12)
    c = np.linspace(-3, 5, 8)
    v = np.broadcast_to(c, q.shape).copy()
    o, _ = oracle.attn_fwd(q, k, v, causal=causal)
    assert np.max(np.abs(o - c)) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_gives_mean_of_v(causal):
    _, k, v = _qkv(1, 2, 40, 8, 13)
    q = np.zeros_like(k)
    o, lse = oracle.attn_fwd(q, k, v, causal=causal)
    N = q.shape[2]
    if causal:
        counts = np.arange(1, N + 1, dtype=np.float64)
        mean = np.cumsum(v, axis=2) / counts[None, None, :, None]
        want_lse = np.broadcast_to(np.log(counts), lse.shape)
    else:
        mean = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        want_lse = np.full(lse.shape, np.log(N))
    assert np.max(np.abs(o - mean)) <= 1e-13
    assert np.max(np.abs(lse - want_lse)) <= 1e-13


def test_equal_keys_give_mean_of_v():
    q, k, v = _qkv(1, 1, 30, 8, 14)
    k[:] = k[:, :, :1, :]          # every key row identical -> equal scores per query
    o, lse = oracle.attn_fwd(q, k, v)
    assert np.max(np.abs(o - v.mean(axis=2, keepdims=True))) <= 1e-13
    # LSE = s + ln N with s the common score
    s = (q[0, 0] @ k[0, 0, 0]) / np.sqrt(8)
    assert np.max(np.abs(lse[0, 0] - (s + np.log(30)))) <= 1e-12


def test_causal_row0_returns_v0():
    q, k, v = _qkv(2, 2, 16, 8, 15)
    o, lse = oracle.attn_fwd(q, k, v, causal=True, scale=0.37)
    assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :])
    want = 0.37 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    assert np.max(np.abs(lse[:, :, 0] - want)) <= 1e-14


def _mp_attention(q, k, v, causal, scale):
    import mpmath as mp
    mp.mp.dps = 50
    N, d = q.shape
    O = [[None] * d for _ in range(N)]
    L = [None] * N
    for i in range(N):
        js = range(i + 1) if causal else range(N)
        s = {j: mp.mpf(scale) * mp.fsum(mp.mpf(q[i, c]) * mp.mpf(k[j, c]) for c in range(d)) for j in js}
        z = mp.fsum(mp.e ** s[j] for j in js)
        for c in range(d):
            O[i][c] = mp.fsum(mp.e ** s[j] * mp.mpf(v[j, c]) for j in js) / z
        L[i] = mp.log(z)
    return np.array([[float(x) for x in row] for row in O]), np.array([float(x) for x in L])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 1), (3, 2), (5, 4), (8, 3)])
def test_brute_force_mpmath(causal, N, d):
    g = np.random.default_rng(100 + N * 10 + d)
    q, k, v = (g.standard_normal((1, 1, N, d)) * 2 for _ in range(3))
    scale = 0.7
    o, lse = oracle.attn_fwd(q, k, v, causal=causal, scale=scale)
    o_mp, l_mp = _mp_attention(q[0, 0], k[0, 0], v[0, 0], causal, scale)
    assert np.max(np.abs(o[0, 0] - o_mp)) <= 1e-13
    assert np.max(np.abs(lse[0, 0] - l_mp)) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(causal):
    import torch
    import torch.nn.functional as F
    q, k, v = _qkv(2, 3, 65, 32, 16)
    o, _ = oracle.attn_fwd(q, k, v, causal=causal)
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                             torch.from_numpy(v), is_causal=causal).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12


def test_joint_kv_permutation_invariance():
    q, k, v = _qkv(1, 2, 33, 8, 17)
    perm = np.random.default_rng(5).permutation(33)
    o1, l1 = oracle.attn_fwd(q, k, v)
    o2, l2 = oracle.attn_fwd(q, k[:, :, perm], v[:, :, perm])
    assert np.max(np.abs(o1 - o2)) <= 1e-13
    assert np.max(np.abs(l1 - l2)) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift(causal):
    q, k, v = _qkv(1, 2, 29, 8, 18)
    c = np.random.default_rng(6).standard_normal(8)
    o1, l1 = oracle.attn_fwd(q, k, v, causal=causal)
    o2, l2 = oracle.attn_fwd(q, k + c, v, causal=causal)
    scale = 1 / np.sqrt(8)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs((l2 - l1) - scale * (q @ c))) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_row_subset_matches_full(causal):
    q, k, v = _qkv(2, 2, 47, 16, 19)
    o, lse = oracle.attn_fwd(q, k, v, causal=causal)
    rows = sample_rows(2, 2, 47, 30, 3)
    o_r, l_r = oracle.attn_fwd(q, k, v, causal=causal, rows=rows)
    assert np.array_equal(o_r, o.reshape(-1, 16)[rows])
    assert np.array_equal(l_r, lse.reshape(-1)[rows])


def test_hard_attention_limit():
    # scale -> large: softmax concentrates on the arg-max key (distinct scores)
    q, k, v = _qkv(1, 1, 20, 8, 20)
    o, _ = oracle.attn_fwd(q, k, v, scale=1e4)
    s = q[0, 0] @ k[0, 0].T
    am = np.argmax(s, axis=1)
    assert np.max(np.abs(o[0, 0] - v[0, 0, am])) <= 1e-9
