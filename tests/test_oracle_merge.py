"""Pins of the oracle's (O, LSE) merge (oracle.merge) against attention over
all keys computed by the oracle's own pinned forward: splitting the keys into
disjoint sets, attending to each set and merging must reproduce attention
over the union (the rescaling identity of the FlashAttention analysis page,
sec. 6.3), in any order of the parts.  The forward oracle takes as many
queries as keys, so the full problem repeats the queries once per part and
keeps the first copy's rows (every row is independent without a mask)."""
import numpy as np
import pytest

import oracle


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


@pytest.mark.parametrize("parts", [2, 3, 4])
def test_split_keys_reproduces_full_attention(parts):
    B, H, N, d = 2, 3, 24, 16
    q = _rand((B, H, N, d), 1)
    k = 1.7 * _rand((B, H, parts * N, d), 2)
    v = _rand((B, H, parts * N, d), 3)
    o_full, l_full = oracle.attn_fwd(np.concatenate([q] * parts, axis=2), k, v)
    o_full, l_full = o_full[:, :, :N], l_full[:, :, :N]
    os, ls = [], []
    for s in range(parts):
        o_s, l_s = oracle.attn_fwd(q, k[:, :, s * N:(s + 1) * N], v[:, :, s * N:(s + 1) * N])
        os.append(o_s)
        ls.append(l_s)
    o, lse = oracle.merge(np.stack(os), np.stack(ls))
    assert np.max(np.abs(o - o_full)) < 1e-12
    assert np.max(np.abs(lse - l_full)) < 1e-12
    perm = np.random.Generator(np.random.PCG64(parts)).permutation(parts)
    o2, lse2 = oracle.merge(np.stack(os)[perm], np.stack(ls)[perm])
    assert np.max(np.abs(o2 - o_full)) < 1e-12 and np.max(np.abs(lse2 - l_full)) < 1e-12


def test_single_part_is_identity():
    o = _rand((1, 2, 5, 8), 4)
    lse = _rand((1, 2, 5), 5)
    mo, ml = oracle.merge(o, lse)
    assert np.array_equal(mo, o[0]) and np.allclose(ml, lse[0], rtol=0, atol=1e-15)


def test_two_equal_parts_double_the_sum():
    o = _rand((2, 7, 8), 6)
    lse = _rand((2, 7), 7)
    mo, ml = oracle.merge(np.stack([o, o]), np.stack([lse, lse]))
    assert np.max(np.abs(mo - o)) < 1e-14
    assert np.max(np.abs(ml - (lse + np.log(2.0)))) < 1e-14


def test_extreme_lse_and_empty_parts():
    # weights exp(LSE_s - LSE) of widely separated parts: the larger one wins
    o = np.stack([np.full((1, 4), 2.0), np.full((1, 4), -3.0)])
    lse = np.array([[800.0], [0.0]])
    mo, ml = oracle.merge(o, lse)
    assert np.allclose(mo, 2.0) and ml[0] == 800.0
    # a part with no keys (LSE = -inf) contributes nothing
    lse = np.array([[0.5], [-np.inf]])
    mo, ml = oracle.merge(o, lse)
    assert np.allclose(mo, 2.0) and ml[0] == 0.5
    # no keys at all: O = 0, LSE = -inf
    mo, ml = oracle.merge(o, np.full((2, 1), -np.inf))
    assert np.all(mo == 0.0) and ml[0] == -np.inf


def test_empty_part_with_undefined_output_adds_nothing():
    # an empty shard's normalised output is 0/0: its weight is 0 and so is its
    # contribution, NaN or not
    o = np.stack([np.full((2, 4), 2.0), np.full((2, 4), np.nan), np.full((2, 4), np.inf)])
    lse = np.array([[0.5, -1.0], [-np.inf, -np.inf], [-np.inf, 3.0]])
    mo, ml = oracle.merge(o, lse)
    assert np.array_equal(mo[0], np.full(4, 2.0)) and ml[0] == 0.5
    assert np.all(np.isinf(mo[1]))          # row 1: the third part carries weight
