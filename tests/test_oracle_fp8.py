"""Pins of the oracle's FP8 pieces: the OCP e4m3fn codec, the Hadamard rotation
and block quantisation ("FlashAttention-3: Fast and Accurate Attention with
Asynchrony and Low-precision", sec. 技術 3: FP8 e4m3, per-block scales,
M = diag(+-1) * Hadamard with (QM)(KM)^T = QK^T).

Checked against library routines (torch.float8_e4m3fn casts, scipy's Sylvester
Hadamard matrix) and against closed forms (orthogonality, exact round trip of
every code, ties-to-even at every midpoint, saturation).
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import hadamard_signs


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_all_codes():
    ours = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.nanmax(ours) == 448.0 and np.nanmin(ours) == -448.0
    assert ours[1] == 2.0 ** -9          # smallest subnormal


def test_round_trip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    back = oracle.e4m3_encode(oracle.e4m3_decode(codes))
    assert np.array_equal(back, codes)


def test_midpoints_round_to_even():
    vals = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))   # 0 .. 448, increasing
    mids = (vals[:-1] + vals[1:]) / 2
    got = oracle.e4m3_encode(mids)
    lo = np.arange(0, 0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_encode_matches_torch_random():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 150)])
    x = np.clip(x, -460, 460)
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_saturation_and_nan():
    got = oracle.e4m3_encode(np.array([449.0, 1e9, np.inf, -500.0, -np.inf, np.nan, 464.0]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x7E]


@pytest.mark.parametrize("d", [2, 16, 64, 128])
def test_rotation_matches_scipy_hadamard(d):
    from scipy.linalg import hadamard
    signs = hadamard_signs(d)
    eye = np.eye(d)
    rot = oracle.rotate(eye, signs)         # rows: e_i -> s_i H[i, :] / sqrt(d)
    want = np.diag(signs.astype(np.float64)) @ hadamard(d).astype(np.float64) / np.sqrt(d)
    assert np.max(np.abs(rot - want)) <= 1e-15
    assert np.max(np.abs(rot @ rot.T - eye)) <= 1e-14      # orthogonal


def test_rotation_preserves_scores():
    g = np.random.default_rng(1)
    q = g.standard_normal((3, 128))
    k = g.standard_normal((5, 128))
    s = hadamard_signs(128)
    qm, km = oracle.rotate(q, s), oracle.rotate(k, s)
    assert np.max(np.abs(qm @ km.T - q @ k.T)) <= 1e-12


def test_quantize_blocks_properties():
    g = np.random.default_rng(2)
    x = g.standard_normal((1, 2, 70, 16))
    x[0, 1, 64:] = 0.0                       # an all-zero short block
    codes, scales = oracle.quantize_blocks(x, 32)
    assert scales.shape == (1, 2, 3)
    assert scales[0, 1, 2] == 1.0 and np.all(codes[0, 1, 64:] == 0)
    vals = oracle.e4m3_decode(codes)
    for h in range(2):
        for b in range(3):
            blk = x[0, h, 32 * b: 32 * b + 32]
            amax = np.max(np.abs(blk))
            if amax == 0:
                continue
            assert scales[0, h, b] == amax / 448.0
            vb = vals[0, h, 32 * b: 32 * b + 32]
            assert np.max(np.abs(vb)) == 448.0           # the amax element maps to 448
    deq = oracle.dequantize_blocks(codes, scales, 32)
    # relative error of e4m3 RNE for normals is at most 2^-4
    nz = np.abs(x) > 0
    rel = np.abs(deq - x)[nz] / np.maximum(np.abs(x)[nz], 2 ** -6 * np.repeat(scales, 32, axis=2)[:, :, :70, None].repeat(16, -1)[nz])
    assert np.max(rel) <= 2 ** -4 + 1e-12


def test_per_tensor_baseline_is_worse_than_exact_on_outliers():
    from synth_inputs import normal_qkv
    q, k, v = normal_qkv(1, 1, 256, 64, 9, outliers=True)
    o, _ = oracle.attn_fwd(q, k, v)
    o1, _ = oracle.fp8_per_tensor_baseline(q, k, v)
    rmse = np.sqrt(np.mean((o1 - o) ** 2))
    assert 1e-4 < rmse < 0.2


def test_quantize_blocks_pow2_scales():
    g = np.random.default_rng(3)
    x = g.standard_normal((1, 1, 128, 8)) * np.array([1.0, 7.0, 0.01, 448.0 / 4])[None, None, :, None].repeat(32, 2).reshape(1, 1, 128, 1)
    codes, scales = oracle.quantize_blocks(x, 32, pow2=True)
    for b in range(4):
        amax = np.max(np.abs(x[0, 0, 32 * b: 32 * b + 32]))
        sc = scales[0, 0, b]
        m, e = np.frexp(sc)
        assert m == 0.5                               # a power of two
        assert sc >= amax / 448.0 > sc / 2            # the smallest one above amax/448
    vals = oracle.e4m3_decode(codes)
    assert np.max(np.abs(vals)) <= 448.0
    # a block whose amax/448 is exactly a power of two keeps that scale
    y = np.zeros((1, 1, 4, 4)); y[0, 0, 0, 0] = 448.0 * 2.0 ** -3
    _, s2 = oracle.quantize_blocks(y, 4, pow2=True)
    assert s2[0, 0, 0] == 2.0 ** -3


# ---- the per-tensor fp8 baseline's probability path, by closed forms ----
# "FlashAttention-3: ...", 数値誤差: the comparison baseline is standard
# attention with per-tensor fp8 scaling.  Its probabilities enter the product
# with V as e4m3(256 p) / 256 while the row sum keeps the unquantised p (a
# reading of a point the page leaves open).  Inputs below are chosen so that
# every quantised operand is exact (amax 448 gives the per-tensor scale 1 and
# every entry is an e4m3 value), so the expected results are hand-written.

def test_per_tensor_baseline_zero_q_gives_mean_of_v():
    # Q = 0: every score is 0, every p = 1 and e4m3(256)/256 = 1 exactly.
    v = np.array([[448.0, -3.0], [0.5, 12.0], [-0.25, 1.125], [7.0, -448.0], [2.0, 0.0]])
    q = np.zeros((1, 1, 5, 2))
    k = np.random.default_rng(4).standard_normal((1, 1, 5, 2))
    o, lse = oracle.fp8_per_tensor_baseline(q, k, v[None, None])
    assert np.max(np.abs(o[0, 0] - v.mean(axis=0))) <= 1e-13
    assert np.max(np.abs(lse - np.log(5.0))) <= 1e-15


def _two_key_case(p1):
    """q = (448, 0), keys (0, 0) and (-448, 0), scale = -ln(p1)/448^2: the
    scores are 0 and ln(p1), so the probabilities are 1 and p1."""
    q = np.array([[[[448.0, 0.0]]]])
    k = np.array([[[[0.0, 0.0], [-448.0, 0.0]]]])
    v = np.array([[[[448.0, 1.0], [-16.0, 3.0]]]])
    scale = -np.log(p1) / 448.0 ** 2
    # a single query row: repeat the query so that Q, K, V share one shape
    q2 = np.concatenate([q, q], axis=2)
    return q2, k, v, scale


@pytest.mark.parametrize("kexp", [0, 3, 9, 17])
def test_per_tensor_baseline_power_of_two_probabilities(kexp):
    # p1 = 2^-k: 256 p1 is an e4m3 value for k <= 17 (2^-9 is the smallest
    # subnormal), so R1 = (v0 + 2^-k v1) / (1 + 2^-k) exactly.
    p1 = 2.0 ** -kexp
    q, k, v, scale = _two_key_case(p1)
    o, lse = oracle.fp8_per_tensor_baseline(q, k, v, scale=scale)
    want = (v[0, 0, 0] + p1 * v[0, 0, 1]) / (1.0 + p1)
    assert np.max(np.abs(o[0, 0, 0] - want)) <= 1e-12
    assert abs(lse[0, 0, 0] - np.log(1.0 + p1)) <= 1e-12


def test_per_tensor_baseline_rounds_p_not_the_row_sum():
    # p1 = 0.3: 256 * 0.3 = 76.8 lies between the e4m3 values 72 and 80 and
    # rounds to 80, so the weight of key 1 is 80/256 = 0.3125 while the row
    # sum keeps 1 + 0.3.
    q, k, v, scale = _two_key_case(0.3)
    o, _ = oracle.fp8_per_tensor_baseline(q, k, v, scale=scale)
    want = (v[0, 0, 0] + 0.3125 * v[0, 0, 1]) / 1.3
    assert np.max(np.abs(o[0, 0, 0] - want)) <= 1e-12
