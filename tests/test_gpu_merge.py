"""GPU parity of the (O, LSE) merge against the fp64 oracle merge.

All calls go through the C ABI.  The oracle receives the exact values the GPU
consumed (bf16 parts upcast exactly).  Tolerances (max |err|): LSE <= 1e-5
(fp32 arithmetic of a log-sum-exp of a few terms); O <= 1e-5 for fp32 parts;
O <= 2e-2 for bf16 parts (one bf16 rounding of |O| <= 4, as for the forward).
End to end, forwards over disjoint key sets merged on the GPU must match the
oracle's attention over all the keys within the bf16 forward tolerance.
"""
import numpy as np
import pytest

import oracle
from synth_inputs import normal_qkv, to_bf16

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-5, "bf16": 2e-2}
TOL_LSE = 1e-5


def _torch():
    import torch
    return torch


def _parts(S, B, H, N, d, seed, dtype, empty_rows=()):
    g = np.random.Generator(np.random.PCG64(seed))
    o = g.standard_normal((S, B, H, N, d)).astype(np.float32)
    lse = (5.0 + 3.0 * g.standard_normal((S, B, H, N))).astype(np.float32)
    if S > 1:
        lse[0, 0, 0, : min(N, 3)] = -np.inf          # a part with no keys for some rows
    for r in empty_rows:                            # rows with no key in any part
        lse[:, 0, 0, r] = -np.inf
    torch = _torch()
    if dtype == "bf16":
        t, ref = to_bf16(o)
    else:
        t, ref = torch.from_numpy(o), o.astype(np.float64)
    return t.cuda(), torch.from_numpy(lse).cuda(), ref, lse.astype(np.float64)


def _merge(o_parts, lse_parts):
    import exact_attention_77_amd as fa
    o, lse = fa.flash_attn_merge(o_parts, lse_parts)
    _torch().cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _compare(o, lse, o_ref, l_ref, tol_o, report=print):
    assert np.array_equal(np.isinf(lse), np.isinf(l_ref))
    fin = np.isfinite(l_ref)
    eo = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    el = float(np.max(np.abs(lse[fin] - l_ref[fin]))) if fin.any() else 0.0
    report(f"max|dO|={eo:.3e} ({eo / tol_o:.0%} of {tol_o}) max|dLSE|={el:.3e} ({el / TOL_LSE:.0%} of {TOL_LSE})")
    assert eo <= tol_o and el <= TOL_LSE


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 37, 300])
@pytest.mark.parametrize("S", [1, 2, 3, 5, 7, 8])
def test_merge_parity(S, N, d, dtype):
    o_parts, lse_parts, ref_o, ref_l = _parts(S, 2, 3, N, d, 100 * S + N + d, dtype,
                                              empty_rows=(N - 1,) if N > 5 else ())
    o, lse = _merge(o_parts, lse_parts)
    o_ref, l_ref = oracle.merge(ref_o, ref_l)
    _compare(o, lse, o_ref, l_ref, TOL_O[dtype])
    if N > 5:  # no key in any part: O = 0, LSE = -inf
        assert np.all(o[0, 0, N - 1] == 0.0) and lse[0, 0, N - 1] == -np.inf


@pytest.mark.parametrize("S", [2, 5])
def test_merge_empty_part_with_nan_output(S):
    """A part with LSE = -inf (no key) whose O is NaN (0/0 of an empty shard)
    must not reach the merged row, in the four-part loop and in the tail."""
    torch = _torch()
    o_parts, lse_parts, ref_o, ref_l = _parts(S, 2, 3, 40, 128, 17 + S, "bf16")
    o_parts[S - 1, 1, 2, :7] = float("nan")
    lse_parts[S - 1, 1, 2, :7] = -float("inf")
    o_parts[0, 0, 0, :3] = float("nan")             # rows 0..2 of part 0 are empty already
    ref_o = o_parts.float().cpu().numpy().astype(np.float64)
    ref_l = lse_parts.cpu().numpy().astype(np.float64)
    o, lse = _merge(o_parts, lse_parts)
    assert np.all(np.isfinite(o))
    o_ref, l_ref = oracle.merge(ref_o, ref_l)
    _compare(o, lse, o_ref, l_ref, TOL_O["bf16"])


def test_merge_strided_parts():
    """Parts stored [S, B, N, H, d] and viewed as [S, B, H, N, d]."""
    torch = _torch()
    o_parts, lse_parts, ref_o, ref_l = _parts(4, 2, 3, 50, 128, 9, "bf16")
    strided = o_parts.permute(0, 1, 3, 2, 4).contiguous().permute(0, 1, 3, 2, 4)
    assert not strided.is_contiguous() and torch.equal(strided, o_parts)
    o, lse = _merge(strided, lse_parts)
    o_ref, l_ref = oracle.merge(ref_o, ref_l)
    _compare(o, lse, o_ref, l_ref, TOL_O["bf16"])


@pytest.mark.parametrize("parts", [2, 4])
def test_forward_over_key_shards_then_merge(parts):
    """Attention of N queries over parts * N keys: one GPU forward per key
    shard, merged on the GPU, against the oracle over all the keys (the
    oracle takes as many queries as keys, so it gets the queries repeated)."""
    import exact_attention_77_amd as fa
    torch = _torch()
    B, H, N, d = 2, 4, 256, 128
    q, _, _ = normal_qkv(B, H, N, d, 40)
    _, k, v = normal_qkv(B, H, parts * N, d, 41)
    qt, qr = to_bf16(q)
    kt, kr = to_bf16(k)
    vt, vr = to_bf16(v)
    qd = qt.cuda()
    os_, ls_ = [], []
    for s in range(parts):
        ks = kt[:, :, s * N:(s + 1) * N].contiguous().cuda()
        vs = vt[:, :, s * N:(s + 1) * N].contiguous().cuda()
        o_s, l_s = fa.flash_attn_fwd(qd, ks, vs)
        os_.append(o_s)
        ls_.append(l_s)
    o, lse = _merge(torch.stack(os_), torch.stack(ls_))
    o_ref, l_ref = oracle.attn_fwd(np.concatenate([qr] * parts, axis=2), kr, vr)
    eo = float(np.max(np.abs(o - o_ref[:, :, :N])))
    el = float(np.max(np.abs(lse - l_ref[:, :, :N])))
    print(f"end to end: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= 2e-2 and el <= 1e-2


def test_merge_full_size_all_rows(margin):
    """Eight parts of the headline shape (B=2, H=16, N=8192, d=128, bf16),
    every row against the oracle merge."""
    torch = _torch()
    import exact_attention_77_amd as fa
    from synth_inputs import WORKLOADS, merge_parts
    w = WORKLOADS["merge_bf16_s8_n8192_d128"]
    o_parts, lse_parts = merge_parts(w, "cuda")
    o, lse = fa.flash_attn_merge(o_parts, lse_parts)
    torch.cuda.synchronize()
    op = o_parts.float().cpu().numpy().astype(np.float64)
    lp = lse_parts.cpu().numpy().astype(np.float64)
    o_ref, l_ref = oracle.merge(op, lp)
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    rows = og.shape[0] * og.shape[1] * og.shape[2]
    _compare(og, lg, o_ref, l_ref, TOL_O["bf16"],
             lambda line: margin(f"merge {w.name} all {rows} rows: {line} RMSE(O)="
                                 f"{np.sqrt(np.mean((og - o_ref) ** 2)):.3e}"))
