"""GPU parity of the fp32 / bf16 forward kernels against the fp64 oracle.

All calls go through the C ABI (via the ctypes binding).  Inputs are seeded
synthetic tensors from synth_inputs; the oracle receives the exact fp64 values
the GPU consumed.  Tolerances (max |err| over the compared elements):
  fp32: O and LSE <= 1e-5;   bf16: O <= 2e-2, LSE <= 1e-2.
Every shape is compared on every element (several tiles and a ragged tail,
and the full-size workloads), except the N = 65536 case beyond the
workloads, which is compared on seeded rows.
"""
import math

import numpy as np
import pytest

import oracle
from synth_inputs import WORKLOADS, normal_qkv, sample_rows, to_bf16

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-2)}


def _torch():
    import torch
    return torch


def _inputs(B, H, N, d, seed, dtype):
    torch = _torch()
    q, k, v = normal_qkv(B, H, N, d, seed)
    if dtype == "bf16":
        tens, ref = zip(*(to_bf16(x) for x in (q, k, v)))
    else:
        tens = [torch.from_numpy(x) for x in (q, k, v)]
        ref = [x.astype(np.float64) for x in (q, k, v)]
    dev = [t.cuda() for t in tens]
    return dev, ref


def _run(dev, causal, **kw):
    import exact_attention_77_amd as fa
    torch = _torch()
    o, lse = fa.flash_attn_fwd(*dev, causal=causal, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(o, lse, ref, causal, dtype, rows=None, scale=None):
    o_ref, l_ref = oracle.attn_fwd(*ref, causal=causal, rows=rows, scale=scale)
    d = o.shape[-1]
    if rows is not None:
        o = o.reshape(-1, d)[rows]
        lse = lse.reshape(-1)[rows]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    tol_o, tol_l = TOL[dtype]
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse - l_ref)))
    print(f"max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= tol_o, eo
    # an fp32 LSE cannot come closer than a few of its own ulps (2^-24
    # relative): beyond |LSE| = 40 the bound grows with the magnitude
    assert np.all(np.abs(lse - l_ref) <= np.maximum(tol_l, 2.0 ** -22 * np.abs(l_ref))), el


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_f32_workload(causal):
    w = WORKLOADS["tiny_f32"]
    dev, ref = _inputs(w.B, w.H, w.N, w.d, w.seed, "f32")
    o, lse = _run(dev, causal)
    _check(o, lse, ref, causal, "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 64, 255, 600, 1000])
def test_parity_full_compare(dtype, causal, d, N):
    dev, ref = _inputs(2, 3, N, d, 1000 + N + d, dtype)
    o, lse = _run(dev, causal)
    _check(o, lse, ref, causal, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("tile_cfg", [0, 1, 2])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_tile_configs(tile_cfg, causal, d, dtype):
    """Every workgroup shape (automatic, 8 waves, 4 waves) on a ragged N."""
    dev, ref = _inputs(1, 4, 1000, d, 77, dtype)
    o, lse = _run(dev, causal, tile_cfg=tile_cfg)
    _check(o, lse, ref, causal, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("tau", [0.0, 8.0, 64.0])
def test_tau_agree(tau, dtype):
    # Large-magnitude scores make the running maximum move a lot.
    dev, ref = _inputs(1, 2, 700, 64, 78, dtype)
    scale = 1.0
    o, lse = _run(dev, True, tau_log2=tau, scale=scale)
    _check(o, lse, ref, True, dtype, scale=scale)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mag", [40.0, 400.0])
def test_late_dominant_key(causal, mag, dtype):
    """Key 777 of 1000 aligns with every query (a shared component of 6 on
    head dim 0), so its score jumps far above everything before it: by ~25
    (log2) with mag 40, which must trigger a rescale, and by ~300 with mag
    400, where exp2 relative to the earlier maximum would leave the fp32
    range."""
    torch = _torch()
    B, H, N, d = 1, 2, 1000, 128
    q, k, v = normal_qkv(B, H, N, d, 82)
    q[..., 0] += 6.0
    k[:, :, 777, :] = 0.0
    k[:, :, 777, 0] = mag
    if dtype == "bf16":
        tens, ref = zip(*(to_bf16(x) for x in (q, k, v)))
    else:
        tens = [torch.from_numpy(x) for x in (q, k, v)]
        ref = [x.astype(np.float64) for x in (q, k, v)]
    o, lse = _run([t.cuda() for t in tens], causal)
    _check(o, lse, ref, causal, dtype)
    if mag == 400.0:  # rows that see key 777 return (almost exactly) V[777]
        first = 777 if causal else 0
        assert np.max(np.abs(o[0, 0, first:] - ref[2][0, 0, 777])) <= TOL[dtype][0]


def test_bf16_bnhd_layout():
    """[B, N, H, d] memory viewed as [B, H, N, d] through strides."""
    torch = _torch()
    B, N, H, d = 2, 300, 3, 128
    q, k, v = normal_qkv(B, N, H, d, 79)          # drawn as [B, N, H, d]
    tens, ref = zip(*(to_bf16(x) for x in (q, k, v)))
    dev = [t.cuda().transpose(1, 2) for t in tens]  # views [B, H, N, d]
    o, lse = _run(dev, True)
    ref_bhnd = [np.ascontiguousarray(r.transpose(0, 2, 1, 3)) for r in ref]
    _check(o, lse, ref_bhnd, True, "bf16")


def test_bf16_deterministic():
    torch = _torch()
    import exact_attention_77_amd as fa
    dev, _ = _inputs(2, 4, 777, 128, 80, "bf16")
    o1, l1 = fa.flash_attn_fwd(*dev, causal=True)
    o2, l2 = fa.flash_attn_fwd(*dev, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_nan_input_stays_in_its_tiles():
    """Non-finite inputs are outside the contract: the rows that use them get
    unspecified values (the kernels are compiled assuming no NaN operands).
    What still holds: a call with a NaN completes, and causal rows whose key
    range never includes that key's K/V tile are unaffected."""
    torch = _torch()
    import exact_attention_77_amd as fa
    dev, ref = _inputs(1, 1, 130, 64, 81, "bf16")
    dev[2][0, 0, 100, 3] = float("nan")            # one V entry, key 100
    o, lse = fa.flash_attn_fwd(*dev, causal=True)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    o_ref, l_ref = oracle.attn_fwd(*ref, causal=True)
    # causal rows < 64 never load keys >= 64
    assert np.max(np.abs(o[0, 0, :64] - o_ref[0, 0, :64])) <= 2e-2
    assert np.max(np.abs(lse[0, 0, :64] - l_ref[0, 0, :64])) <= 1e-2


def test_empty_seqlen():
    torch = _torch()
    import exact_attention_77_amd as fa
    z = torch.empty((2, 3, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.flash_attn_fwd(z, z, z)
    assert o.shape == z.shape and lse.shape == (2, 3, 0)


@pytest.mark.parametrize("name", ["bf16_n2048_d64", "bf16_causal_n8192_d128", "f32_causal_n4096_d128"])
def test_full_size_workload_all_rows(name, margin):
    """The benchmark's launch configuration at full size, every row of every
    head against the oracle (B4 H16 N2048 d64 non-causal; B2 H16 N8192 d128
    causal, the headline; the fp32 path at B2 H16 N4096 d128 causal)."""
    w = WORKLOADS[name]
    print(f"full size {name}: B{w.B} H{w.H} N{w.N} d{w.d} causal={w.causal}", flush=True)
    dev, ref = _inputs(w.B, w.H, w.N, w.d, w.seed, w.dtype)
    o, lse = _run(dev, w.causal)
    o_ref, l_ref = oracle.attn_fwd(*ref, causal=w.causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    eo, el = np.abs(o - o_ref), np.abs(lse - l_ref)
    tol_o, tol_l = TOL[w.dtype]
    margin(f"{name} all {o.shape[0] * o.shape[1] * o.shape[2]} rows: max|dO|={eo.max():.3e} "
           f"({eo.max() / tol_o:.0%} of {tol_o}) RMSE(O)={np.sqrt(np.mean(eo ** 2)):.3e} "
           f"max|dLSE|={el.max():.3e} ({el.max() / tol_l:.0%} of {tol_l})")
    assert eo.max() <= tol_o and el.max() <= tol_l


@pytest.mark.parametrize("causal", [False, True])
def test_long_sequence_sampled(causal):
    """N = 65536, eight times the longest workload: 1024 key tiles per head,
    so long chains of online-softmax updates; seeded rows (including the
    first and last rows of both heads) against the oracle."""
    B, H, N, d = 1, 2, 65536, 128
    dev, ref = _inputs(B, H, N, d, 11, "bf16")
    o, lse = _run(dev, causal)
    rows = sample_rows(B, H, N, 256, 11)
    _check(o, lse, ref, causal, "bf16", rows=rows)
