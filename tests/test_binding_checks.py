"""The Python binding rejects tensors the kernels cannot take before any
library call or device use: wrong device, shapes, dtypes, contiguity, the fp8
padding and scale counts, the Hadamard signs and caller-supplied outputs.
Host only: every tensor here is a CPU tensor, so the device check (made last)
is the expected error only when everything else is right."""
import pytest
import torch

import exact_attention_77_amd as fa

ERR_NULL, ERR_SHAPE, ERR_LAYOUT, ERR_DTYPE, ERR_ARG = 1, 2, 3, 4, 6


def _status(fn, *a, **kw):
    with pytest.raises(fa.FlashAttnError) as e:
        fn(*a, **kw)
    return e.value.status


def _qkv(B=1, H=2, N=100, d=64, dtype=torch.bfloat16):
    return [torch.zeros((B, H, N, d), dtype=dtype) for _ in range(3)]


def test_fwd_rejects_host_tensors():
    assert _status(fa.flash_attn_fwd, *_qkv()) == ERR_ARG


def test_fwd_rejects_bad_lse_and_out():
    q, k, v = _qkv()
    assert _status(fa.flash_attn_fwd, q, k, v, lse=torch.zeros((1, 2, 99))) == ERR_SHAPE
    assert _status(fa.flash_attn_fwd, q, k, v, lse=torch.zeros((1, 2, 100), dtype=torch.float64)) == ERR_DTYPE
    assert _status(fa.flash_attn_fwd, q, k, v, lse=torch.zeros((1, 100, 2)).transpose(1, 2)) == ERR_LAYOUT
    assert _status(fa.flash_attn_fwd, q, k, v, out=torch.zeros((1, 2, 100, 64))) == ERR_LAYOUT


def _fp8_inputs(B=1, H=2, N=100, d=128):
    npad = (N + 63) // 64 * 64
    q8 = torch.zeros((2, B, H, N, d), dtype=torch.uint8)
    k8 = torch.zeros((B, H, N, d), dtype=torch.uint8)
    v8 = torch.zeros((B, H, d, npad), dtype=torch.uint8)
    qs = torch.ones((B, H, (N + 31) // 32))
    ks = torch.ones((B, H, (N + 31) // 32))
    vs = torch.ones((B, H, npad // 64))
    return [q8, k8, v8, qs, ks, vs]


def test_fwd_fp8_rejects_host_tensors():
    assert _status(fa.flash_attn_fwd_fp8, *_fp8_inputs()) == ERR_ARG


def test_fwd_fp8_rejects_single_plane_q():
    a = _fp8_inputs()
    a[0] = a[0][0].contiguous()                          # [B, H, N, d]: the residual plane missing
    assert _status(fa.flash_attn_fwd_fp8, *a) == ERR_SHAPE


def test_fwd_fp8_rejects_unpadded_v():
    a = _fp8_inputs()
    a[2] = torch.zeros((1, 2, 128, 100), dtype=torch.uint8)    # N_pad must be 128
    assert _status(fa.flash_attn_fwd_fp8, *a) == ERR_SHAPE


@pytest.mark.parametrize("which", [3, 4, 5])
def test_fwd_fp8_rejects_bad_scales(which):
    a = _fp8_inputs()
    good = a[which]
    a[which] = good[..., :-1].contiguous()
    assert _status(fa.flash_attn_fwd_fp8, *a) == ERR_SHAPE
    a[which] = good.double()
    assert _status(fa.flash_attn_fwd_fp8, *a) == ERR_LAYOUT
    a[which] = torch.ones(good.shape[::-1]).transpose(0, 2)   # right count, not contiguous
    assert _status(fa.flash_attn_fwd_fp8, *a) == ERR_LAYOUT


def test_fwd_fp8_rejects_bad_out_and_lse():
    a = _fp8_inputs()
    assert _status(fa.flash_attn_fwd_fp8, *a, out=torch.zeros((1, 2, 100, 128))) == ERR_DTYPE
    assert _status(fa.flash_attn_fwd_fp8, *a, out=torch.zeros((1, 2, 99, 128), dtype=torch.bfloat16)) == ERR_SHAPE
    assert _status(fa.flash_attn_fwd_fp8, *a, lse=torch.zeros((1, 2, 100), dtype=torch.bfloat16)) == ERR_DTYPE


def test_quantize_rejects_bad_signs_and_host_tensors():
    x = torch.zeros((1, 2, 100, 128))
    assert _status(fa.flash_attn_fp8_quantize, x, fa.ROLE_Q, rotate=True) == ERR_NULL
    assert _status(fa.flash_attn_fp8_quantize, x, fa.ROLE_Q, rotate=True,
                   signs=torch.ones(128)) == ERR_DTYPE
    assert _status(fa.flash_attn_fp8_quantize, x, fa.ROLE_Q, rotate=True,
                   signs=torch.ones(64, dtype=torch.int8)) == ERR_SHAPE
    assert _status(fa.flash_attn_fp8_quantize, x, fa.ROLE_Q, rotate=True,
                   signs=torch.ones(256, dtype=torch.int8)[::2]) == ERR_LAYOUT
    assert _status(fa.flash_attn_fp8_quantize, x, 7) == ERR_ARG
    assert _status(fa.flash_attn_fp8_quantize, x, fa.ROLE_Q, rotate=True,
                   signs=torch.ones(128, dtype=torch.int8)) == ERR_ARG


def test_bwd_rejects_host_tensors():
    q, k, v = _qkv()
    lse = torch.zeros((1, 2, 100))
    assert _status(fa.flash_attn_bwd, q, k, v, q, lse, q) == ERR_ARG


def test_bwd_dtypes():
    """One dtype for every tensor, bfloat16 or float32; fp32 host tensors get
    as far as the device check."""
    q, k, v = _qkv()
    qf, kf, vf = _qkv(dtype=torch.float32)
    lse = torch.zeros((1, 2, 100))
    assert _status(fa.flash_attn_bwd, qf, kf, vf, qf, lse, qf) == ERR_ARG
    assert _status(fa.flash_attn_bwd, q, kf, v, q, lse, q) == ERR_DTYPE
    assert _status(fa.flash_attn_bwd, q.half(), k.half(), v.half(), q.half(), lse, q.half()) == ERR_DTYPE
    assert _status(fa.flash_attn_bwd_noalloc, qf, kf, vf, qf, lse, qf, qf, kf, q) == ERR_DTYPE


def test_merge_rejects_out_of_another_shape():
    parts = torch.zeros((3, 2, 2, 50, 64), dtype=torch.bfloat16)
    lse = torch.zeros((3, 2, 2, 50))
    small = torch.zeros((3, 1, 2, 50, 64), dtype=torch.bfloat16)[0]   # same strides, one batch
    assert small.stride() == parts.stride()[1:]
    assert _status(fa.flash_attn_merge, parts, lse, out=small) == ERR_LAYOUT
    assert _status(fa.flash_attn_merge, parts, lse, lse=torch.zeros((2, 2, 49))) == ERR_SHAPE
    assert _status(fa.flash_attn_merge, parts, lse) == ERR_ARG
