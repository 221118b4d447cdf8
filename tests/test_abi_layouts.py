"""Property checks of the C ABI's layout validation (no GPU): every layout the
library accepts maps (b, h, i, c) one-to-one onto element offsets (checked by
enumerating the offsets of small shapes), and every dense layout -- any order
of the batch, head and sequence dimensions, with or without padding between
rows, heads or batches -- is accepted.  Pointers are never dereferenced and no
kernel is launched: the probe is flash_attn_bwd without a workspace, whose
layout checks (the forward's) come before the workspace check, so an
accepted layout reports FLASH_ATTN_ERR_WORKSPACE."""
import itertools

import pytest
from hypothesis import given, settings, strategies as st

import exact_attention_77_amd as fa

P = 4096  # a 16-byte aligned fake address; never dereferenced on these paths
ACCEPTED, REJECTED = 7, 3   # FLASH_ATTN_ERR_WORKSPACE after the layout checks, FLASH_ATTN_ERR_LAYOUT


def status(lay):
    return fa.load().flash_attn_bwd(P, P, P, P, P, P, P, P, P, lay, fa.DTYPE_BF16, 0, 0.125, None, 0, None)


def one_to_one(lay):
    offs = {b * lay.stride_b + h * lay.stride_h + i * lay.stride_s + c
            for b in range(lay.batch) for h in range(lay.heads)
            for i in range(lay.seqlen) for c in range(lay.head_dim)}
    return len(offs) == lay.batch * lay.heads * lay.seqlen * lay.head_dim


@settings(max_examples=400, deadline=None)
@given(B=st.integers(1, 3), H=st.integers(1, 3), N=st.integers(1, 4), d=st.sampled_from([64, 128]),
       sb=st.integers(0, 96), sh=st.integers(0, 96), ss=st.integers(0, 96))
def test_every_accepted_layout_is_one_to_one(B, H, N, d, sb, sh, ss):
    # strides in units of 8 elements (16 bytes of bf16), so alignment never decides
    lay = fa.Layout(B, H, N, d, 8 * sb, 8 * sh, 8 * ss)
    s = status(lay)
    assert s in (ACCEPTED, REJECTED)
    if s == ACCEPTED:
        assert one_to_one(lay), lay


@settings(max_examples=200, deadline=None)
@given(B=st.integers(1, 4), H=st.integers(1, 4), N=st.integers(1, 6), d=st.sampled_from([64, 128]),
       order=st.sampled_from(list(itertools.permutations("bhs"))),
       pads=st.tuples(st.integers(0, 3), st.integers(0, 3), st.integers(0, 3)))
def test_every_dense_layout_is_accepted(B, H, N, d, order, pads):
    # innermost first: order[0] steps over head_dim (+ padding), and so on outwards
    ext = {"b": B, "h": H, "s": N}
    stride, span = {}, d
    for dim, pad in zip(order, pads):
        stride[dim] = span + 8 * pad
        span = stride[dim] * ext[dim]
    lay = fa.Layout(B, H, N, d, stride["b"], stride["h"], stride["s"])
    assert one_to_one(lay)
    if stride["s"] >= d:   # the ABI requires a row stride of at least head_dim
        assert status(lay) == ACCEPTED, lay


@pytest.mark.parametrize("elt_off", [1, 2, 4])
def test_unaligned_strides_rejected(elt_off):
    # a bf16 stride that is not a multiple of 8 elements breaks 16-byte rows
    for lay in (fa.Layout(1, 2, 3, 64, 0, 3 * 64 + elt_off, 64),
                fa.Layout(1, 2, 3, 64, 0, 3 * 72, 64 + elt_off)):
        assert status(lay) == REJECTED
