"""C-ABI checks that need no GPU: the library loads, exports every function
include/flash_attn.h declares, and rejects bad arguments with the documented
status codes before any HIP call (pointers here are never dereferenced)."""
import ctypes
import os
import re

import pytest

import exact_attention_77_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flash_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flash_attn_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strings():
    assert fa.flash_attn_abi_version() == 2
    for code, name in fa.STATUS.items():
        assert fa.flash_attn_status_str(code) == name
    lay = _lay(B=2, H=3, N=130, d=128)
    assert fa.flash_attn_fp8_buffer_bytes(lay, fa.ROLE_Q) == 2 * 2 * 3 * 130 * 128   # code + residual term
    assert fa.flash_attn_fp8_buffer_bytes(lay, fa.ROLE_K) == 2 * 3 * 130 * 128
    assert fa.flash_attn_fp8_buffer_bytes(lay, fa.ROLE_V) == 2 * 3 * 192 * 128   # padded to 64 keys
    assert fa.flash_attn_fp8_num_scales(lay, fa.ROLE_Q) == 2 * 3 * 5
    assert fa.flash_attn_fp8_num_scales(lay, fa.ROLE_K) == 2 * 3 * 5
    assert fa.flash_attn_fp8_num_scales(lay, fa.ROLE_V) == 2 * 3 * 3
    assert fa.flash_attn_fp8_num_scales(lay, 7) == 0


def _lay(B=1, H=2, N=128, d=64, sb=None, sh=None, ss=None):
    ss = d if ss is None else ss
    sh = N * ss if sh is None else sh
    sb = H * sh if sb is None else sb
    return fa.Layout(B, H, N, d, sb, sh, ss)


P = 4096  # a 16-byte aligned fake address; never dereferenced on these paths


def fwd(q=P, k=P, v=P, o=P, lse=P, lay=None, dtype=fa.DTYPE_BF16, causal=0, scale=0.125,
        opts=None):
    return fa.load().flash_attn_fwd(q, k, v, o, lse, lay or _lay(), dtype, causal, scale, opts, None)


def test_null_pointers():
    for kw in ("q", "k", "v", "o", "lse"):
        assert fwd(**{kw: None}) == 1


def test_empty_inputs_are_noops():
    assert fwd(q=None, k=None, v=None, o=None, lse=None, lay=_lay(N=0)) == 0
    assert fwd(q=None, k=None, v=None, o=None, lse=None, lay=_lay(B=0)) == 0
    assert fwd(q=None, k=None, v=None, o=None, lse=None, lay=_lay(H=0)) == 0


@pytest.mark.parametrize("lay", [_lay(N=-1), _lay(B=-2), _lay(N=(1 << 24) + 1),
                                 fa.Layout(1 << 13, 1 << 12, 16, 64, 64, 64, 64),
                                 # each size within its limit, the row count 2^32 beyond int32
                                 fa.Layout(1 << 12, 1 << 12, 1 << 8, 64, 64, 64, 64),
                                 fa.Layout(1, 1 << 8, 1 << 24, 64, 64, 64, 64)])
def test_bad_shapes(lay):
    assert fwd(lay=lay) == 2


@pytest.mark.parametrize("d", [32, 96, 256])
def test_unsupported_head_dim(d):
    assert fwd(lay=_lay(d=d)) == 5


@pytest.mark.parametrize("lay", [_lay(ss=60), _lay(ss=68), _lay(sh=8), _lay(sb=4, H=1, B=2),
                                 _lay(N=2, ss=(1 << 24) + 8)])   # row stride beyond 2^24 elements
def test_bad_strides(lay):
    assert fwd(lay=lay) == 3


def test_row_stride_limit():
    # 2^24 elements is accepted (the backward's workspace check comes next)
    lay = _lay(N=2, ss=1 << 24)
    assert fa.load().flash_attn_bwd(P, P, P, P, P, P, P, P, P, lay, fa.DTYPE_BF16, 0, 0.125,
                                    None, 0, None) == 7


@pytest.mark.parametrize("lay", [
    # rows of different (b, h, i) that share memory: two workgroups would write
    # the same output element
    fa.Layout(1, 2, 2, 64, 128, 64, 64),          # stride_h == stride_s
    fa.Layout(1, 2, 4, 64, 1024, 128, 64),        # head 1 starts inside head 0's rows
    fa.Layout(2, 2, 4, 64, 128, 256, 64),         # batch 1 starts inside head 0 of batch 0
    fa.Layout(2, 1, 8, 64, 0, 512, 64),           # batch stride 0 with two batches
    fa.Layout(1, 3, 2, 128, 0, 192, 128)])        # head 1 starts inside head 0's second row
def test_overlapping_rows_rejected(lay):
    assert fwd(lay=lay) == 3
    assert fa.load().flash_attn_bwd(P, P, P, P, P, P, P, P, P, lay, fa.DTYPE_BF16, 0, 0.125,
                                    P, 1 << 30, None) == 3


@pytest.mark.parametrize("lay", [
    fa.Layout(2, 3, 5, 64, 3 * 5 * 64, 5 * 64, 64),   # [B, H, N, d]
    fa.Layout(2, 3, 5, 64, 5 * 3 * 64, 64, 3 * 64),   # [B, N, H, d]
    fa.Layout(1, 4, 1, 128, 0, 128, 128),            # one row: its stride is irrelevant
    fa.Layout(3, 1, 7, 64, 7 * 64 + 64, 0, 64)])     # one head, padded batches
def test_one_to_one_layouts_accepted(lay):
    # flash_attn_bwd checks the forward's layout rules before its workspace:
    # without a workspace an accepted layout reports FLASH_ATTN_ERR_WORKSPACE
    # (no kernel is launched)
    assert fa.load().flash_attn_bwd(P, P, P, P, P, P, P, P, P, lay, fa.DTYPE_BF16, 0, 0.125,
                                    None, 0, None) == 7


def test_misaligned_pointers():
    assert fwd(q=P + 2) == 3
    assert fwd(o=P + 8) == 3
    assert fwd(lse=P + 2) == 3


def test_bad_dtype():
    assert fwd(dtype=fa.DTYPE_FP8_E4M3) == 4
    assert fwd(dtype=7) == 4


@pytest.mark.parametrize("scale", [0.0, -1.0, float("inf"), float("nan"), 3e38])
def test_bad_scale(scale):
    assert fwd(scale=scale) == 6


def test_bad_causal_flag():
    assert fwd(causal=2) == 6


@pytest.mark.parametrize("opts", [fa.FwdOpts(65.0, 0, 0), fa.FwdOpts(float("nan"), 0, 0),
                                  fa.FwdOpts(8.0, 9, 0), fa.FwdOpts(8.0, 3, 0), fa.FwdOpts(8.0, -1, 0),
                                  fa.FwdOpts(8.0, 0, 3), fa.FwdOpts(8.0, 0, -1)])
def test_bad_options(opts):
    assert fwd(opts=ctypes.byref(opts)) == 6


def test_f32_strides_need_16_bytes():
    # 4 floats = 16 bytes: stride 68 ok for f32 alignment, 66 is not
    assert fwd(lay=_lay(ss=66), dtype=fa.DTYPE_F32) == 3


def test_quantize_validation():
    lib = fa.load()
    lay = _lay()
    assert lib.flash_attn_fp8_quantize(P, 1, lay, fa.ROLE_Q, 1, None, P, P, None) == 1   # rotate needs signs
    assert lib.flash_attn_fp8_quantize(P, 1, lay, 5, 0, None, P, P, None) == 6           # unknown role
    assert lib.flash_attn_fp8_quantize(P, 1, lay, fa.ROLE_V, 1, P, P, P, None) == 6      # V is never rotated
    assert lib.flash_attn_fp8_quantize(P, 2, lay, fa.ROLE_Q, 0, None, P, P, None) == 4
    assert lib.flash_attn_fp8_quantize(None, 1, _lay(N=0), 0, 0, None, None, None, None) == 0


def test_fp8_fwd_validation():
    lib = fa.load()
    lay = _lay()
    assert lib.flash_attn_fwd_fp8(P, P, P, P, P, P, P, None, lay, 0, 0.1, None, None) == 1
    assert lib.flash_attn_fwd_fp8(P, P, P, P, P, P, P, P, lay, 0, -0.1, None, None) == 6
    assert lib.flash_attn_fwd_fp8(P, P, P, P, P, P, P, P, _lay(d=80), 0, 0.1, None, None) == 5


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fa, "_lib", None)
    with pytest.raises(fa.FlashAttnError):
        fa.load()


def bwd(lay=None, dtype=fa.DTYPE_BF16, causal=0, scale=0.125, ws=P, ws_bytes=1 << 40, **ptrs):
    p = {n: P for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv")}
    p.update(ptrs)
    return fa.load().flash_attn_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], p["dq"],
                                    p["dk"], p["dv"], lay or _lay(), dtype, causal, scale, ws,
                                    ws_bytes, None)


def test_bwd_workspace_size():
    lay = _lay(B=2, H=3, N=130, d=128)
    rows = 2 * 3 * 130
    part = lambda n: (4 * n + 255) // 256 * 256
    assert fa.flash_attn_bwd_workspace_size(lay) == 2 * part(rows)
    assert fa.flash_attn_bwd_workspace_size(lay, fa.DTYPE_F32) == 2 * part(rows)
    assert fa.flash_attn_bwd_workspace_size(lay, fa.DTYPE_FP8_E4M3) == 0
    assert fa.flash_attn_bwd_workspace_size(_lay(N=0)) == 0
    assert fa.flash_attn_bwd_workspace_size(_lay(d=96)) == 0


def test_bwd_validation():
    for name in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv"):
        assert bwd(**{name: None}) == 1, name
    # fp32 is accepted: the same checks apply, with fp32 element strides
    for name in ("q", "dout", "dv"):
        assert bwd(dtype=fa.DTYPE_F32, **{name: None}) == 1, name
    assert bwd(dtype=fa.DTYPE_F32, lay=_lay(ss=66)) == 3     # rows not 16-byte aligned
    assert bwd(dtype=fa.DTYPE_F32, ws=None) == 7
    assert bwd(dtype=fa.DTYPE_F32, dk=P + 4) == 3
    assert bwd(dtype=fa.DTYPE_FP8_E4M3) == 4
    assert bwd(causal=2) == 6
    assert bwd(scale=float("nan")) == 6
    assert bwd(lay=_lay(d=80)) == 5
    assert bwd(lay=_lay(ss=60)) == 3
    assert bwd(dq=P + 2) == 3
    need = fa.flash_attn_bwd_workspace_size(_lay())
    assert bwd(ws=None) == 7
    assert bwd(ws_bytes=need - 1) == 7
    assert bwd(ws=P + 16, ws_bytes=need) == 7
    assert bwd(lay=_lay(N=0), ws=None, ws_bytes=0, **{n: None for n in ("q", "k", "v", "o", "lse",
                                                                      "dout", "dq", "dk", "dv")}) == 0


def merge(o_parts=P, lse_parts=P, n=2, part_stride=1 << 20, o=P, lse=P, lay=None, dtype=fa.DTYPE_BF16):
    return fa.load().flash_attn_merge(o_parts, lse_parts, n, part_stride, o, lse, lay or _lay(),
                                      dtype, None)


def test_merge_validation():
    assert merge(o_parts=None) == 1 and merge(lse=None) == 1
    assert merge(n=0) == 6 and merge(n=4097) == 6
    assert merge(part_stride=0) == 3 and merge(part_stride=12) == 3
    assert merge(dtype=fa.DTYPE_FP8_E4M3) == 4
    assert merge(lay=_lay(d=96)) == 5
    assert merge(o=P + 8) == 3
    assert merge(o_parts=None, lse_parts=None, o=None, lse=None, lay=_lay(N=0)) == 0


def test_c_consumer_compiles(tmp_path):
    """The C consumer builds against the public header and the two libraries."""
    import importlib.util
    import subprocess
    spec = importlib.util.spec_from_file_location("c_api_build", os.path.join(
        os.path.dirname(os.path.abspath(__file__)), "c_api", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    out = str(tmp_path / "abi_consumer")
    subprocess.run(mod.command(out), check=True)
    assert os.path.getsize(out) > 0


def bwd_noalloc(lay, q=P, lse=P, dtype=fa.DTYPE_BF16):
    return fa.load().flash_attn_bwd_noalloc(q, P, P, P, lse, P, P, P, P, lay, dtype, 0, 0.125, None)


def test_bwd_noalloc_validation():
    # the fixed scratch array holds two fp32 values for at most 2^21 rows
    big = fa.Layout(2, 16, 65537, 64, 16 * 65537 * 64, 65537 * 64, 64)
    assert bwd_noalloc(big) == 7                      # ERR_WORKSPACE, before any HIP call
    assert bwd_noalloc(_lay(N=0)) == 0
    assert bwd_noalloc(_lay(), q=None) == 1
    assert bwd_noalloc(_lay(ss=66), dtype=fa.DTYPE_F32) == 3
    assert bwd_noalloc(_lay(), dtype=fa.DTYPE_FP8_E4M3) == 4
    assert bwd_noalloc(_lay(ss=60)) == 3
    assert bwd_noalloc(_lay(), lse=P + 2) == 3
