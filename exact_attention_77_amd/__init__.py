"""Python binding of libflashattn.so, the gfx950 fused exact-attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/flash_attn.h``.  PyTorch is used
for device memory and the current stream.  The functions carry the C names:

    flash_attn_fwd(q, k, v, causal=False, scale=None) -> (o, lse)
    flash_attn_fp8_quantize(x, role, rotate=False, signs=None) -> (x_fp8, scales)
    flash_attn_fwd_fp8(q8, k8, v8t, qs, ks, vs, causal, scale) -> (o_bf16, lse)
    flash_attn_bwd(q, k, v, o, lse, dout, causal=False, scale=None) -> (dq, dk, dv)
    flash_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal, scale)
    flash_attn_merge(o_parts, lse_parts) -> (o, lse)

If the shared library is missing this module raises on first use: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

__all__ = [
    "FlashAttnError", "lib_path", "load", "flash_attn_fwd", "flash_attn_fp8_quantize",
    "flash_attn_fwd_fp8", "flash_attn_fp8_buffer_bytes", "flash_attn_fp8_num_scales",
    "flash_attn_bwd", "flash_attn_bwd_workspace_size", "flash_attn_bwd_noalloc", "flash_attn_merge",
    "flash_attn_status_str", "flash_attn_last_error", "flash_attn_abi_version", "Layout",
    "FwdOpts", "STATUS", "DTYPE_F32", "DTYPE_BF16", "DTYPE_FP8_E4M3", "ROLE_Q", "ROLE_K",
    "ROLE_V", "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libflashattn.so")
_lock = threading.Lock()
_lib = None

DTYPE_F32, DTYPE_BF16, DTYPE_FP8_E4M3 = 0, 1, 2
ROLE_Q, ROLE_K, ROLE_V = 0, 1, 2
STATUS = {
    0: "FLASH_ATTN_OK", 1: "FLASH_ATTN_ERR_NULL", 2: "FLASH_ATTN_ERR_SHAPE",
    3: "FLASH_ATTN_ERR_LAYOUT", 4: "FLASH_ATTN_ERR_DTYPE", 5: "FLASH_ATTN_ERR_UNSUPPORTED",
    6: "FLASH_ATTN_ERR_ARG", 7: "FLASH_ATTN_ERR_WORKSPACE", 8: "FLASH_ATTN_ERR_HIP",
}
# Every function include/flash_attn.h declares.
EXPORTED_SYMBOLS = (
    "flash_attn_fwd", "flash_attn_fp8_quantize", "flash_attn_fp8_buffer_bytes",
    "flash_attn_fp8_num_scales", "flash_attn_fwd_fp8", "flash_attn_bwd",
    "flash_attn_bwd_workspace_size", "flash_attn_bwd_noalloc", "flash_attn_merge",
    "flash_attn_status_str", "flash_attn_last_error", "flash_attn_abi_version",
)


class FlashAttnError(RuntimeError):
    def __init__(self, status: int, detail: str = ""):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(self.name + (f": {detail}" if detail else ""))


class Layout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("heads", ctypes.c_int64),
                ("seqlen", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_s", ctypes.c_int64)]


class FwdOpts(ctypes.Structure):
    _fields_ = [("tau_log2", ctypes.c_float), ("tile_cfg", ctypes.c_int32),
                ("fp8_q_terms", ctypes.c_int32)]


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libflashattn.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise FlashAttnError(-1, f"{_LIB_PATH} is missing: build it with "
                                     "exact_attention_77_amd/build.py (or __graft_entry__.build())")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.flash_attn_fwd.argtypes = [P, P, P, P, P, Layout, I, I, F, P, P]
        lib.flash_attn_fwd.restype = I
        lib.flash_attn_fp8_quantize.argtypes = [P, I, Layout, I, I, P, P, P, P]
        lib.flash_attn_fp8_quantize.restype = I
        lib.flash_attn_fp8_buffer_bytes.argtypes = [Layout, I]
        lib.flash_attn_fp8_buffer_bytes.restype = ctypes.c_size_t
        lib.flash_attn_fp8_num_scales.argtypes = [Layout, I]
        lib.flash_attn_fp8_num_scales.restype = ctypes.c_int64
        lib.flash_attn_fwd_fp8.argtypes = [P, P, P, P, P, P, P, P, Layout, I, F, P, P]
        lib.flash_attn_fwd_fp8.restype = I
        lib.flash_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, Layout, I, I, F, P,
                                       ctypes.c_size_t, P]
        lib.flash_attn_bwd.restype = I
        lib.flash_attn_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, Layout, I, I, F, P]
        lib.flash_attn_bwd_noalloc.restype = I
        lib.flash_attn_bwd_workspace_size.argtypes = [Layout, I]
        lib.flash_attn_bwd_workspace_size.restype = ctypes.c_size_t
        lib.flash_attn_merge.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, P, P, Layout, I, P]
        lib.flash_attn_merge.restype = I
        lib.flash_attn_status_str.argtypes = [I]
        lib.flash_attn_status_str.restype = ctypes.c_char_p
        lib.flash_attn_last_error.argtypes = []
        lib.flash_attn_last_error.restype = ctypes.c_char_p
        lib.flash_attn_abi_version.argtypes = []
        lib.flash_attn_abi_version.restype = I
        _lib = lib
        return lib


def _check(status: int):
    if status != 0:
        detail = load().flash_attn_last_error().decode() if status == 8 else ""
        raise FlashAttnError(status, detail)


def flash_attn_status_str(status: int) -> str:
    return load().flash_attn_status_str(status).decode()


def flash_attn_last_error() -> str:
    return load().flash_attn_last_error().decode()


def flash_attn_abi_version() -> int:
    return int(load().flash_attn_abi_version())


def flash_attn_fp8_buffer_bytes(layout: Layout, role: int) -> int:
    return int(load().flash_attn_fp8_buffer_bytes(layout, int(role)))


def flash_attn_fp8_num_scales(layout: Layout, role: int) -> int:
    return int(load().flash_attn_fp8_num_scales(layout, int(role)))


def _layout_of(t) -> Layout:
    B, H, N, d = t.shape
    if d and t.stride(3) != 1:
        raise FlashAttnError(3, "head_dim must be the contiguous dimension")
    return Layout(B, H, N, d, t.stride(0), t.stride(1), t.stride(2))


def _need(ok: bool, status: int, msg: str):
    if not ok:
        raise FlashAttnError(status, msg)


def _check_buffer(t, name, dtype, shape, contiguous=True):
    """A caller-supplied output or side input: exact dtype and shape (and
    contiguity where the C ABI fixes the layout)."""
    _need(t.dtype == dtype, 4, f"{name} must be {dtype}, got {t.dtype}")
    _need(tuple(t.shape) == tuple(shape), 2, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous:
        _need(t.is_contiguous(), 3, f"{name} must be contiguous")


def _on_gpu(*named):
    """Every tensor the kernels will read or write must live on the current
    GPU: a host pointer handed to a kernel would fault the device.  Checked
    last, after the shape and dtype checks, so each of those is testable on a
    host without a GPU."""
    import torch
    dev = None
    for name, t in named:
        if t is None:
            continue
        _need(t.is_cuda, 6, f"{name} is not on the GPU (device {t.device})")
        if dev is None:
            dev = t.device
        _need(t.device == dev, 6, f"{name} is on {t.device}, the other tensors on {dev}")
    _need(dev is None or dev.index == torch.cuda.current_device(), 6,
          f"tensors are on {dev}, the current device is cuda:{torch.cuda.current_device()}")


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _opts(tau_log2, tile_cfg, q_terms=0):
    if tau_log2 is None and not tile_cfg and not q_terms:
        return None
    return ctypes.byref(FwdOpts(-1.0 if tau_log2 is None else float(tau_log2), int(tile_cfg),
                                int(q_terms)))


def flash_attn_fwd(q, k, v, causal: bool = False, scale: float | None = None,
                   tau_log2: float | None = None, tile_cfg: int = 0, out=None, lse=None):
    """O = softmax(scale * Q K^T) V and the natural-log LSE, on the GPU.

    q, k, v: CUDA tensors [B, H, N, d] (any strides with a contiguous head_dim,
    so a [B, N, H, d] buffer viewed with .transpose(1, 2) works), all float32 or
    all bfloat16, same shape and strides.  Returns (o, lse) with o like q and
    lse float32 [B, H, N].
    """
    import torch
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise FlashAttnError(4, f"unsupported dtype {q.dtype}")
    if not (q.dtype == k.dtype == v.dtype) or not (q.shape == k.shape == v.shape):
        raise FlashAttnError(2, "q, k, v must share dtype and shape")
    if q.dim() != 4:
        raise FlashAttnError(2, "expected [B, H, N, d] tensors")
    lay = _layout_of(q)
    if k.stride() != q.stride() or v.stride() != q.stride():
        raise FlashAttnError(3, "q, k, v must share strides")
    B, H, N, d = q.shape
    if out is not None and (out.stride() != q.stride() or out.shape != q.shape or out.dtype != q.dtype):
        raise FlashAttnError(3, "out must match q's shape, dtype and strides")
    if lse is not None:
        _check_buffer(lse, "lse", torch.float32, (B, H, N))
    _on_gpu(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse))
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d) if d else 1.0
    dt = DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F32
    _check(load().flash_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr(), lay, dt, int(bool(causal)), float(scale),
                                 _opts(tau_log2, tile_cfg), _stream()))
    return out, lse


def flash_attn_fp8_quantize(x, role: int, rotate: bool = False, signs=None):
    """Rotate (optionally, Q/K) and block-quantise x [B, H, N, d] (f32/bf16) to e4m3.

    Returns (x_fp8, scales): uint8 [2, B, H, N, d] for Q (the code and its
    residual term), [B, H, N, d] for K, the transposed [B, H, d, N_pad] for V;
    fp32 scales [B, H, n_blocks].
    """
    import torch
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise FlashAttnError(4, f"unsupported dtype {x.dtype}")
    _need(x.dim() == 4, 2, "expected an [B, H, N, d] tensor")
    _need(role in (ROLE_Q, ROLE_K, ROLE_V), 6, f"unknown role {role}")
    B, H, N, d = x.shape
    lay = _layout_of(x)
    if rotate:
        _need(signs is not None, 1, "rotate needs the +-1 signs")
        _check_buffer(signs, "signs", torch.int8, (d,))
    _on_gpu(("x", x), ("signs", signs if rotate else None))
    nbytes = flash_attn_fp8_buffer_bytes(lay, role)
    nsc = flash_attn_fp8_num_scales(lay, role)
    if role == ROLE_V:
        npad = (N + 63) // 64 * 64
        out = torch.empty((B, H, d, npad), dtype=torch.uint8, device=x.device)
    elif role == ROLE_Q:   # the code and its residual term
        out = torch.empty((2, B, H, N, d), dtype=torch.uint8, device=x.device)
    else:
        out = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    assert out.numel() == nbytes
    nblk = nsc // max(B * H, 1) if B * H else 0
    scales = torch.empty((B, H, nblk), dtype=torch.float32, device=x.device)
    sp = signs.data_ptr() if (rotate and signs is not None) else None
    dt = DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_F32
    _check(load().flash_attn_fp8_quantize(x.data_ptr(), dt, lay, int(role), int(bool(rotate)), sp,
                                          out.data_ptr(), scales.data_ptr(), _stream()))
    return out, scales


def flash_attn_fwd_fp8(q8, k8, v8t, q_scale, k_scale, v_scale, causal: bool = False,
                       scale: float | None = None, tau_log2: float | None = None,
                       tile_cfg: int = 0, out=None, lse=None, q_terms: int = 0):
    """FP8 attention on the pre-pass outputs (q8 [2, B, H, N, d], k8 [B, H, N, d],
    v8t [B, H, d, N_pad] uint8 and their scales) -> (o bf16 [B, H, N, d], lse fp32 [B, H, N])."""
    import torch
    _need(q8.dim() == 5 and q8.shape[0] == 2, 2, "q8 must be [2, B, H, N, d] (code, residual term)")
    _, B, H, N, d = q8.shape
    for t in (q8, k8, v8t):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise FlashAttnError(3, "fp8 inputs must be contiguous uint8 tensors")
    npad = (N + 63) // 64 * 64
    if tuple(k8.shape) != (B, H, N, d) or tuple(v8t.shape) != (B, H, d, npad):
        raise FlashAttnError(2, f"k8 must match q8 and v8t must be [B, H, d, {npad}]")
    lay = Layout(B, H, N, d, H * N * d, N * d, d)
    for name, t, role in (("q_scale", q_scale, ROLE_Q), ("k_scale", k_scale, ROLE_K),
                          ("v_scale", v_scale, ROLE_V)):
        nsc = flash_attn_fp8_num_scales(lay, role)
        _need(t.dtype == torch.float32 and t.is_contiguous(), 3, f"{name} must be contiguous float32")
        _need(t.numel() == nsc, 2, f"{name} must hold {nsc} scales, got {t.numel()}")
    if out is not None:
        _check_buffer(out, "out", torch.bfloat16, (B, H, N, d), contiguous=False)
        _need(d == 0 or out.stride(3) == 1, 3, "out must have a contiguous head_dim")
    if lse is not None:
        _check_buffer(lse, "lse", torch.float32, (B, H, N))
    _on_gpu(("q8", q8), ("k8", k8), ("v8t", v8t), ("q_scale", q_scale), ("k_scale", k_scale),
            ("v_scale", v_scale), ("out", out), ("lse", lse))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d) if d else 1.0
    _check(load().flash_attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8t.data_ptr(),
                                     q_scale.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(),
                                     out.data_ptr(), lse.data_ptr(), _layout_of(out),
                                     int(bool(causal)), float(scale),
                                     _opts(tau_log2, tile_cfg, q_terms), _stream()))
    return out, lse


def flash_attn_bwd_workspace_size(layout: Layout, dtype: int = DTYPE_BF16) -> int:
    return int(load().flash_attn_bwd_workspace_size(layout, int(dtype)))


def flash_attn_bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
                   dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv) of the forward for the upstream gradient dout.

    q, k, v, o, dout: bfloat16 or float32 CUDA tensors (one dtype for all)
    [B, H, N, d] sharing shape and strides (o and lse are the forward's
    outputs); lse: float32 [B, H, N].  The fp32 workspace is allocated here
    unless given (uint8 tensor of at least flash_attn_bwd_workspace_size bytes).
    """
    import torch
    ts = (q, k, v, o, dout)
    if q.dtype not in (torch.bfloat16, torch.float32) or any(t.dtype != q.dtype for t in ts):
        raise FlashAttnError(4, "the backward takes q, k, v, o, dout of one dtype, bfloat16 or float32")
    dt_code = DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F32
    if q.dim() != 4 or any(t.shape != q.shape for t in ts):
        raise FlashAttnError(2, "q, k, v, o, dout must share a [B, H, N, d] shape")
    if any(t.stride() != q.stride() for t in ts):
        raise FlashAttnError(3, "q, k, v, o, dout must share strides")
    B, H, N, d = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise FlashAttnError(3, "lse must be a contiguous float32 [B, H, N] tensor")
    lay = _layout_of(q)
    for t in (dq, dk, dv):
        if t is not None and (t.stride() != q.stride() or t.shape != q.shape or t.dtype != q.dtype):
            raise FlashAttnError(3, "gradient outputs must match q's shape, dtype and strides")
    if workspace is not None:
        _need(workspace.is_contiguous(), 3, "workspace must be contiguous")
    _on_gpu(("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout), ("dq", dq),
            ("dk", dk), ("dv", dv), ("workspace", workspace))
    outs = [t if t is not None else
            torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
            for t in (dq, dk, dv)]
    need = flash_attn_bwd_workspace_size(lay, dt_code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d) if d else 1.0
    _check(load().flash_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), dout.data_ptr(), outs[0].data_ptr(),
                                 outs[1].data_ptr(), outs[2].data_ptr(), lay, dt_code,
                                 int(bool(causal)), float(scale), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream()))
    return tuple(outs)


def flash_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal: bool = False,
                           scale: float | None = None):
    """The backward into caller-supplied dq, dk, dv without any device
    allocation: the per-row workspace is the library's fixed device array
    (B * H * N <= 2^21 rows).  Same arguments and result as flash_attn_bwd."""
    import torch
    ts = (q, k, v, o, dout, dq, dk, dv)
    if q.dtype not in (torch.bfloat16, torch.float32) or any(t.dtype != q.dtype for t in ts):
        raise FlashAttnError(4, "the backward takes tensors of one dtype, bfloat16 or float32")
    dt_code = DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F32
    if q.dim() != 4 or any(t.shape != q.shape for t in ts):
        raise FlashAttnError(2, "q, k, v, o, dout, dq, dk, dv must share a [B, H, N, d] shape")
    if any(t.stride() != q.stride() for t in ts):
        raise FlashAttnError(3, "q, k, v, o, dout, dq, dk, dv must share strides")
    B, H, N, d = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise FlashAttnError(3, "lse must be a contiguous float32 [B, H, N] tensor")
    lay = _layout_of(q)
    _on_gpu(("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout), ("dq", dq),
            ("dk", dk), ("dv", dv))
    if scale is None:
        scale = 1.0 / math.sqrt(d) if d else 1.0
    _check(load().flash_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                         lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                         dk.data_ptr(), dv.data_ptr(), lay, dt_code,
                                         int(bool(causal)), float(scale), _stream()))
    return dq, dk, dv


def flash_attn_merge(o_parts, lse_parts, out=None, lse=None):
    """Merge results over disjoint key sets: o_parts [S, B, H, N, d] (float32
    or bfloat16, each part with the same strides, head_dim contiguous),
    lse_parts float32 [S, B, H, N] contiguous -> (o [B, H, N, d], lse [B, H, N])."""
    import torch
    if o_parts.dtype not in (torch.float32, torch.bfloat16):
        raise FlashAttnError(4, f"unsupported dtype {o_parts.dtype}")
    if o_parts.dim() != 5 or lse_parts.shape != o_parts.shape[:4]:
        raise FlashAttnError(2, "o_parts [S, B, H, N, d] and lse_parts [S, B, H, N]")
    if lse_parts.dtype != torch.float32 or not lse_parts.is_contiguous():
        raise FlashAttnError(3, "lse_parts must be contiguous float32")
    S, B, H, N, d = o_parts.shape
    lay = _layout_of(o_parts[0])
    if out is not None and (out.stride() != o_parts.stride()[1:] or out.dtype != o_parts.dtype
                            or tuple(out.shape) != (B, H, N, d)):
        raise FlashAttnError(3, "out must have a part's shape, strides and dtype")
    if lse is not None:
        _check_buffer(lse, "lse", torch.float32, (B, H, N))
    _on_gpu(("o_parts", o_parts), ("lse_parts", lse_parts), ("out", out), ("lse", lse))
    if out is None:
        out = torch.empty_strided((B, H, N, d), o_parts.stride()[1:], dtype=o_parts.dtype,
                                  device=o_parts.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    dt = DTYPE_BF16 if o_parts.dtype == torch.bfloat16 else DTYPE_F32
    _check(load().flash_attn_merge(o_parts.data_ptr(), lse_parts.data_ptr(), S, o_parts.stride(0),
                                   out.data_ptr(), lse.data_ptr(), lay, dt, _stream()))
    return out, lse
