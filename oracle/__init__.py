"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``exact_attention_77_amd``) and neither imports the other.

The numerics live in ``oracle.c`` (plain two-pass fp64 attention, its analytic
gradient, an OCP e4m3 codec, a dense Hadamard rotation and block quantisation);
this module compiles it with gcc on first use and wraps it with ctypes over
numpy arrays.  The (O, LSE) merge of partial results is plain numpy here.  See ``oracle.c`` for the passages each function follows:
"FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析" sec. 2.1, 6.1,
7.2, 11.3 and "FlashAttention-3: Fast and Accurate Attention with Asynchrony and
Low-precision" sec. 技術 3 / 数値誤差.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
closed forms, invariants, brute force in 50-digit arithmetic (mpmath) and
library routines (torch fp64 SDPA, torch.float8_e4m3fn, scipy's Hadamard).
The fp8 P-quantisation rule of the per-tensor baseline (``p_quant=1``:
e4m3(256 p)/256 in the product with V, the row sum of the unquantised p) is a
reading of a point the pages leave open; its arithmetic is pinned by closed
forms on exactly representable inputs (tests/test_oracle_fp8.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test of the pins themselves may point the wrapper at a deliberately broken
# build of oracle.c (see tests/test_oracle_mutants.py); nothing else sets this.
_LIB_OVERRIDE = os.environ.get("ORACLE_LIB_OVERRIDE")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2 -fopenmp)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


_NATIVE = os.path.join(_HERE, "liboracle_native.so")
_use_native = False


# Flags of the host-tuned build that use_native_build() makes.
NATIVE_CFLAGS = ("-O3", "-march=native", "-ffp-contract=off", "-fopenmp")


def use_native_build() -> str:
    """Compile oracle.c for the host it runs on (gcc -O3 -march=native, FMA
    contraction off so the rounding is that of the plain build, no fast-math)
    and make this process load that build.  For timing the oracle as a CPU
    baseline; must be called before the first oracle call."""
    global _use_native
    if _lib is not None:
        raise RuntimeError("the oracle library is already loaded")
    tmp = _NATIVE + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *NATIVE_CFLAGS, "-fPIC", "-shared", "-std=c11", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _NATIVE)
    _use_native = True
    return _NATIVE


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if _LIB_OVERRIDE:
                lib = ctypes.CDLL(_LIB_OVERRIDE)
            elif _use_native:
                lib = ctypes.CDLL(_NATIVE)
            else:
                build()
                lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I = ctypes.c_int64
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_attn_fwd_rows.argtypes = [P, P, P, I, I, I, I, ctypes.c_int,
                                                 ctypes.c_double, ctypes.c_int, P, I, P, P]
            lib.oracle_attn_probs_row.argtypes = [P, P, I, I, I, I, ctypes.c_int,
                                                  ctypes.c_double, I, P]
            lib.oracle_attn_bwd_rows.argtypes = [P, P, P, P, I, I, I, I, ctypes.c_int,
                                                 ctypes.c_double, P, I, P, I, P, P, P]
            lib.oracle_e4m3_encode.argtypes = [P, I, P]
            lib.oracle_e4m3_decode.argtypes = [P, I, P]
            lib.oracle_rotate_rows.argtypes = [P, I, I, P, P]
            lib.oracle_quantize_blocks.argtypes = [P, I, I, I, I, ctypes.c_int, P, P]
            _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(_load().oracle_num_threads())


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None,
             rows=None, p_quant: bool = False):
    """Exact attention O = softmax(scale*QK^T) V and LSE = m + ln(l), fp64.

    q, k, v: [B, H, N, d] (any float dtype; upcast to fp64 exactly).
    rows: None for every row, else flat row ids (b*H + h)*N + i.
    Returns (o, lse): o is [B, H, N, d] / [len(rows), d], lse [B, H, N] / [len(rows)].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lib = _load()
    if rows is None:
        o = np.empty((B, H, N, d), np.float64)
        lse = np.empty((B, H, N), np.float64)
        lib.oracle_attn_fwd_rows(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, int(causal),
                                 float(scale), int(p_quant), None, 0, _ptr(o), _ptr(lse))
        return o, lse
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    assert r.ndim == 1 and (r.size == 0 or (r.min() >= 0 and r.max() < B * H * N))
    o = np.empty((r.size, d), np.float64)
    lse = np.empty((r.size,), np.float64)
    if r.size:
        lib.oracle_attn_fwd_rows(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, int(causal),
                                 float(scale), int(p_quant), _ptr(r), r.size, _ptr(o), _ptr(lse))
    return o, lse


def attn_probs_row(q, k, flat_row: int, causal: bool = False, scale: float | None = None):
    """Row P[i, :] of the probability matrix of one (b, h); zeros where masked."""
    q, k = _f64(q), _f64(k)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    p = np.empty((N,), np.float64)
    _load().oracle_attn_probs_row(_ptr(q), _ptr(k), B, H, N, d, int(causal), float(scale),
                                  int(flat_row), _ptr(p))
    return p


def attn_bwd(q, k, v, dout, causal: bool = False, scale: float | None = None,
             qrows=None, krows=None):
    """Analytic gradient (dQ, dK, dV) of the exact-attention definition, fp64.

    With qrows/krows None every row is returned as [B, H, N, d]; otherwise the
    selected rows as [len(rows), d].
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lib = _load()
    full = qrows is None and krows is None
    if full:
        dq = np.empty((B, H, N, d)); dk = np.empty((B, H, N, d)); dv = np.empty((B, H, N, d))
        lib.oracle_attn_bwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, N, d, int(causal),
                                 float(scale), None, 0, None, 0, _ptr(dq), _ptr(dk), _ptr(dv))
        return dq, dk, dv
    qr = np.ascontiguousarray(np.asarray([] if qrows is None else qrows, dtype=np.int64))
    kr = np.ascontiguousarray(np.asarray([] if krows is None else krows, dtype=np.int64))
    dq = np.empty((max(qr.size, 1), d)); dk = np.empty((max(kr.size, 1), d)); dv = np.empty((max(kr.size, 1), d))
    lib.oracle_attn_bwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, N, d, int(causal),
                             float(scale), _ptr(qr), qr.size, _ptr(kr), kr.size,
                             _ptr(dq), _ptr(dk), _ptr(dv))
    return dq[:qr.size], dk[:kr.size], dv[:kr.size]


def e4m3_encode(x) -> np.ndarray:
    """OCP e4m3fn codes (uint8) of x: RNE, saturating at +-448, NaN -> 0x7F."""
    x = _f64(x)
    out = np.empty(x.shape, np.uint8)
    _load().oracle_e4m3_encode(_ptr(x), x.size, _ptr(out))
    return out


def e4m3_decode(codes) -> np.ndarray:
    """Values (fp64) of OCP e4m3fn codes."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, np.float64)
    _load().oracle_e4m3_decode(_ptr(c), c.size, _ptr(out))
    return out


def rotate(x, signs) -> np.ndarray:
    """Incoherent processing x -> (x * signs) H_d / sqrt(d), dense, along the last axis."""
    x = _f64(x)
    d = x.shape[-1]
    s = np.ascontiguousarray(np.asarray(signs, dtype=np.int8))
    assert s.shape == (d,) and d & (d - 1) == 0
    out = np.empty_like(x)
    _load().oracle_rotate_rows(_ptr(x), x.size // d, d, _ptr(s), _ptr(out))
    return out


def quantize_blocks(x, block_rows: int, pow2: bool = False):
    """Per-block e4m3 quantisation of x [B, H, N, d] -> (codes uint8, scales [B, H, nblk]).

    scale = amax(block)/448, or its power-of-two ceiling when pow2 is set."""
    x = _f64(x)
    B, H, N, d = x.shape
    nblk = (N + block_rows - 1) // block_rows
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty((B, H, nblk), np.float64)
    _load().oracle_quantize_blocks(_ptr(x), B * H, N, d, int(block_rows), int(bool(pow2)),
                                   _ptr(codes), _ptr(scales))
    return codes, scales


def dequantize_blocks(codes, scales, block_rows: int) -> np.ndarray:
    """Inverse of quantize_blocks in fp64 (code value times its block's scale)."""
    vals = e4m3_decode(codes)
    B, H, N, d = vals.shape
    rep = np.repeat(np.asarray(scales, np.float64), block_rows, axis=2)[:, :, :N]
    return vals * rep[..., None]


def quantize_per_tensor(x):
    """One scale for the whole tensor: amax/448 (1 if all zero) -> (codes, scale)."""
    x = _f64(x)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    sc = amax / 448.0 if amax > 0 else 1.0
    return e4m3_encode(x / sc), sc


def fp8_per_tensor_baseline(q, k, v, causal: bool = False, scale: float | None = None, rows=None):
    """Comparison baseline R1: per-tensor e4m3 Q, K, V (no rotation), P through
    e4m3(p*256)/256, everything else fp64 ("standard attention FP8, per-tensor
    scale" of the FP8 error comparison)."""
    deq = []
    for x in (q, k, v):
        c, sc = quantize_per_tensor(x)
        deq.append(e4m3_decode(c) * sc)
    return attn_fwd(deq[0], deq[1], deq[2], causal=causal, scale=scale, rows=rows, p_quant=True)


def merge(o_parts, lse_parts):
    """Attention over the union of disjoint key sets from the results over each
    set, fp64 ("FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析"
    sec. 6.2-6.3: the running sum and output are rescaled to a common maximum
    and added; here every part is already normalised, so its sum is exp(LSE_s)).

    o_parts: [S, ..., d] normalised outputs; lse_parts: [S, ...] natural-log LSE.
    Returns (o, lse) with LSE = ln sum_s exp(LSE_s) and
    o = sum_s exp(LSE_s - LSE) o_s.  A part with LSE_s = -inf adds nothing
    (even if its o_s is not finite); a row whose parts all have LSE = -inf (no
    key at all) gets o = 0 and LSE = -inf.
    """
    o = _f64(o_parts)
    lse = _f64(lse_parts)
    assert o.shape[:-1] == lse.shape and lse.shape[0] >= 1
    m = lse.max(axis=0)                      # common reference: the largest LSE
    alive = np.isfinite(m)
    m0 = np.where(alive, m, 0.0)
    w = np.exp(lse - m0)                     # exp(-inf) = 0 for empty parts
    total = w.sum(axis=0)
    lse_out = np.where(alive, m0 + np.log(np.where(alive, total, 1.0)), -np.inf)
    frac = np.where(alive, w / np.where(alive, total, 1.0), 0.0)
    # a part of weight 0 contributes nothing, whatever its O holds (an empty
    # part's O may be undefined, e.g. 0/0)
    terms = np.where(frac[..., None] > 0, frac[..., None] * np.where(frac[..., None] > 0, o, 0.0), 0.0)
    return terms.sum(axis=0), lse_out


def bf16_round(x) -> np.ndarray:
    """x rounded to the nearest bfloat16 value (8 significant bits, ties to
    even), returned as fp64.  Written from the format: x = m * 2^e with
    m in [0.5, 1); m * 2^8 is rounded to the nearest integer, ties to even
    (numpy's rint), and scaled back.  Normal range only (|x| >= 2^-126 or 0),
    which covers every value it is used on here."""
    x = _f64(x)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def attn_bwd_bf16_baseline(q, k, v, dout, causal: bool = False, scale: float | None = None):
    """Comparison baseline for the bf16 backward: standard (non-fused)
    attention whose materialised intermediates are stored in bf16, in the
    comparison style of the FP16 rows of "FlashAttention-3: ...", 数値誤差
    ("standard attention" against an fp64 reference).  Per (b, h), in fp64:
    P = softmax(scale Q K^T) (masked), O = bf16(P V);
    dV = bf16(P)^T dO;  dP = dO V^T;  D = rowsum(dO o O);
    dS = bf16(P o (dP - D));  dQ = scale dS K;  dK = scale dS^T Q;
    each gradient rounded to bf16 at the end.  The roundings are the ones a
    bf16 implementation cannot avoid (P and dS enter products as bf16, O and
    the gradients are stored as bf16); everything else is exact fp64."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq, dk, dv = (np.empty_like(q) for _ in range(3))
    mask = np.tril(np.ones((N, N), dtype=bool)) if causal else None
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            if causal:
                s = np.where(mask, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o = bf16_round(p @ v[b, h])
            dv[b, h] = bf16_round(bf16_round(p).T @ dout[b, h])
            dp = dout[b, h] @ v[b, h].T
            D = np.sum(dout[b, h] * o, axis=1, keepdims=True)
            ds = bf16_round(p * (dp - D))
            dq[b, h] = bf16_round(scale * (ds @ k[b, h]))
            dk[b, h] = bf16_round(scale * (ds.T @ q[b, h]))
    return dq, dk, dv
