"""dense_matrix_unit_amd -- MFMA GEMM (BF16 / scaled FP8) for AMD MI355X.

Thin Python binding over the C ABI of ``libdmu.so`` (``include/dmu.h``): the
functions below only check tensor metadata and marshal pointers, leading
dimensions and the current HIP stream; every step of the computation runs in
the library's HIP kernels.  Tensors must live on the GPU (PyTorch is used for
device memory and streams only).  There is no fallback: if the library is
missing, importing the binding raises.

BF16 operands are passed as ``torch.bfloat16`` (or ``torch.uint16``/``int16``
bit patterns); FP8 operands as ``torch.uint8`` codes (or torch float8
tensors).
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdmu.so")

DMU_OK = 0
DMU_ERR_INVALID_ARG = -1
DMU_ERR_UNSUPPORTED = -2
DMU_ERR_HIP = -3
OUT_F32 = 0
OUT_BF16 = 1
B_ROW_MAJOR = 0
B_COL_MAJOR = 1
E4M3 = 0
E5M2 = 1
SCALE_TENSOR = 0
SCALE_BLOCK = 1
PROBE_BF16_16X16X32 = 0
PROBE_BF16_32X32X16 = 1
PROBE_FP8_16X16X128 = 2
PROBE_FP8_32X32X64 = 3
PROBE_MXFP8_32X32X64 = 4  # rate probe only: scaled form, unit E8M0 scales
PROBE_MXFP4_32X32X64 = 5  # rate probe only: E2M1 operands, unit E8M0 scales
OUT_FP8_E4M3 = 2  # fused entry points: FP8 output with a dequantisation scale
OUT_FP8_E5M2 = 3
ACT_NONE, ACT_RELU, ACT_GELU, ACT_SILU = 0, 1, 2, 3
MX_BLOCK = 32  # values of K per E8M0 scale (DMU_MX_BLOCK)
E2M1 = 4  # FP4 elements of MXFP4 (DMU_FP4_E2M1), packed two per byte
PROBE_MX_16X16X128 = 0  # shapes of dmu_probe_mfma_mx
PROBE_MX_32X32X64 = 1

# (name, restype, argtypes) of every exported C symbol
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
SYMBOLS = {
    "gemm_bf16": (_I, [_P, _I64, _P, _I64, _I, _P, _I64, _P, _I64, _I, _I64, _I64, _I64, _P]),
    "gemm_fp8_scaled": (_I, [_P, _I64, _I, _P, _I64, _I, _P, _P, _I, _P, _I64, _P, _I64, _I,
                             _I64, _I64, _I64, _P]),
    "quantize_fp8": (_I, [_P, _I64, _I64, _I64, _I, _I64, _I64, _P, _I64, _P, _P]),
    "quantize_fp8_noalloc": (_I, [_P, _I64, _I64, _I64, _I, _I64, _I64, _P, _I64, _P, _P]),
    "gemm_bf16_fused": (_I, [_P, _I64, _P, _I64, _I, _P, _I, _P, _I64, _I, _P, _I64, _I64, _I64,
                             _P]),
    "gemm_fp8_fused": (_I, [_P, _I64, _I, _P, _I64, _I, _P, _P, _P, _I, _P, _I64, _I, _P, _I64,
                            _I64, _I64, _P]),
    "gemm_grouped_bf16": (_I, [_P, _I64, _P, _I64, _I64, _P, _I64, _P, _I64, _I, _I64, _I64,
                               _I64, _P]),
    "attention_bf16": (_I, [_P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P,
                            _I64, _I64, _I64, _I64, ctypes.c_float, _I, _P]),
    "gemm_mxfp8": (_I, [_P, _I64, _I, _P, _I64, _I, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _I,
                        _I64, _I64, _I64, _P]),
    "quantize_mxfp8": (_I, [_P, _I64, _I64, _I64, _I, _P, _I64, _P, _I64, _P]),
    "gemm_mxfp4": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _I, _I64,
                        _I64, _I64, _P]),
    "quantize_mxfp4": (_I, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P]),
    "dmu_status_string": (ctypes.c_char_p, [_I]),
    "dmu_version": (_I, []),
    "dmu_probe_mfma": (_I, [_I, _I, _I, _P, _P, _P, _P, _P]),
    "dmu_probe_mfma_batch": (_I, [_I, _I, _I, _P, _P, _P, _P, _I, _P]),
    "dmu_probe_lds_load": (_I, [_P, _P, _I, _I, _P]),
    "dmu_probe_gemm_bf16_layout": (_I, [_I, _P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _P]),
    "dmu_probe_mfma_rate": (_I, [_I, _P, _I, _I, _P, _P]),
    "dmu_probe_cvt_fp8": (_I, [_P, _I64, _I, _I, _P, _P]),
    "dmu_probe_quantize_tensor_resident": (_I, [_P, _I64, _I64, _I, _P, _P, _I, _P]),
    "dmu_probe_lds_tr16": (_I, [_P, _P, _P, _P]),
    "dmu_probe_mfma_mx": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
}

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libdmu.so and declare its C signatures (no GPU needed)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            "libdmu.so is not built (%s); run `python -m dense_matrix_unit_amd.build`" % path)
    L = ctypes.CDLL(path)
    for name, (res, args) in SYMBOLS.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    if path == LIB_PATH:
        _lib = L
    return L


class DmuError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load_library().dmu_status_string(status).decode()
        super().__init__("%s: %s (status %d)" % (fn, msg, status))
        self.status = status


def _check(fn: str, rc: int):
    if rc != DMU_OK:
        raise DmuError(fn, rc)


def _torch():
    import torch

    return torch


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev_ptr(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    return ctypes.c_void_p(t.data_ptr())


def _ld(t, name):
    """Leading dimension (elements) of a 2-D row-major tensor."""
    if t.dim() != 2 or (t.stride(1) != 1 and t.size(1) > 1):
        raise ValueError("%s must be 2-D with unit column stride" % name)
    return t.stride(0)


def _check_dtype(t, allowed, name):
    if t.dtype not in allowed:
        raise TypeError("%s has dtype %s; expected one of %s" % (name, t.dtype, allowed))


def gemm_bf16(A, B, out, b_layout: int = B_COL_MAJOR, C=None, stream=None):
    """out = A @ B (+ C).  A: [M, K] BF16.  B: [K, N] BF16 if b_layout is
    B_ROW_MAJOR, or [N, K] (B stored N x K) if B_COL_MAJOR.  out: [M, N] float32
    or bfloat16.  C: optional [M, N] float32."""
    torch = _torch()
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    _check_dtype(A, bf, "A")
    _check_dtype(B, bf, "B")
    _check_dtype(out, (torch.float32, torch.bfloat16), "out")
    M, K = A.shape
    N = B.shape[1] if b_layout == B_ROW_MAJOR else B.shape[0]
    if (B.shape[0] if b_layout == B_ROW_MAJOR else B.shape[1]) != K:
        raise ValueError("inner dimensions differ")
    if tuple(out.shape) != (M, N):
        raise ValueError("out has shape %s, expected %s" % (tuple(out.shape), (M, N)))
    cptr, ldc = None, 0
    if C is not None:
        _check_dtype(C, (torch.float32,), "C")
        if tuple(C.shape) != (M, N):
            raise ValueError("C shape")
        cptr, ldc = _dev_ptr(C, "C"), _ld(C, "C")
    rc = load_library().gemm_bf16(
        _dev_ptr(A, "A"), _ld(A, "A"), _dev_ptr(B, "B"), _ld(B, "B"), b_layout, cptr, ldc,
        _dev_ptr(out, "out"), _ld(out, "out"),
        OUT_F32 if out.dtype == torch.float32 else OUT_BF16, M, N, K, _stream(stream))
    _check("gemm_bf16", rc)
    return out


def _fused_out(out, out_fmt, out_scale, bias, N):
    """(d_dtype, d_scale pointer, bias pointer) of a fused call."""
    torch = _torch()
    if out.dtype == torch.uint8:
        if out_fmt not in (E4M3, E5M2) or out_scale is None:
            raise ValueError("FP8 output needs out_fmt (E4M3/E5M2) and out_scale")
        _check_dtype(out_scale, (torch.float32,), "out_scale")
        dt = OUT_FP8_E4M3 if out_fmt == E4M3 else OUT_FP8_E5M2
        sp = _dev_ptr(out_scale, "out_scale")
    else:
        _check_dtype(out, (torch.float32, torch.bfloat16), "out")
        dt = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
        sp = None
    bp = None
    if bias is not None:
        _check_dtype(bias, (torch.float32,), "bias")
        if bias.numel() != N or not bias.is_contiguous():
            raise ValueError("bias needs N contiguous floats")
        bp = _dev_ptr(bias, "bias")
    return dt, sp, bp


def gemm_bf16_fused(A, B, out, b_layout: int = B_COL_MAJOR, bias=None, act: int = ACT_NONE,
                    out_fmt=None, out_scale=None, stream=None):
    """out = cast(act(A @ B + bias)).  A, B as gemm_bf16; bias float32 [N] or
    None; out float32, bfloat16, or uint8 FP8 codes (out_fmt E4M3/E5M2 with
    out_scale, a one-float GPU tensor: out ~ decode(q) * out_scale)."""
    torch = _torch()
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    _check_dtype(A, bf, "A")
    _check_dtype(B, bf, "B")
    M, K = A.shape
    N = B.shape[1] if b_layout == B_ROW_MAJOR else B.shape[0]
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape")
    dt, sp, bp = _fused_out(out, out_fmt, out_scale, bias, N)
    rc = load_library().gemm_bf16_fused(
        _dev_ptr(A, "A"), _ld(A, "A"), _dev_ptr(B, "B"), _ld(B, "B"), b_layout, bp, act,
        _dev_ptr(out, "out"), _ld(out, "out"), dt, sp, M, N, K, _stream(stream))
    _check("gemm_bf16_fused", rc)
    return out


def gemm_fp8_fused(A, B, scale_a, scale_b, out, fmt_a: int = E4M3, fmt_b: int = E4M3,
                   bias=None, act: int = ACT_NONE, out_fmt=None, out_scale=None, stream=None):
    """out = cast(act(scale_a * scale_b * (A @ B^T) + bias)), per-tensor FP8
    inputs as gemm_fp8_scaled; out as gemm_bf16_fused."""
    torch = _torch()
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError("shape mismatch")
    _check_dtype(scale_a, (torch.float32,), "scale_a")
    _check_dtype(scale_b, (torch.float32,), "scale_b")
    dt, sp, bp = _fused_out(out, out_fmt, out_scale, bias, N)
    rc = load_library().gemm_fp8_fused(
        _fp8_ptr(A, "A"), _ld(A, "A"), fmt_a, _fp8_ptr(B, "B"), _ld(B, "B"), fmt_b,
        _dev_ptr(scale_a, "scale_a"), _dev_ptr(scale_b, "scale_b"), bp, act,
        _dev_ptr(out, "out"), _ld(out, "out"), dt, sp, M, N, K, _stream(stream))
    _check("gemm_fp8_fused", rc)
    return out


def gemm_grouped_bf16(A, B, offsets, out, stream=None):
    """Mixture-of-experts grouped product: out[r] = A[r] @ B[g].T for rows r in
    [offsets[g], offsets[g+1]).  A: [max_m, K] BF16; B: [G, N, K] BF16 (each
    expert's weight stored N x K); offsets: int64 GPU tensor [G+1] (read on the
    device); out: [max_m, N] float32 or bfloat16 (rows outside every expert's
    range are left as they are)."""
    torch = _torch()
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    _check_dtype(A, bf, "A")
    _check_dtype(B, bf, "B")
    _check_dtype(offsets, (torch.int64,), "offsets")
    _check_dtype(out, (torch.float32, torch.bfloat16), "out")
    if B.dim() != 3 or B.stride(2) != 1 or B.stride(1) < B.shape[2]:
        raise ValueError("B must be [G, N, K] with unit K stride")
    G, N, K = B.shape
    max_m = A.shape[0]
    if A.shape[1] != K or tuple(out.shape) != (max_m, N):
        raise ValueError("shape mismatch")
    if offsets.numel() != G + 1 or not offsets.is_contiguous():
        raise ValueError("offsets needs G + 1 contiguous entries")
    rc = load_library().gemm_grouped_bf16(
        _dev_ptr(A, "A"), _ld(A, "A"), _dev_ptr(B, "B"), B.stride(1), B.stride(0),
        _dev_ptr(offsets, "offsets"), G, _dev_ptr(out, "out"), _ld(out, "out"),
        OUT_F32 if out.dtype == torch.float32 else OUT_BF16, max_m, N, K, _stream(stream))
    _check("gemm_grouped_bf16", rc)
    return out


def attention_bf16(Q, K, V, O, scale: float, causal: bool = False, lse=None, stream=None):
    """O = softmax(scale * Q K^T) V per head (attention_bf16 in dmu.h).  Q, O:
    [heads, Sq, d] BF16; K, V: [heads, Sk, d] BF16 (2-D tensors are one head);
    any row and head strides with a unit d stride.  lse: optional float32
    [heads, Sq] contiguous tensor for log sum_j exp(s_j)."""
    torch = _torch()
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (O, "O")):
        _check_dtype(t, bf, n)
        if t.dim() not in (2, 3) or t.stride(-1) != 1:
            raise ValueError("%s must be [heads, S, d] or [S, d] with a unit d stride" % n)
    def hs(t):
        return t.stride(0) if t.dim() == 3 else 0
    def h3(t):
        return t.shape if t.dim() == 3 else (1,) + tuple(t.shape)
    heads, Sq, d = h3(Q)
    Sk = h3(K)[1]
    if tuple(h3(K)) != (heads, Sk, d) or tuple(h3(V)) != (heads, Sk, d) or \
            tuple(h3(O)) != (heads, Sq, d):
        raise ValueError("shape mismatch")
    lp = None
    if lse is not None:
        _check_dtype(lse, (torch.float32,), "lse")
        if lse.numel() != heads * Sq or not lse.is_contiguous():
            raise ValueError("lse needs heads * Sq contiguous float32 entries")
        lp = _dev_ptr(lse, "lse")
    rc = load_library().attention_bf16(
        _dev_ptr(Q, "Q"), Q.stride(-2), hs(Q), _dev_ptr(K, "K"), K.stride(-2), hs(K),
        _dev_ptr(V, "V"), V.stride(-2), hs(V), _dev_ptr(O, "O"), O.stride(-2), hs(O), lp,
        heads, Sq, Sk, d, float(scale), int(bool(causal)), _stream(stream))
    _check("attention_bf16", rc)
    return O


def _fp8_ptr(t, name):
    torch = _torch()
    _check_dtype(t, (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2), name)
    return _dev_ptr(t, name)


def gemm_fp8_scaled(A, B, scale_a, scale_b, out, fmt_a: int = E4M3, fmt_b: int = E4M3,
                    scale_mode: int = SCALE_TENSOR, C=None, stream=None):
    """out = (A*scale_a) @ (B*scale_b)^T (+ C).  A: [M, K] FP8 codes, B: [N, K]
    FP8 codes (B stored N x K).  scale_a/scale_b: float32 device tensors, one
    element each (SCALE_TENSOR) or [M, K/128] and [ceil(N/128), K/128]
    (SCALE_BLOCK)."""
    torch = _torch()
    _check_dtype(out, (torch.float32, torch.bfloat16), "out")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError("shape mismatch")
    _check_dtype(scale_a, (torch.float32,), "scale_a")
    _check_dtype(scale_b, (torch.float32,), "scale_b")
    if scale_mode == SCALE_BLOCK:
        if tuple(scale_a.shape) != (M, K // 128) or tuple(scale_b.shape) != ((N + 127) // 128, K // 128):
            raise ValueError("block scale shapes")
        if not (scale_a.is_contiguous() and scale_b.is_contiguous()):
            raise ValueError("block scales must be contiguous")
    elif scale_a.numel() < 1 or scale_b.numel() < 1:
        raise ValueError("per-tensor scales need one element")
    cptr, ldc = None, 0
    if C is not None:
        _check_dtype(C, (torch.float32,), "C")
        cptr, ldc = _dev_ptr(C, "C"), _ld(C, "C")
    rc = load_library().gemm_fp8_scaled(
        _fp8_ptr(A, "A"), _ld(A, "A"), fmt_a, _fp8_ptr(B, "B"), _ld(B, "B"), fmt_b,
        _dev_ptr(scale_a, "scale_a"), _dev_ptr(scale_b, "scale_b"), scale_mode, cptr, ldc,
        _dev_ptr(out, "out"), _ld(out, "out"),
        OUT_F32 if out.dtype == torch.float32 else OUT_BF16, M, N, K, _stream(stream))
    _check("gemm_fp8_scaled", rc)
    return out


def quantize_fp8(X, Q, scales, fmt: int = E4M3, block=None, stream=None):
    """Q, scales = FP8 quantisation of X (float32 [rows, cols]).  block: None
    (one scale for the tensor), (1, 128) or (128, 128).  Q: uint8 [rows, cols];
    scales: float32 [rows/br, cols/bc] (dequantisation factors)."""
    return _quantize_fp8("quantize_fp8", X, Q, scales, fmt, block, stream)


def quantize_fp8_noalloc(X, Q, scales, fmt: int = E4M3, block=None, stream=None):
    """quantize_fp8 through the entry point that allocates nothing (static
    scratch; calls overlapping on one GPU race, see include/dmu.h)."""
    return _quantize_fp8("quantize_fp8_noalloc", X, Q, scales, fmt, block, stream)


def _quantize_fp8(fn, X, Q, scales, fmt, block, stream):
    torch = _torch()
    _check_dtype(X, (torch.float32,), "X")
    rows, cols = X.shape
    br, bc = (rows, cols) if block is None else block
    if tuple(Q.shape) != (rows, cols):
        raise ValueError("Q shape")
    if scales.numel() < (rows // br) * (cols // bc) or not scales.is_contiguous():
        raise ValueError("scales must be contiguous with one element per block")
    _check_dtype(scales, (torch.float32,), "scales")
    rc = getattr(load_library(), fn)(
        _dev_ptr(X, "X"), rows, cols, _ld(X, "X"), fmt, br, bc, _fp8_ptr(Q, "Q"), _ld(Q, "Q"),
        _dev_ptr(scales, "scales"), _stream(stream))
    _check(fn, rc)
    return Q, scales


def gemm_mxfp8(A, B, scale_a, scale_b, out, fmt_a: int = E4M3, fmt_b: int = E4M3, C=None,
               stream=None):
    """out = (A x 2^(scale_a-127)) @ (B x 2^(scale_b-127))^T (+ C), microscaled
    FP8.  A: [M, K] FP8 codes, B: [N, K] FP8 codes (B stored N x K), K a
    multiple of 128.  scale_a: uint8 [M, >= K/32] and scale_b: uint8
    [N, >= K/32] E8M0 codes, one per row and 32 values of K, row strides a
    multiple of 4 bytes."""
    torch = _torch()
    _check_dtype(out, (torch.float32, torch.bfloat16), "out")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError("shape mismatch")
    _check_dtype(scale_a, (torch.uint8,), "scale_a")
    _check_dtype(scale_b, (torch.uint8,), "scale_b")
    if scale_a.shape[0] != M or scale_b.shape[0] != N:
        raise ValueError("scale arrays need one row per row of A / stored row of B")
    if scale_a.shape[1] < K // MX_BLOCK or scale_b.shape[1] < K // MX_BLOCK:
        raise ValueError("scale rows need K/32 codes")
    cptr, ldc = None, 0
    if C is not None:
        _check_dtype(C, (torch.float32,), "C")
        if tuple(C.shape) != (M, N):
            raise ValueError("C shape")
        cptr, ldc = _dev_ptr(C, "C"), _ld(C, "C")
    rc = load_library().gemm_mxfp8(
        _fp8_ptr(A, "A"), _ld(A, "A"), fmt_a, _fp8_ptr(B, "B"), _ld(B, "B"), fmt_b,
        _dev_ptr(scale_a, "scale_a"), _ld(scale_a, "scale_a"), _dev_ptr(scale_b, "scale_b"),
        _ld(scale_b, "scale_b"), cptr, ldc, _dev_ptr(out, "out"), _ld(out, "out"),
        OUT_F32 if out.dtype == torch.float32 else OUT_BF16, M, N, K, _stream(stream))
    _check("gemm_mxfp8", rc)
    return out


def quantize_mxfp8(X, Q, S, fmt: int = E4M3, stream=None):
    """Q, S = MX quantisation of X (float32 [rows, cols], cols % 32 == 0): Q
    uint8 [rows, cols] FP8 codes, S uint8 [rows, >= cols/32] E8M0 codes."""
    torch = _torch()
    _check_dtype(X, (torch.float32,), "X")
    _check_dtype(S, (torch.uint8,), "S")
    rows, cols = X.shape
    if tuple(Q.shape) != (rows, cols):
        raise ValueError("Q shape")
    if S.shape[0] != rows or S.shape[1] < cols // MX_BLOCK:
        raise ValueError("S shape")
    rc = load_library().quantize_mxfp8(
        _dev_ptr(X, "X"), rows, cols, _ld(X, "X"), fmt, _fp8_ptr(Q, "Q"), _ld(Q, "Q"),
        _dev_ptr(S, "S"), _ld(S, "S"), _stream(stream))
    _check("quantize_mxfp8", rc)
    return Q, S


def _packed_ld(t, name):
    """Leading dimension, in elements, of a packed E2M1 array held as uint8."""
    return 2 * _ld(t, name)


def gemm_mxfp4(A, B, scale_a, scale_b, out, C=None, stream=None):
    """out = (A x 2^(scale_a-127)) @ (B x 2^(scale_b-127))^T (+ C), microscaled
    FP4.  A: uint8 [M, K/2] and B: uint8 [N, K/2] packed E2M1 (element 2i in
    the low nibble of byte i), K a multiple of 512.  scale_a: uint8
    [M, >= K/32], scale_b: uint8 [N, >= K/32] E8M0 codes, row strides a
    multiple of 16 bytes."""
    torch = _torch()
    _check_dtype(out, (torch.float32, torch.bfloat16), "out")
    _check_dtype(A, (torch.uint8,), "A")
    _check_dtype(B, (torch.uint8,), "B")
    M, K = A.shape[0], 2 * A.shape[1]
    N = B.shape[0]
    if 2 * B.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError("shape mismatch")
    _check_dtype(scale_a, (torch.uint8,), "scale_a")
    _check_dtype(scale_b, (torch.uint8,), "scale_b")
    if scale_a.shape[0] != M or scale_b.shape[0] != N:
        raise ValueError("scale arrays need one row per row of A / stored row of B")
    if scale_a.shape[1] < K // MX_BLOCK or scale_b.shape[1] < K // MX_BLOCK:
        raise ValueError("scale rows need K/32 codes")
    cptr, ldc = None, 0
    if C is not None:
        _check_dtype(C, (torch.float32,), "C")
        if tuple(C.shape) != (M, N):
            raise ValueError("C shape")
        cptr, ldc = _dev_ptr(C, "C"), _ld(C, "C")
    rc = load_library().gemm_mxfp4(
        _dev_ptr(A, "A"), _packed_ld(A, "A"), _dev_ptr(B, "B"), _packed_ld(B, "B"),
        _dev_ptr(scale_a, "scale_a"), _ld(scale_a, "scale_a"), _dev_ptr(scale_b, "scale_b"),
        _ld(scale_b, "scale_b"), cptr, ldc, _dev_ptr(out, "out"), _ld(out, "out"),
        OUT_F32 if out.dtype == torch.float32 else OUT_BF16, M, N, K, _stream(stream))
    _check("gemm_mxfp4", rc)
    return out


def quantize_mxfp4(X, Q, S, stream=None):
    """Q, S = MXFP4 quantisation of X (float32 [rows, cols], cols % 32 == 0): Q
    uint8 [rows, cols/2] packed E2M1, S uint8 [rows, >= cols/32] E8M0 codes."""
    torch = _torch()
    _check_dtype(X, (torch.float32,), "X")
    _check_dtype(Q, (torch.uint8,), "Q")
    _check_dtype(S, (torch.uint8,), "S")
    rows, cols = X.shape
    if tuple(Q.shape) != (rows, cols // 2):
        raise ValueError("Q shape")
    if S.shape[0] != rows or S.shape[1] < cols // MX_BLOCK:
        raise ValueError("S shape")
    rc = load_library().quantize_mxfp4(
        _dev_ptr(X, "X"), rows, cols, _ld(X, "X"), _dev_ptr(Q, "Q"), _packed_ld(Q, "Q"),
        _dev_ptr(S, "S"), _ld(S, "S"), _stream(stream))
    _check("quantize_mxfp4", rc)
    return Q, S


def probe_mfma(kind: int, A, B, C, D, fmt_a: int = E4M3, fmt_b: int = E4M3, stream=None):
    """Run one matrix instruction (see include/dmu_probe.h)."""
    rc = load_library().dmu_probe_mfma(kind, fmt_a, fmt_b, _dev_ptr(A, "A"), _dev_ptr(B, "B"),
                                       _dev_ptr(C, "C"), _dev_ptr(D, "D"), _stream(stream))
    _check("dmu_probe_mfma", rc)
    return D


PROBE_SHAPES = {PROBE_BF16_16X16X32: (16, 16, 32), PROBE_BF16_32X32X16: (32, 32, 16),
                PROBE_FP8_16X16X128: (16, 16, 128), PROBE_FP8_32X32X64: (32, 32, 64)}


def probe_mfma_batch(kind: int, A, B, C, D, fmt_a: int = E4M3, fmt_b: int = E4M3, stream=None):
    """Run count independent matrix instructions of `kind` in one launch (see
    include/dmu_probe.h): A [count][m][k], B [count][n][k], C and D
    [count][m][n] FP32, all contiguous on the GPU."""
    torch = _torch()
    if kind not in PROBE_SHAPES:
        raise ValueError("unknown probe kind %r" % kind)
    m, n, k = PROBE_SHAPES[kind]
    count = A.shape[0] if A.dim() == 3 else -1
    for t, shp, name in ((A, (count, m, k), "A"), (B, (count, n, k), "B"),
                         (C, (count, m, n), "C"), (D, (count, m, n), "D")):
        if tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError("%s must be contiguous with shape %s" % (name, shp))
    esz = 2 if kind in (PROBE_BF16_16X16X32, PROBE_BF16_32X32X16) else 1
    if A.element_size() != esz or B.element_size() != esz:
        raise TypeError("A and B must hold %d-byte elements" % esz)
    _check_dtype(C, (torch.float32,), "C")
    _check_dtype(D, (torch.float32,), "D")
    rc = load_library().dmu_probe_mfma_batch(kind, fmt_a, fmt_b, _dev_ptr(A, "A"),
                                             _dev_ptr(B, "B"), _dev_ptr(C, "C"),
                                             _dev_ptr(D, "D"), count, _stream(stream))
    _check("dmu_probe_mfma_batch", rc)
    return D


def probe_mfma_mx(shape: int, A, B, SA, SB, C, D, fmt_a: int = E4M3, fmt_b: int = E4M3,
                  opsel: int = 0, stream=None):
    """Run one scaled (MX) matrix instruction (see include/dmu_probe.h)."""
    rc = load_library().dmu_probe_mfma_mx(shape, fmt_a, fmt_b, opsel, _dev_ptr(A, "A"),
                                          _dev_ptr(B, "B"), _dev_ptr(SA, "SA"),
                                          _dev_ptr(SB, "SB"), _dev_ptr(C, "C"), _dev_ptr(D, "D"),
                                          _stream(stream))
    _check("dmu_probe_mfma_mx", rc)
    return D


def probe_cvt_fp8(x, q, fmt: int = E4M3, clamp: int = 1, stream=None):
    """Hardware FP32 -> FP8 conversion of x (float32, even length) into q
    (uint8, same length; half the length for fmt E2M1, two codes per byte);
    see include/dmu_probe.h."""
    torch = _torch()
    _check_dtype(x, (torch.float32,), "x")
    _check_dtype(q, (torch.uint8,), "q")
    want = x.numel() // 2 if fmt == E2M1 else x.numel()
    if q.numel() != want or not (x.is_contiguous() and q.is_contiguous()):
        raise ValueError("x and q: contiguous, q of %d bytes" % want)
    rc = load_library().dmu_probe_cvt_fp8(_dev_ptr(x, "x"), x.numel(), fmt, clamp,
                                          _dev_ptr(q, "q"), _stream(stream))
    _check("dmu_probe_cvt_fp8", rc)
    return q


def probe_quantize_tensor_resident(X, Q, scale, fmt: int = E4M3, spin_limit: int = 0,
                                   stream=None):
    """Per-tensor quantize_fp8 of a contiguous X (float32 [rows, cols]) into
    Q (uint8, same shape) and scale (one float32) through the one-pass kernel
    with the given wait bound; see include/dmu_probe.h."""
    torch = _torch()
    _check_dtype(X, (torch.float32,), "X")
    _check_dtype(Q, (torch.uint8,), "Q")
    _check_dtype(scale, (torch.float32,), "scale")
    if X.dim() != 2 or tuple(Q.shape) != tuple(X.shape) or not (X.is_contiguous() and
                                                                Q.is_contiguous()):
        raise ValueError("X and Q: contiguous, same 2-D shape")
    rc = load_library().dmu_probe_quantize_tensor_resident(
        _dev_ptr(X, "X"), X.shape[0], X.shape[1], fmt, _dev_ptr(Q, "Q"),
        _dev_ptr(scale, "scale"), spin_limit, _stream(stream))
    _check("dmu_probe_quantize_tensor_resident", rc)
    return Q, scale


def probe_lds_tr16(src, offsets, out, stream=None):
    """ds_read_b64_tr_b16 probe (include/dmu_probe.h): src 1024 16-bit values
    (GPU), offsets 64 byte offsets (host sequence), out 256 16-bit values (GPU)."""
    torch = _torch()
    _check_dtype(src, (torch.int16, torch.uint16, torch.bfloat16), "src")
    _check_dtype(out, (torch.int16, torch.uint16, torch.bfloat16), "out")
    if src.numel() != 1024 or out.numel() != 256 or not (src.is_contiguous() and
                                                          out.is_contiguous()):
        raise ValueError("src: 1024 and out: 256 contiguous values")
    offs = (ctypes.c_uint32 * 64)(*[int(o) for o in offsets])
    rc = load_library().dmu_probe_lds_tr16(_dev_ptr(src, "src"), ctypes.cast(offs, _P),
                                           _dev_ptr(out, "out"), _stream(stream))
    _check("dmu_probe_lds_tr16", rc)
    return out


LDS_SWIZZLED, LDS_PLAIN, LDS_PADDED = 0, 1, 2  # layouts of dmu_probe_gemm_bf16_layout


def probe_gemm_bf16_layout(layout: int, A, B, out, stream=None):
    """gemm_bf16 (B stored N x K, BF16 out) with LDS layout `layout` (see
    include/dmu_probe.h): A [M][K], B [N][K] BF16, out [M][N] BF16."""
    torch = _torch()
    for t, name in ((A, "A"), (B, "B"), (out, "out")):
        _check_dtype(t, (torch.bfloat16, torch.int16), name)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError("shapes")
    rc = load_library().dmu_probe_gemm_bf16_layout(
        layout, _dev_ptr(A, "A"), _ld(A, "A"), _dev_ptr(B, "B"), _ld(B, "B"), _dev_ptr(out, "out"),
        _ld(out, "out"), M, N, K, _stream(stream))
    _check("dmu_probe_gemm_bf16_layout", rc)
    return out


def probe_lds_load(src, dst, mode: int, oob_from: int = 64, stream=None):
    rc = load_library().dmu_probe_lds_load(_dev_ptr(src, "src"), _dev_ptr(dst, "dst"), mode,
                                           oob_from, _stream(stream))
    _check("dmu_probe_lds_load", rc)
    return dst


def probe_mfma_rate(kind: int, src, iters: int, grid: int, out, stream=None):
    """Sustained MFMA loop on fragments read from `src` (see include/dmu_probe.h).
    `src` needs 8 KiB (BF16 kind) or 16 KiB (FP8 kind); `out` grid*256 floats."""
    torch = _torch()
    need = 8 * 64 * (16 if kind == PROBE_BF16_32X32X16 else 32)
    if src.numel() * src.element_size() < need or not src.is_contiguous():
        raise ValueError("src must be contiguous and hold %d bytes" % need)
    if out.numel() < grid * 256 or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be contiguous float32 with grid*256 elements")
    rc = load_library().dmu_probe_mfma_rate(kind, _dev_ptr(src, "src"), iters, grid,
                                            _dev_ptr(out, "out"), _stream(stream))
    _check("dmu_probe_mfma_rate", rc)
    return out
