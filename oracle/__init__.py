"""CPU oracle for the dense matrix-unit GEMM path -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it and
has no fallback to it.  It shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain C, FP64, exact decoding); this
module loads it with ctypes and marshals numpy arrays.  What each function
computes, and the page passages it follows, is documented in ``oracle.c``.
The two error metrics below are the definitions used on the page "Tensor
Cores: Matrix Instructions, Swizzling and FP8, Measured", Step 2 (relative
error = RMS of the error over RMS of the value) and Step 5 ("total" versus
"from the sums" errors against an FP64 product).

Every function here is pinned by ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_TOL_SRC = os.path.join(_HERE, "tolerance.c")  # tolerance helper, not a definition
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

E4M3 = 0
E5M2 = 1
E2M1 = 4  # FP4 element format of MXFP4; codes packed two per byte in MX arrays
B_ROW_MAJOR = 0
B_COL_MAJOR = 1
SCALE_TENSOR = 0
SCALE_BLOCK = 1
FMAX = {E4M3: 448.0, E5M2: 57344.0}


def build(force: bool = False) -> str:
    """Compile oracle.c and tolerance.c into liboracle.so with gcc (no
    fast-math, no FMA contraction) and return its path."""
    if force or not os.path.exists(_LIB_PATH) or any(
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(src) for src in (_SRC, _TOL_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = [
            "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-std=c11", "-shared", "-fPIC", _SRC, _TOL_SRC, "-o", tmp, "-lm",
        ]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = i32
        L.orc_decode_bf16_array.argtypes = [p, i64, p]
        L.orc_decode_fp8_array.argtypes = [p, i64, i32, p]
        L.orc_encode_bf16_array.argtypes = [p, i64, p]
        L.orc_encode_fp8_array.argtypes = [p, i64, i32, p]
        L.orc_quantize_fp8.argtypes = [p, i64, i64, i64, i32, i64, i64, p, i64, p]
        L.orc_quantize_fp8.restype = i32
        L.orc_gemm_bf16.argtypes = [p, i64, p, i64, i32, p, i64, i64, i64, i64, p, i64, p, p]
        L.orc_gemm_bf16.restype = i32
        L.orc_gemm_fp8.argtypes = [p, i64, i32, p, i64, i32, p, p, i32, p, i64, i64, i64,
                                   i64, p, i64, p, p]
        L.orc_gemm_fp8.restype = i32
        L.orc_gemm_grouped_bf16.argtypes = [p, i64, p, i64, i64, p, i64, i64, i64, p, i64, p,
                                            p]
        L.orc_gemm_grouped_bf16.restype = i32
        L.orc_epilogue.argtypes = [p, i64, i64, ctypes.c_double, p, i32, p]
        L.orc_attention_bf16.argtypes = [p, p, p, i64, i64, i64, i64, ctypes.c_double, i32, p,
                                         p, p]
        L.orc_epilogue.restype = i32
        L.orc_encode_fp4_array.argtypes = [p, i64, p]
        L.orc_decode_fp4_array.argtypes = [p, i64, p]
        L.orc_decode_e8m0.argtypes = [ctypes.c_uint8]
        L.orc_decode_e8m0.restype = ctypes.c_double
        L.orc_quantize_mx.argtypes = [p, i64, i64, i64, i32, p, i64, p, i64]
        L.orc_quantize_mx.restype = i32
        L.orc_gemm_mx.argtypes = [p, i64, i32, p, i64, i32, p, i64, p, i64, p, i64, i64, i64, i64,
                                  p, i64, p, p]
        L.orc_gemm_mx.restype = i32
        L.orc_fp8_group_loss.argtypes = [p, i64, i32, p, i64, i32, i64, i64, i64, p, i64, p,
                                         i64, i64, i64, p, i64, p]
        L.orc_fp8_group_loss.restype = i32
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().orc_num_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data


def decode_bf16(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    lib().orc_decode_bf16_array(_ptr(h), h.size, _ptr(out))
    return out


def decode_fp8(v, fmt: int) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.uint8)
    out = np.empty(v.shape, dtype=np.float64)
    lib().orc_decode_fp8_array(_ptr(v), v.size, fmt, _ptr(out))
    return out


def encode_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_encode_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def encode_fp8(x, fmt: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_encode_fp8_array(_ptr(x), x.size, fmt, _ptr(out))
    return out


def decode_fp4(v) -> np.ndarray:
    """E2M1 codes (one per array element, low 4 bits) -> exact values."""
    v = np.ascontiguousarray(v, dtype=np.uint8)
    out = np.empty(v.shape, dtype=np.float64)
    lib().orc_decode_fp4_array(_ptr(v), v.size, _ptr(out))
    return out


def encode_fp4(x) -> np.ndarray:
    """FP32 -> E2M1 codes, one per array element (not packed)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_encode_fp4_array(_ptr(x), x.size, _ptr(out))
    return out


def pack_fp4(codes) -> np.ndarray:
    """[rows][cols] E2M1 codes -> [rows][cols/2] bytes, element 2i in the low
    nibble of byte i and element 2i+1 in the high nibble."""
    c = np.ascontiguousarray(codes, dtype=np.uint8) & 15
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed) -> np.ndarray:
    """Inverse of pack_fp4."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def decode_elems(A, fmt: int) -> np.ndarray:
    """Exact values of an MX element array: FP8 codes, or packed E2M1."""
    if fmt == E2M1:
        return decode_fp4(unpack_fp4(A))
    return decode_fp8(A, fmt)


def quantize_fp8(X, fmt: int, block_rows: int | None = None, block_cols: int | None = None):
    """Return (Q uint8 like X, scales float32 [rows/br][cols/bc]).  Block
    (None, None) means one block for the whole tensor."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    rows, cols = X.shape
    br = rows if block_rows is None else block_rows
    bc = cols if block_cols is None else block_cols
    Q = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty((rows // br, cols // bc), dtype=np.float32)
    rc = lib().orc_quantize_fp8(_ptr(X), rows, cols, cols, fmt, br, bc, _ptr(Q), cols,
                                _ptr(scales))
    if rc != 0:
        raise ValueError("orc_quantize_fp8: bad arguments")
    return Q, scales


def _rows_arg(rows, M):
    if rows is None:
        return None, M
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, r.size


def gemm_bf16(A, B, b_layout: int, C=None, rows=None):
    """FP64 D = A*B + C (selected rows) and S = sum_k |a*b|.  A: [M][K] uint16
    BF16 codes.  B: [K][N] (row-major) or [N][K] (column-major) uint16."""
    A = np.ascontiguousarray(A, dtype=np.uint16)
    B = np.ascontiguousarray(B, dtype=np.uint16)
    M, K = A.shape
    N = B.shape[1] if b_layout == B_ROW_MAJOR else B.shape[0]
    assert (B.shape[0] if b_layout == B_ROW_MAJOR else B.shape[1]) == K
    if C is not None:
        C = np.ascontiguousarray(C, dtype=np.float32)
        assert C.shape == (M, N)
    r, nr = _rows_arg(rows, M)
    D = np.empty((nr, N), dtype=np.float64)
    S = np.empty((nr, N), dtype=np.float64)
    rc = lib().orc_gemm_bf16(_ptr(A), K, _ptr(B), B.shape[1], b_layout, _ptr(C), N, M, N, K,
                             _ptr(r), nr, _ptr(D), _ptr(S))
    if rc != 0:
        raise ValueError("orc_gemm_bf16: bad arguments")
    return D, S


def gemm_fp8(A, B, fmt_a: int, fmt_b: int, sa, sb, scale_mode: int, C=None, rows=None):
    """FP64 scaled FP8 product (selected rows) and S = sum |a sa| |b sb|.
    A: [M][K] uint8, B: [N][K] uint8 (column-major B)."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    if C is not None:
        C = np.ascontiguousarray(C, dtype=np.float32)
        assert C.shape == (M, N)
    r, nr = _rows_arg(rows, M)
    D = np.empty((nr, N), dtype=np.float64)
    S = np.empty((nr, N), dtype=np.float64)
    rc = lib().orc_gemm_fp8(_ptr(A), K, fmt_a, _ptr(B), K, fmt_b, _ptr(sa), _ptr(sb),
                            scale_mode, _ptr(C), N, M, N, K, _ptr(r), nr, _ptr(D), _ptr(S))
    if rc != 0:
        raise ValueError("orc_gemm_fp8: bad arguments")
    return D, S


def fp8_group_loss(A, B, fmt_a: int, fmt_b: int, sa=None, sb=None, k_per_scale=None,
                   b_rows_per_scale: int = 1, rows=None) -> np.ndarray:
    """Tolerance term for FP8 products formed by gfx950's matrix unit (see
    tolerance.c; not a definition): per output element, the sum over k of
    |a_ik b_jk| mod 2^(E_g - 13), E_g the largest exponent-field sum of k's
    aligned group of 8, times |sa(i, k) sb(j, k)|.  A: [M][K] and B: [N][K]
    FP8 codes.  Scales (optional): sa [M][K / k_per_scale] and sb
    [ceil(N / b_rows_per_scale)][K / k_per_scale], or one value each (per
    tensor)."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    ld_sa = ld_sb = 0
    if sa is not None:
        sa = np.ascontiguousarray(sa, dtype=np.float64)
        sb = np.ascontiguousarray(sb, dtype=np.float64)
        if sa.size == 1 and sb.size == 1:  # per tensor: one scale block spans everything
            sa, sb = sa.reshape(1), sb.reshape(1)
            k_per_scale, b_rows_per_scale = K, N
        else:
            assert k_per_scale and K % k_per_scale == 0
            sa = sa.reshape(M, -1)
            sb = sb.reshape(-1, sa.shape[1])
            ld_sa, ld_sb = sa.shape[1], sb.shape[1]
    kps = k_per_scale or K
    r, nr = _rows_arg(rows, M)
    L = np.empty((nr, N), dtype=np.float64)
    rc = lib().orc_fp8_group_loss(_ptr(A), K, fmt_a, _ptr(B), K, fmt_b, M, N, K,
                                  _ptr(sa), ld_sa, _ptr(sb), ld_sb, b_rows_per_scale, kps,
                                  _ptr(r), nr, _ptr(L))
    if rc != 0:
        raise ValueError("orc_fp8_group_loss: bad arguments")
    return L


MX_BLOCK = 32


def decode_e8m0(codes) -> np.ndarray:
    """E8M0 scale codes -> 2^(code-127) (code 255: NaN)."""
    c = np.asarray(codes, dtype=np.uint8)
    return np.vectorize(lambda v: lib().orc_decode_e8m0(int(v)), otypes=[np.float64])(c)


def quantize_mx(X, fmt: int):
    """MX quantisation with 1 x 32 blocks along each row: returns (Q, S uint8
    E8M0 codes [rows][cols/32]).  Q is uint8 like X for FP8, or [rows][cols/2]
    packed E2M1 for fmt E2M1."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    rows, cols = X.shape
    qc = cols // 2 if fmt == E2M1 else cols
    Q = np.empty((rows, qc), dtype=np.uint8)
    S = np.empty((rows, cols // MX_BLOCK), dtype=np.uint8)
    rc = lib().orc_quantize_mx(_ptr(X), rows, cols, cols, fmt, _ptr(Q), qc, _ptr(S),
                               cols // MX_BLOCK)
    if rc != 0:
        raise ValueError("orc_quantize_mx: bad arguments")
    return Q, S


def gemm_mx(A, B, fmt_a: int, fmt_b: int, SA, SB, C=None, rows=None):
    """FP64 MX product (selected rows) and S = sum of |scaled a * scaled b|.
    A: [M][K] and B: [N][K] uint8 FP8 codes, or [M][K/2] / [N][K/2] packed
    E2M1 for that operand's format; SA: [M][K/32], SB: [N][K/32] uint8."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    M = A.shape[0]
    K = A.shape[1] * (2 if fmt_a == E2M1 else 1)
    N = B.shape[0]
    assert B.shape[1] * (2 if fmt_b == E2M1 else 1) == K and K % MX_BLOCK == 0
    SA = np.ascontiguousarray(SA, dtype=np.uint8)
    SB = np.ascontiguousarray(SB, dtype=np.uint8)
    assert SA.shape == (M, K // MX_BLOCK) and SB.shape == (N, K // MX_BLOCK)
    if C is not None:
        C = np.ascontiguousarray(C, dtype=np.float32)
        assert C.shape == (M, N)
    r, nr = _rows_arg(rows, M)
    D = np.empty((nr, N), dtype=np.float64)
    S = np.empty((nr, N), dtype=np.float64)
    rc = lib().orc_gemm_mx(_ptr(A), A.shape[1], fmt_a, _ptr(B), B.shape[1], fmt_b, _ptr(SA),
                           K // MX_BLOCK,
                           _ptr(SB), K // MX_BLOCK, _ptr(C), N, M, N, K, _ptr(r), nr, _ptr(D),
                           _ptr(S))
    if rc != 0:
        raise ValueError("orc_gemm_mx: bad arguments")
    return D, S


def gemm_grouped_bf16(A, B, offsets, rows=None):
    """FP64 grouped product (mixture of experts): rows offsets[g] ..
    offsets[g+1]-1 of A ([M][K] BF16 codes) use expert g's weight B[g]
    ([G][N][K] BF16 codes, stored N x K).  Returns (D, S) for the selected rows
    (default: rows offsets[0] .. offsets[G]-1), one row of D per row."""
    A = np.ascontiguousarray(A, dtype=np.uint16)
    B = np.ascontiguousarray(B, dtype=np.uint16)
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    G, N, K = B.shape
    assert off.shape == (G + 1,) and A.shape[1] == K and off[-1] <= A.shape[0]
    if rows is None:
        r, nr = None, int(off[-1] - off[0])
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        nr = r.size
    D = np.empty((nr, N), dtype=np.float64)
    S = np.empty((nr, N), dtype=np.float64)
    if nr == 0:
        return D, S
    rc = lib().orc_gemm_grouped_bf16(_ptr(A), K, _ptr(B), K, N * K, _ptr(off), G, N, K, _ptr(r),
                                     nr, _ptr(D), _ptr(S))
    if rc != 0:
        raise ValueError("orc_gemm_grouped_bf16: bad arguments")
    return D, S


ACT_NONE, ACT_RELU, ACT_GELU, ACT_SILU = 0, 1, 2, 3


def epilogue(D, alpha: float = 1.0, bias=None, act: int = ACT_NONE) -> np.ndarray:
    """Y = act(alpha * D + bias) in FP64 for FP64 products D [rows][N]; bias
    float32 [N] or None."""
    D = np.ascontiguousarray(D, dtype=np.float64)
    rows, N = D.shape
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (N,)
    Y = np.empty_like(D)
    rc = lib().orc_epilogue(_ptr(D), rows, N, float(alpha), _ptr(bias), act, _ptr(Y))
    if rc != 0:
        raise ValueError("orc_epilogue: bad arguments")
    return Y


# ------------------------------------------------------------------ attention chain

def attention_bf16(Q, K, V, scale: float, causal: bool = False):
    """Softmax attention per head in FP64 (orc_attention_bf16): Q [BH, Sq, d],
    K and V [BH, Sk, d] BF16 bit patterns (uint16; 2-D arrays are one head).
    Returns (O [BH, Sq, d], lse [BH, Sq], Aabs [BH, Sq, d]) in the input's
    rank, Aabs = sum_j w_j |v_j| / l, the scale of the rounding error of O."""
    two = np.ndim(Q) == 2
    Q, K, V = (np.ascontiguousarray(np.asarray(x, dtype=np.uint16)) for x in (Q, K, V))
    if two:
        Q, K, V = Q[None], K[None], V[None]
    BH, Sq, d = Q.shape
    Sk = K.shape[1]
    assert K.shape == (BH, Sk, d) and V.shape == (BH, Sk, d)
    O = np.empty((BH, Sq, d))
    lse = np.empty((BH, Sq))
    A = np.empty((BH, Sq, d))
    rc = lib().orc_attention_bf16(_ptr(Q), _ptr(K), _ptr(V), BH, Sq, Sk, d, float(scale),
                                  int(bool(causal)), _ptr(O), _ptr(lse), _ptr(A))
    if rc != 0:
        raise ValueError("orc_attention_bf16: bad arguments")
    return (O[0], lse[0], A[0]) if two else (O, lse, A)


# ------------------------------------------------------------------ metrics

def rel_rms(D, D_ref) -> float:
    """Relative RMS error: sqrt(sum (D - D_ref)^2) / sqrt(sum D_ref^2)."""
    D = np.asarray(D, dtype=np.float64)
    D_ref = np.asarray(D_ref, dtype=np.float64)
    return float(np.sqrt(np.sum((D - D_ref) ** 2)) / np.sqrt(np.sum(D_ref ** 2)))


def bound_ratio(D, D_ref, S) -> float:
    """max |D - D_ref| / S elementwise (S = sum_k |a_ik b_kj|); the FP32-output
    acceptance bound is bound_ratio <= 1e-5."""
    D = np.asarray(D, dtype=np.float64)
    err = np.abs(D - D_ref)
    S = np.asarray(S, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(S > 0, err / np.where(S > 0, S, 1.0), np.where(err > 0, np.inf, 0.0))
    return float(np.max(r)) if r.size else 0.0


def within_bound(D, D_ref, S, bf16_out: bool, rel: float = 1e-5) -> np.ndarray:
    """Per-element acceptance: |D - D_ref| <= rel*S (FP32 out), plus
    2^-8*|D_ref| for BF16 output."""
    D = np.asarray(D, dtype=np.float64)
    tol = rel * np.asarray(S, dtype=np.float64)
    if bf16_out:
        tol = tol + 2.0 ** -8 * np.abs(D_ref)
    return np.abs(D - D_ref) <= tol
