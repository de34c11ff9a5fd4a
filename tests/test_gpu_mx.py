"""Parity of the microscaling (MX) path -- quantize_mxfp8 and gemm_mxfp8 (HIP)
-- against the oracle's quantize_mx / gemm_mx: one E8M0 scale per row and 32
values of K, the block-scaled product of "How Blackwell's Tensor Memory
Actually Works", section "Quantization became an allocation problem".

The quantizer has one correct result and is compared bit for bit.  The GEMM
is exact where every product feeding an output carries the same power of two
(integer-valued data); otherwise it meets the FP8 bound of
test_gpu_gemm_fp8.py: 1e-5 * sum|ab| (+ 2^-8 |D| for BF16 output) plus 2^-12
x the sum over the 64-wide K runs of one scaled MFMA of the largest scaled
|a*b| in the run (the instruction's inner sum keeps ~14 bits below its
largest term, pinned by test_gpu_probe.py)."""
import numpy as np
import pytest
import torch

import oracle
import dense_matrix_unit_amd as dmu
from dense_matrix_unit_amd import workloads as wl
from gpu_helpers import empty_padded, out_to_f64, padded, round_out, within_fp8_bound

pytestmark = pytest.mark.gpu
FMT_PAIRS = [(0, 0), (0, 1), (1, 0), (1, 1)]


def gpu_quantize(X, fmt):
    rows, cols = X.shape
    Xd = padded(X, 8)
    Q = empty_padded(rows, cols, torch.uint8, 16)
    S = empty_padded(rows, cols // 32, torch.uint8, 16)
    Q.fill_(0xAA)
    S.fill_(0xAA)
    dmu.quantize_mxfp8(Xd, Q, S, fmt)
    torch.cuda.synchronize()
    return Q.cpu().numpy(), S.cpu().numpy()


def special_blocks(X):
    X = X.copy()
    r = X.shape[0]
    X[0, :32] = 0.0                                   # all-zero block
    X[min(1, r - 1), :32] *= np.float32(1e-39)        # FP32 subnormals: code 0
    if X.shape[1] >= 64:
        X[0, 32:64] *= np.float32(1e30)               # huge block
        X[min(2, r - 1), 32:64] = -0.0                # negative zeros
    if r > 3:
        X[3, 5] = np.nan                              # NaN block
        X[3, -1] = -np.inf                            # Inf block
        X[2, :32] = np.float32(448.0)                 # E4M3 max exactly
        X[2, 7] = np.float32(-449.0)                  # just above: scale step
    return X


@pytest.mark.parametrize("fmt", [dmu.E4M3, dmu.E5M2])
@pytest.mark.parametrize("shape", [(64, 512), (37, 96), (1, 32), (300, 4128)])
def test_quantize_mx_bit_exact(fmt, shape):
    X, _ = wl.normal_with_outlier_rows(shape, 7, frac=0.05)
    X = special_blocks(X)
    Q, S = gpu_quantize(X, fmt)
    Qr, Sr = oracle.quantize_mx(X, fmt)
    assert np.array_equal(S, Sr)
    assert np.array_equal(Q, Qr)


@pytest.mark.parametrize("fmt", [dmu.E4M3, dmu.E5M2])
def test_quantize_mx_4096_bit_exact(fmt):
    X, _ = wl.normal_with_outlier_rows((4096, 4096), wl.SEED_A)
    Q, S = gpu_quantize(X, fmt)
    Qr, Sr = oracle.quantize_mx(X, fmt)
    assert np.array_equal(S, Sr)
    assert np.array_equal(Q, Qr)


def run_mx(A, B, fa, fb, SA, SB, out_dtype, C=None):
    M, N = A.shape[0], B.shape[0]
    out = empty_padded(M, N, out_dtype)
    dmu.gemm_mxfp8(padded(A, 16), padded(B, 16), padded(SA, 16), padded(SB, 16), out, fa, fb,
                   C=None if C is None else padded(C, 4))
    torch.cuda.synchronize()
    return out_to_f64(out)


def mx_loss(A, B, fa, fb, SA, SB, rows=None):
    """What the scaled FP8 instruction discards per output element: the exact
    per-product cut of oracle.fp8_group_loss (groups of 8 K positions, grid
    2^(E - 13); pinned in test_gpu_probe.py), times each product's two E8M0
    scales.  E2M1 x E2M1 products lose nothing: they are multiples of 2^-2
    below 2^6, so every one lies on its group's grid."""
    if fa == oracle.E2M1 and fb == oracle.E2M1:
        M = A.shape[0] if rows is None else len(rows)
        return np.zeros((M, B.shape[0]))
    return oracle.fp8_group_loss(A, B, fa, fb, oracle.decode_e8m0(SA), oracle.decode_e8m0(SB),
                                 k_per_scale=32, b_rows_per_scale=1, rows=rows)


def check(A, B, fa, fb, SA, SB, out_dtype, C=None, rows=None, what=""):
    D = run_mx(A, B, fa, fb, SA, SB, out_dtype, C)
    Dref, S = oracle.gemm_mx(A, B, fa, fb, SA, SB, C=C, rows=rows)
    if rows is not None:
        D = D[rows]
    if C is not None:
        S = S + np.abs(C if rows is None else C[rows])
    sel = np.arange(A.shape[0]) if rows is None else np.asarray(rows)
    ok, tol = within_fp8_bound(D, Dref, S, out_dtype == torch.bfloat16,
                               lambda r: mx_loss(A, B, fa, fb, SA, SB, sel[r]))
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError("%s: %d of %d outside the bound; first %s: got %r ref %r tol %r"
                             % (what, (~ok).sum(), ok.size, i, D[i], Dref[i], tol[i]))
    return D, Dref


def cancelling_codes(M, N, nkb, seed):
    """SA[i][g] = a_i + u_g, SB[j][g] = b_j - u_g: all products feeding D[i][j]
    carry 2^(a_i + b_j - 254), so integer data stays exact, while a scale taken
    from the wrong row, column or K run changes the result."""
    rng = np.random.default_rng(seed)
    u = rng.integers(-4, 5, size=nkb)
    a = rng.integers(122, 131, size=M)
    b = rng.integers(122, 131, size=N)
    return ((a[:, None] + u[None, :]).astype(np.uint8), (b[:, None] - u[None, :]).astype(np.uint8))


@pytest.mark.parametrize("fa,fb", FMT_PAIRS)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gemm_mx_integer_exact(fa, fb, out_dtype):
    M, N, K = 272, 288, 384
    A = oracle.encode_fp8(wl.small_ints((M, K), 1), fa)
    B = oracle.encode_fp8(wl.small_ints((N, K), 2), fb)
    SA, SB = cancelling_codes(M, N, K // 32, 3)
    C = wl.small_ints((M, N), 4, -1000, 1000)
    D = run_mx(A, B, fa, fb, SA, SB, out_dtype, C)
    Dref, _ = oracle.gemm_mx(A, B, fa, fb, SA, SB, C=C)
    assert np.array_equal(D, round_out(Dref, out_dtype == torch.bfloat16))


@pytest.mark.parametrize("fa,fb", FMT_PAIRS)
@pytest.mark.parametrize("shape", [(320, 264, 512), (1, 16, 128), (513, 600, 1152)])
def test_gemm_mx_random_codes(fa, fb, shape):
    M, N, K = shape
    rng = np.random.default_rng(11)
    A = oracle.encode_fp8(wl.normal((M, K), 1), fa)
    B = oracle.encode_fp8(wl.normal((N, K), 2), fb)
    SA = rng.integers(116, 139, size=(M, K // 32)).astype(np.uint8)
    SB = rng.integers(116, 139, size=(N, K // 32)).astype(np.uint8)
    C = wl.normal((M, N), 3) if M == 320 else None
    out = torch.float32 if M == 320 else torch.bfloat16
    check(A, B, fa, fb, SA, SB, out, C=C, what=str(shape))


@pytest.mark.parametrize("fmt", [dmu.E4M3, dmu.E5M2])
def test_gemm_mx_gpu_quantized_pipeline(fmt):
    # GPU quantizer feeding the GPU GEMM: its output is the oracle's (bit for
    # bit), so the oracle's product of the oracle's quantization is the target
    M, N, K = 384, 320, 640
    Xa, _ = wl.normal_with_outlier_rows((M, K), 5, frac=0.03)
    Xb = wl.normal((N, K), 6)
    Qa, Sa = gpu_quantize(Xa, fmt)
    Qb, Sb = gpu_quantize(Xb, fmt)
    Qa_r, Sa_r = oracle.quantize_mx(Xa, fmt)
    Qb_r, Sb_r = oracle.quantize_mx(Xb, fmt)
    assert np.array_equal(Qa, Qa_r) and np.array_equal(Sa, Sa_r)
    assert np.array_equal(Qb, Qb_r) and np.array_equal(Sb, Sb_r)
    D, Dref = check(Qa_r, Qb_r, fmt, fmt, Sa_r, Sb_r, torch.float32, what="pipeline")
    total = Xa.astype(np.float64) @ Xb.astype(np.float64).T
    print("MX fmt %d: rel-RMS from the sums %.3e, total %.3e"
          % (fmt, oracle.rel_rms(D, Dref), oracle.rel_rms(D, total)))


def test_gemm_mx_extreme_codes_cancel():
    # 2^-127 x 2^127 per product: exact if the unit combines the exponents
    # before scaling.  Where both codes are 0 the products are 2^-254 x small
    # integers and D is zero; where both are 254 every 64-wide run overflows
    # FP32 on its own, so runs of opposite sign may meet as Inf - Inf = NaN
    # while the FP64 sum rounds to +-Inf: there D is only required to be
    # non-finite.
    M, N, K = 64, 96, 256
    A = oracle.encode_fp8(wl.small_ints((M, K), 21), 0)
    B = oracle.encode_fp8(wl.small_ints((N, K), 22), 0)
    SA = np.where(np.arange(M)[:, None] % 2 == 0, 0, 254) * np.ones((1, K // 32))
    SB = np.where(np.arange(N)[:, None] % 2 == 0, 254, 0) * np.ones((1, K // 32))
    SA, SB = SA.astype(np.uint8), SB.astype(np.uint8)
    D = run_mx(A, B, 0, 0, SA, SB, torch.float32)
    Dref, _ = oracle.gemm_mx(A, B, 0, 0, SA, SB)
    ri, cj = np.arange(M)[:, None] % 2, np.arange(N)[None, :] % 2
    same = ri == cj
    assert np.array_equal(D[same], Dref[same])
    tiny = (ri == 0) & (cj == 1)
    assert np.all(D[tiny] == 0.0)
    huge = (ri == 1) & (cj == 0) & (Dref != 0)
    assert not np.isfinite(D[huge]).any()


def test_gemm_mx_nan_scale():
    M, N, K = 300, 260, 256
    A = oracle.encode_fp8(wl.small_ints((M, K), 31), 0)
    B = oracle.encode_fp8(wl.small_ints((N, K), 32), 1)
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 126, np.uint8)
    SA[290, 5] = 255   # row 290 of D is NaN
    SB[7, 0] = 255     # column 7 of D is NaN
    D = run_mx(A, B, 0, 1, SA, SB, torch.float32)
    Dref, _ = oracle.gemm_mx(A, B, 0, 1, SA, SB)
    assert np.array_equal(np.isnan(D), np.isnan(Dref))
    assert np.isnan(D[290]).all() and np.isnan(D[:, 7]).all()
    ok = ~np.isnan(Dref)
    assert np.array_equal(D[ok], Dref[ok])


@pytest.mark.parametrize("fmt", [dmu.E4M3, dmu.E5M2])
def test_gemm_mx_4096(fmt):
    # the MX workload in full (4096^3, BF16 out), the bench's launch
    A, SA = oracle.quantize_mx(wl.normal((4096, 4096), wl.SEED_A), fmt)
    B, SB = oracle.quantize_mx(wl.normal((4096, 4096), wl.SEED_B), fmt)
    check(A, B, fmt, fmt, SA, SB, torch.bfloat16, what="4096^3 MX fmt %d" % fmt)


def run_mx_strided(A, B, fa, fb, SA, SB, ld_extra, offset):
    """gemm_mxfp8 with scale rows of K/32 + ld_extra bytes, the arrays starting
    `offset` bytes into their allocation (BF16 out)."""
    M, N = A.shape[0], B.shape[0]
    nkb = SA.shape[1]

    def place(S):
        ld = nkb + ld_extra
        buf = torch.zeros(S.shape[0] * ld + offset, dtype=torch.uint8, device="cuda")
        v = buf[offset:].view(S.shape[0], ld)[:, :nkb]
        v.copy_(torch.from_numpy(np.ascontiguousarray(S)))
        return v
    out = empty_padded(M, N, torch.bfloat16)
    dmu.gemm_mxfp8(padded(A, 16), padded(B, 16), place(SA), place(SB), out, fa, fb)
    torch.cuda.synchronize()
    return out_to_f64(out)


@pytest.mark.parametrize("K", [512, 1536, 2560])
@pytest.mark.parametrize("ld_extra,offset", [(0, 0), (4, 0), (16, 4)])
def test_gemm_mx_scale_fetch_paths(K, ld_extra, offset):
    # K % 512 == 0 with 16-byte scale rows fetches scale codes 4 slices at a
    # time (1, 3, 5 groups: both ring buffers, odd and even group counts);
    # a 4-byte row stride or start falls back to one slice at a time
    M, N = 384, 272
    rng = np.random.default_rng(K + ld_extra)
    A = oracle.encode_fp8(wl.normal((M, K), 1), 0)
    B = oracle.encode_fp8(wl.normal((N, K), 2), 1)
    SA = rng.integers(116, 139, size=(M, K // 32)).astype(np.uint8)
    SB = rng.integers(116, 139, size=(N, K // 32)).astype(np.uint8)
    D = run_mx_strided(A, B, 0, 1, SA, SB, ld_extra, offset)
    Dref, S = oracle.gemm_mx(A, B, 0, 1, SA, SB)
    tol = 1e-5 * S + mx_loss(A, B, 0, 1, SA, SB) + 2.0 ** -8 * np.abs(Dref)
    bad = ~(np.abs(D - Dref) <= tol)
    assert not bad.any(), "%d outside the bound, first at %s" % (bad.sum(), np.argwhere(bad)[0])


# ---------------------------------------------------------------- MXFP4 (E2M1)

def gpu_quantize4(X):
    rows, cols = X.shape
    Q = empty_padded(rows, cols // 2, torch.uint8, 16)
    S = empty_padded(rows, cols // 32, torch.uint8, 16)
    Q.fill_(0xAA)
    S.fill_(0xAA)
    dmu.quantize_mxfp4(padded(X, 8), Q, S)
    torch.cuda.synchronize()
    return Q.cpu().numpy(), S.cpu().numpy()


@pytest.mark.parametrize("shape", [(64, 512), (37, 96), (1, 32), (300, 4128)])
def test_quantize_mxfp4_bit_exact(shape):
    X, _ = wl.normal_with_outlier_rows(shape, 9, frac=0.05)
    X = special_blocks(X)
    if X.shape[1] >= 64 and X.shape[0] > 4:
        X[4, 32:64] = np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5] * 4)  # E2M1 ties
    Q, S = gpu_quantize4(X)
    Qr, Sr = oracle.quantize_mx(X, oracle.E2M1)
    assert np.array_equal(S, Sr)
    assert np.array_equal(Q, Qr)


def test_quantize_mxfp4_4096_bit_exact():
    X, _ = wl.normal_with_outlier_rows((4096, 4096), wl.SEED_A)
    Q, S = gpu_quantize4(X)
    Qr, Sr = oracle.quantize_mx(X, oracle.E2M1)
    assert np.array_equal(S, Sr)
    assert np.array_equal(Q, Qr)


def run_mx4(A, B, SA, SB, out_dtype, C=None):
    M, N = A.shape[0], B.shape[0]
    out = empty_padded(M, N, out_dtype)
    dmu.gemm_mxfp4(padded(A, 16), padded(B, 16), padded(SA, 16), padded(SB, 16), out,
                   C=None if C is None else padded(C, 4))
    torch.cuda.synchronize()
    return out_to_f64(out)


def fp4(X):
    return oracle.pack_fp4(oracle.encode_fp4(X))


def check4(A, B, SA, SB, out_dtype, C=None, rows=None, what=""):
    D = run_mx4(A, B, SA, SB, out_dtype, C)
    Dref, S = oracle.gemm_mx(A, B, 4, 4, SA, SB, C=C, rows=rows)
    if rows is not None:
        D = D[rows]
    if C is not None:
        S = S + np.abs(C if rows is None else C[rows])
    sel = np.arange(A.shape[0]) if rows is None else np.asarray(rows)
    ok, tol = within_fp8_bound(D, Dref, S, out_dtype == torch.bfloat16,
                               lambda r: mx_loss(A, B, 4, 4, SA, SB, sel[r]))
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError("%s: %d of %d outside the bound; first %s: got %r ref %r tol %r"
                             % (what, (~ok).sum(), ok.size, i, D[i], Dref[i], tol[i]))
    return D, Dref


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gemm_mxfp4_integer_exact(out_dtype):
    M, N, K = 272, 288, 1024
    A = fp4(wl.small_ints((M, K), 1) * 0.5)
    B = fp4(wl.small_ints((N, K), 2) * 0.5)
    SA, SB = cancelling_codes(M, N, K // 32, 5)
    C = wl.small_ints((M, N), 4, -1000, 1000)
    D = run_mx4(A, B, SA, SB, out_dtype, C)
    Dref, _ = oracle.gemm_mx(A, B, 4, 4, SA, SB, C=C)
    assert np.array_equal(D, round_out(Dref, out_dtype == torch.bfloat16))


@pytest.mark.parametrize("shape", [(320, 264, 512), (1, 16, 512), (513, 600, 1536), (256, 256, 2560)])
def test_gemm_mxfp4_random_codes(shape):
    M, N, K = shape
    rng = np.random.default_rng(13)
    A = fp4(wl.normal((M, K), 1) * 3)
    B = fp4(wl.normal((N, K), 2) * 3)
    SA = rng.integers(116, 139, size=(M, K // 32)).astype(np.uint8)
    SB = rng.integers(116, 139, size=(N, K // 32)).astype(np.uint8)
    C = wl.normal((M, N), 3) if M == 320 else None
    out = torch.float32 if M == 320 else torch.bfloat16
    check4(A, B, SA, SB, out, C=C, what=str(shape))


def test_gemm_mxfp4_gpu_quantized_pipeline():
    M, N, K = 384, 320, 1024
    Xa, _ = wl.normal_with_outlier_rows((M, K), 5, frac=0.03)
    Xb = wl.normal((N, K), 6)
    Qa, Sa = gpu_quantize4(Xa)
    Qb, Sb = gpu_quantize4(Xb)
    Qa_r, Sa_r = oracle.quantize_mx(Xa, oracle.E2M1)
    Qb_r, Sb_r = oracle.quantize_mx(Xb, oracle.E2M1)
    assert np.array_equal(Qa, Qa_r) and np.array_equal(Sa, Sa_r)
    assert np.array_equal(Qb, Qb_r) and np.array_equal(Sb, Sb_r)
    D, Dref = check4(Qa_r, Qb_r, Sa_r, Sb_r, torch.float32, what="fp4 pipeline")
    total = Xa.astype(np.float64) @ Xb.astype(np.float64).T
    print("MXFP4: rel-RMS from the sums %.3e, total %.3e"
          % (oracle.rel_rms(D, Dref), oracle.rel_rms(D, total)))


def test_gemm_mxfp4_nan_scale():
    M, N, K = 300, 260, 512
    A = fp4(wl.small_ints((M, K), 31) * 0.5)
    B = fp4(wl.small_ints((N, K), 32) * 0.5)
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 126, np.uint8)
    SA[17, 9] = 255
    SB[259, 3] = 255
    D = run_mx4(A, B, SA, SB, torch.float32)
    Dref, _ = oracle.gemm_mx(A, B, 4, 4, SA, SB)
    assert np.array_equal(np.isnan(D), np.isnan(Dref))
    assert np.isnan(D[17]).all() and np.isnan(D[:, 259]).all()
    ok = ~np.isnan(Dref)
    assert np.array_equal(D[ok], Dref[ok])


def test_gemm_mxfp4_4096():
    A, SA = oracle.quantize_mx(wl.normal((4096, 4096), wl.SEED_A), oracle.E2M1)
    B, SB = oracle.quantize_mx(wl.normal((4096, 4096), wl.SEED_B), oracle.E2M1)
    check4(A, B, SA, SB, torch.bfloat16, what="4096^3 MXFP4")
