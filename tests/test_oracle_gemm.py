"""Pins for the oracle's FP64 GEMMs (BF16 and scaled FP8).

Pins: identity/permutation products, small-integer inputs against an int64
matmul, closed forms, an exact-rational brute force on 16x16x16, numpy's FP64
matmul on decoded operands, and scaling invariants.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from dense_matrix_unit_amd import workloads as wl

BF16_ONE = 0x3F80


def to_bf16(x):
    return oracle.encode_bf16(np.asarray(x, np.float32))


def layout_B(Bkn, layout):
    """Return B (K x N logical) stored in the requested layout."""
    return Bkn if layout == oracle.B_ROW_MAJOR else np.ascontiguousarray(Bkn.T)


@pytest.mark.parametrize("layout", [oracle.B_ROW_MAJOR, oracle.B_COL_MAJOR])
def test_identity_and_permutation(layout):
    K = N = 48
    rng = np.random.default_rng(0)
    Bf = wl.normal((K, N), 5)
    Bq = to_bf16(Bf)
    Bdec = oracle.decode_bf16(Bq)
    I = np.zeros((K, K), np.uint16)
    I[np.arange(K), np.arange(K)] = BF16_ONE
    D, S = oracle.gemm_bf16(I, layout_B(Bq, layout), layout)
    assert np.array_equal(D, Bdec)
    assert np.array_equal(S, np.abs(Bdec))
    perm = rng.permutation(K)
    P = np.zeros((K, K), np.uint16)
    P[np.arange(K), perm] = BF16_ONE
    D, _ = oracle.gemm_bf16(P, layout_B(Bq, layout), layout)
    assert np.array_equal(D, Bdec[perm])


@pytest.mark.parametrize("layout", [oracle.B_ROW_MAJOR, oracle.B_COL_MAJOR])
def test_small_integers_exact_vs_int64(layout):
    M, N, K = 37, 53, 96
    A = wl.small_ints((M, K), 1)
    B = wl.small_ints((K, N), 2)
    C = wl.small_ints((M, N), 3, -100, 100)
    D, S = oracle.gemm_bf16(to_bf16(A), layout_B(to_bf16(B), layout), layout, C=C)
    ref = A.astype(np.int64) @ B.astype(np.int64) + C.astype(np.int64)
    assert np.array_equal(D, ref.astype(np.float64))
    assert np.array_equal(S, (np.abs(A).astype(np.int64) @ np.abs(B).astype(np.int64)).astype(np.float64))


def test_closed_form_ones_times_pattern():
    M, N, K = 8, 24, 70
    A = np.full((M, K), BF16_ONE, np.uint16)
    k = np.arange(K)[:, None]
    Bf = ((k % 7) - 3 + 0 * np.arange(N)[None, :]).astype(np.float32)
    D, _ = oracle.gemm_bf16(A, to_bf16(Bf), oracle.B_ROW_MAJOR)
    expect = float(sum((kk % 7) - 3 for kk in range(K)))
    assert np.all(D == expect)


def test_rows_subset_matches_full():
    M, N, K = 40, 33, 64
    A = to_bf16(wl.normal((M, K), 1))
    B = to_bf16(wl.normal((N, K), 2))
    Dfull, Sfull = oracle.gemm_bf16(A, B, oracle.B_COL_MAJOR)
    rows = [39, 0, 17]
    D, S = oracle.gemm_bf16(A, B, oracle.B_COL_MAJOR, rows=rows)
    assert np.array_equal(D, Dfull[rows]) and np.array_equal(S, Sfull[rows])


def exact_product(Adec, Bdec):
    """Exact rational A*B by a naive triple loop (16x16x16)."""
    M, K = Adec.shape
    N = Bdec.shape[1]
    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(float(Adec[i, k])) * Fraction(float(Bdec[k, j]))
            out[i][j] = s
    return out


@pytest.mark.parametrize("layout", [oracle.B_ROW_MAJOR, oracle.B_COL_MAJOR])
def test_brute_force_rational_16(layout):
    A = to_bf16(wl.normal((16, 16), 21))
    B = to_bf16(wl.normal((16, 16), 22))
    Ad, Bd = oracle.decode_bf16(A), oracle.decode_bf16(B)
    # FP64 holds every partial sum exactly when the products' exponents span
    # fewer than 53 - 16 bits; check that, so exact equality is the right test.
    p = np.abs(Ad[:, :, None] * Bd[None, :, :])
    p = p[p > 0]
    assert np.log2(p.max() / p.min()) < 30
    ex = exact_product(Ad, Bd)
    D, _ = oracle.gemm_bf16(A, layout_B(B, layout), layout)
    for i in range(16):
        for j in range(16):
            assert D[i, j] == float(ex[i][j])


def test_fp8_brute_force_rational_16():
    for fmt in (oracle.E4M3, oracle.E5M2):
        A, sa = oracle.quantize_fp8(wl.normal((16, 16), 23), fmt)
        B, sb = oracle.quantize_fp8(wl.normal((16, 16), 24), fmt)
        Ad, Bd = oracle.decode_fp8(A, fmt), oracle.decode_fp8(B, fmt)
        ex = exact_product(Ad, Bd.T)
        D, _ = oracle.gemm_fp8(A, B, fmt, fmt, sa, sb, oracle.SCALE_TENSOR)
        sc = Fraction(float(sa[0, 0])) * Fraction(float(sb[0, 0]))
        for i in range(16):
            for j in range(16):
                # the oracle forms the FP64 sum, then multiplies by the FP64 scale product
                assert D[i, j] == float(Fraction(float(ex[i][j])) * Fraction(float(sc)))


@pytest.mark.parametrize("shape", [(256, 256, 256), (96, 200, 320)])
def test_matches_numpy_fp64(shape):
    M, N, K = shape
    A = to_bf16(wl.uniform_pm1((M, K), 1))
    B = to_bf16(wl.uniform_pm1((K, N), 2))
    C = wl.normal((M, N), 3)
    Ad, Bd = oracle.decode_bf16(A), oracle.decode_bf16(B)
    ref = Ad @ Bd + C.astype(np.float64)
    for layout in (oracle.B_ROW_MAJOR, oracle.B_COL_MAJOR):
        D, S = oracle.gemm_bf16(A, layout_B(B, layout), layout, C=C)
        assert np.all(np.abs(D - ref) <= 1e-12 * (S + np.abs(C)))
        assert np.allclose(S, np.abs(Ad) @ np.abs(Bd), rtol=1e-12)


def test_fp8_matches_torch_float8_decode_and_numpy():
    M, N, K = 64, 96, 256
    for fmt, tdt in ((oracle.E4M3, torch.float8_e4m3fn), (oracle.E5M2, torch.float8_e5m2)):
        A, sa = oracle.quantize_fp8(wl.normal((M, K), 1), fmt)
        B, sb = oracle.quantize_fp8(wl.normal((N, K), 2), fmt)
        Ad = torch.from_numpy(A).view(tdt).double().numpy()
        Bd = torch.from_numpy(B).view(tdt).double().numpy()
        ref = (Ad @ Bd.T) * (float(sa[0, 0]) * float(sb[0, 0]))
        D, S = oracle.gemm_fp8(A, B, fmt, fmt, sa, sb, oracle.SCALE_TENSOR)
        assert np.all(np.abs(D - ref) <= 1e-12 * S)


def fp8_small_int_codes(shape, seed, fmt):
    # integers in [-4, 4] are exact in both FP8 formats
    x = wl.small_ints(shape, seed)
    return oracle.encode_fp8(x, fmt), x.astype(np.int64)


def test_fp8_block_equal_scales_reduce_to_tensor_and_closed_forms():
    M, N, K = 20, 256, 512
    fmt = oracle.E4M3
    A, Ai = fp8_small_int_codes((M, K), 1, fmt)
    B, Bi = fp8_small_int_codes((N, K), 2, fmt)
    nkb = K // 128
    # all scales equal -> same as per-tensor (exact: integer sums, power-of-two scale)
    sa_b = np.full((M, nkb), 0.5, np.float32)
    sb_b = np.full((N // 128, nkb), 4.0, np.float32)
    Db, Sb = oracle.gemm_fp8(A, B, fmt, fmt, sa_b, sb_b, oracle.SCALE_BLOCK)
    Dt, St = oracle.gemm_fp8(A, B, fmt, fmt, np.float32([0.5]), np.float32([4.0]),
                             oracle.SCALE_TENSOR)
    assert np.array_equal(Db, Dt) and np.array_equal(Sb, St)
    assert np.array_equal(Dt, 2.0 * (Ai @ Bi.T))
    # per-block scales 2^kb on A rows (row-dependent) and 3^(jb) on B blocks:
    # D = sum_kb 2^(kb + i%3) * 3^(j//128) * (A_kb @ B_kb^T)
    sa = np.array([[2.0 ** (kb + i % 3) for kb in range(nkb)] for i in range(M)], np.float32)
    sb = np.array([[3.0 ** jb for _ in range(nkb)] for jb in range(N // 128)], np.float32)
    D, _ = oracle.gemm_fp8(A, B, fmt, fmt, sa, sb, oracle.SCALE_BLOCK)
    ref = np.zeros((M, N), np.float64)
    for kb in range(nkb):
        part = Ai[:, kb * 128:(kb + 1) * 128] @ Bi[:, kb * 128:(kb + 1) * 128].T
        ref += part * sa[:, kb:kb + 1].astype(np.float64) * np.repeat(sb[:, kb], 128)[None, :]
    assert np.array_equal(D, ref)


def test_power_of_two_scale_and_C_exact():
    M, N, K = 16, 32, 128
    fmt = oracle.E5M2
    A, Ai = fp8_small_int_codes((M, K), 3, fmt)
    B, Bi = fp8_small_int_codes((N, K), 4, fmt)
    C = wl.small_ints((M, N), 5, -50, 50)
    D1, _ = oracle.gemm_fp8(A, B, fmt, fmt, np.float32([1.0]), np.float32([1.0]), 0)
    D8, _ = oracle.gemm_fp8(A, B, fmt, fmt, np.float32([8.0]), np.float32([1.0]), 0, C=C)
    assert np.array_equal(D8, 8.0 * D1 + C)
