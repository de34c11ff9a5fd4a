"""Pins for the oracle's microscaling (MX) functions: E8M0 scales, the 1 x 32
block quantizer and the MX product.

The pages ("How Blackwell's Tensor Memory Actually Works", section
"Quantization became an allocation problem") define the block-scaled product
as D = C + (A x SFA)(B x SFB) with one scale per 32 elements along K, scales
being bare powers of two (E8M0) as in the Open Compute microscaling
specification.  The references below are written independently of the
oracle's arithmetic: scales are checked through the property that fixes them
(amax / X lands in [2^emax, 2^(emax+1))), elements through a brute-force
nearest-code search, products through numpy matmul of expanded scales and
through exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_matrix_unit_amd import workloads as wl
from test_oracle_codecs import brute_force_fp8

EMAX = {oracle.E4M3: 8, oracle.E5M2: 15}
FMTS = [oracle.E4M3, oracle.E5M2]


def test_e8m0_codes_are_powers_of_two():
    v = oracle.decode_e8m0(np.arange(256))
    assert v[127] == 1.0 and np.isnan(v[255])
    # each code doubles the previous one; code 0 is 2^-127
    assert v[0] == 2.0 ** -127
    assert np.all(v[1:255] == 2.0 * v[0:254])


def mx_blocks(X):
    r, c = X.shape
    return X.reshape(r, c // 32, 32)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_mx_scale_property_and_nearest_codes(fmt):
    X, _ = wl.normal_with_outlier_rows((64, 512), 11, frac=0.05)
    X[3, :64] *= np.float32(1e-30)   # tiny blocks
    X[5, 64:96] *= np.float32(1e30)  # huge block
    Q, S = oracle.quantize_mx(X, fmt)
    scale = oracle.decode_e8m0(S)
    amax = np.abs(mx_blocks(X.astype(np.float64))).max(axis=2)
    ratio = amax / scale
    clamped = (S == 0) | (S == 254)
    assert np.all((ratio[~clamped] >= 2.0 ** EMAX[fmt]) & (ratio[~clamped] < 2.0 ** (EMAX[fmt] + 1)))
    # elements: nearest code (ties to even, saturating) of x / X
    y = mx_blocks(X.astype(np.float64)) / scale[:, :, None]
    expect = brute_force_fp8(y.ravel(), fmt).reshape(Q.shape)
    assert np.array_equal(Q, expect)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_mx_worked_values_and_special_blocks(fmt):
    X = np.zeros((4, 64), np.float32)
    X[0, :32] = 1.0                        # amax 1: X = 2^-emax, elements 2^emax
    X[0, 32] = 448.0                       # amax in [256, 512): scale 2^(8-emax)
    X[1, :32] = -0.0                       # all-zero block (signed zeros)
    X[2, 5] = np.nan                       # NaN block
    X[3, 40] = -np.inf                     # Inf block
    Q, S = oracle.quantize_mx(X, fmt)
    e = EMAX[fmt]
    assert S[0, 0] == 127 - e
    assert np.all(oracle.decode_fp8(Q[0, :32], fmt) == 2.0 ** e)
    assert S[0, 1] == 127 + 8 - e
    assert S[1, 0] == 0 and np.all(Q[1, :32] == 0x80)
    assert S[2, 0] == 255 and np.all(np.isnan(oracle.decode_fp8(Q[2, :32], fmt)))
    assert S[3, 1] == 255 and np.all(np.isnan(oracle.decode_fp8(Q[3, 32:], fmt)))
    assert S[1, 1] == 0 and S[2, 1] == 0  # untouched all-zero blocks


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_mx_power_of_two_equivariance(fmt):
    # scaling a tensor by 2^t changes only the scale codes, by t
    X = wl.normal((16, 256), 21)
    Q0, S0 = oracle.quantize_mx(X, fmt)
    for t in (-9, 1, 17):
        Q1, S1 = oracle.quantize_mx((X * np.float32(2.0 ** t)).astype(np.float32), fmt)
        assert np.array_equal(Q1, Q0)
        assert np.array_equal(S1.astype(int), S0.astype(int) + t)


def expand(S):
    return np.repeat(oracle.decode_e8m0(S), 32, axis=1)


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (1, 1)])
def test_gemm_mx_matches_numpy_with_expanded_scales(fa, fb):
    rng = np.random.default_rng(5)
    M, N, K = 40, 24, 256
    A = oracle.encode_fp8(wl.normal((M, K), 1), fa)
    B = oracle.encode_fp8(wl.normal((N, K), 2), fb)
    SA = rng.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    SB = rng.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    C = wl.normal((M, N), 3)
    D, S = oracle.gemm_mx(A, B, fa, fb, SA, SB, C=C)
    a = oracle.decode_fp8(A, fa) * expand(SA)
    b = oracle.decode_fp8(B, fb) * expand(SB)
    ref = a @ b.T + C.astype(np.float64)
    assert np.all(np.abs(D - ref) <= 1e-12 * (S + np.abs(C)))
    assert np.allclose(S, np.abs(a) @ np.abs(b).T, rtol=1e-12)


def test_gemm_mx_unit_scales_reduce_to_fp8():
    A = oracle.encode_fp8(wl.normal((32, 128), 4), 0)
    B = oracle.encode_fp8(wl.normal((16, 128), 5), 0)
    ones_a = np.full((32, 4), 127, np.uint8)
    ones_b = np.full((16, 4), 127, np.uint8)
    D, _ = oracle.gemm_mx(A, B, 0, 0, ones_a, ones_b)
    D8, _ = oracle.gemm_fp8(A, B, 0, 0, np.float32([1.0]), np.float32([1.0]), oracle.SCALE_TENSOR)
    assert np.array_equal(D, D8)


def test_gemm_mx_brute_force_rational_16():
    # small integers times powers of two: every product and sum is exact
    rng = np.random.default_rng(9)
    M, N, K = 16, 16, 64
    A = oracle.encode_fp8(wl.small_ints((M, K), 6), 0)
    B = oracle.encode_fp8(wl.small_ints((N, K), 7), 1)
    SA = rng.integers(120, 135, size=(M, 2)).astype(np.uint8)
    SB = rng.integers(120, 135, size=(N, 2)).astype(np.uint8)
    D, _ = oracle.gemm_mx(A, B, 0, 1, SA, SB)
    av = oracle.decode_fp8(A, 0)
    bv = oracle.decode_fp8(B, 1)
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (Fraction(av[i, k]) * Fraction(2) ** (int(SA[i, k // 32]) - 127) *
                        Fraction(bv[j, k]) * Fraction(2) ** (int(SB[j, k // 32]) - 127))
            assert D[i, j] == float(acc)


def test_gemm_mx_scale_code_step_doubles_one_block():
    A = oracle.encode_fp8(wl.normal((8, 128), 12), 0)
    B = oracle.encode_fp8(wl.normal((8, 128), 13), 0)
    SA = np.full((8, 4), 127, np.uint8)
    SB = np.full((8, 4), 127, np.uint8)
    D0, _ = oracle.gemm_mx(A, B, 0, 0, SA, SB)
    SA2 = SA.copy()
    SA2[2, 1] += 1
    D1, _ = oracle.gemm_mx(A, B, 0, 0, SA2, SB)
    a = oracle.decode_fp8(A, 0)
    b = oracle.decode_fp8(B, 0)
    block = a[2, 32:64] @ b[:, 32:64].T
    assert np.allclose(D1[2] - D0[2], block, rtol=0, atol=1e-12 * np.abs(block).max())
    assert np.array_equal(np.delete(D1, 2, axis=0), np.delete(D0, 2, axis=0))


# ---------------------------------------------------------------- MXFP4 (E2M1)

import json
import os

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp4_e2m1.json")))
MAGS = np.array(GOLD["magnitudes"])


def test_fp4_decode_matches_the_format_table():
    v = oracle.decode_fp4(np.arange(16))
    assert np.array_equal(v[:8], MAGS)
    assert np.array_equal(v[8:], -MAGS)
    assert np.signbit(v[8])  # code 8 is -0
    # the table itself follows from the field split: subnormal m/2, normal (1 + m/2) 2^(e - 1)
    for c in range(8):
        e, m = c >> 1, c & 1
        want = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - GOLD["bias"])
        assert Fraction(MAGS[c]) == want


def brute_fp4(x):
    """nearest E2M1 value, ties to the even code, saturating at +-6, -0 kept"""
    out = np.empty(np.shape(x), np.uint8)
    for idx, xv in np.ndenumerate(np.asarray(x, np.float64)):
        s = 8 if np.signbit(xv) else 0
        a = min(abs(xv), MAGS[-1])
        d = np.abs(MAGS - a)
        cands = np.flatnonzero(d == d.min())
        c = cands[0] if len(cands) == 1 else [k for k in cands if k % 2 == 0][0]
        out[idx] = s | c
    return out


def test_fp4_encode_is_the_nearest_code():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-8, 8, 4000), MAGS, -MAGS, (MAGS[1:] + MAGS[:-1]) / 2,
                        [0.25, -0.25, 7.0, 1e9, -1e9, np.inf, -np.inf, -0.0, 1e-30]]).astype(np.float32)
    assert np.array_equal(oracle.encode_fp4(x), brute_fp4(x))
    # decode o encode is the identity on every code
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(oracle.encode_fp4(oracle.decode_fp4(codes).astype(np.float32)), codes)


def test_fp4_packing_order():
    codes = np.array([[1, 2, 3, 4, 15, 8]], np.uint8)
    p = oracle.pack_fp4(codes)
    assert p.tolist() == [[0x21, 0x43, 0x8F]]
    assert np.array_equal(oracle.unpack_fp4(p), codes)


def test_quantize_mx_fp4_scale_property_and_nearest_codes():
    X, _ = wl.normal_with_outlier_rows((48, 256), 17, frac=0.05)
    X[3, :32] *= np.float32(1e-30)
    X[6, 64:96] *= np.float32(1e25)
    Q, S = oracle.quantize_mx(X, oracle.E2M1)
    assert Q.shape == (48, 128)
    scale = oracle.decode_e8m0(S)
    amax = np.abs(mx_blocks(X.astype(np.float64))).max(axis=2)
    ratio = amax / scale
    clamped = (S == 0) | (S == 254)
    assert np.all((ratio[~clamped] >= 4.0) & (ratio[~clamped] < 8.0))
    y = mx_blocks(X.astype(np.float64)) / scale[:, :, None]
    assert np.array_equal(oracle.unpack_fp4(Q), brute_fp4(y.ravel()).reshape(X.shape))


def test_quantize_mx_fp4_worked_values_and_special_blocks():
    X = np.zeros((3, 96), np.float32)
    X[0, :32] = 6.0              # amax 6: X = 1, every element code 7
    X[0, 32:64] = 1.0            # amax 1: X = 2^-2, elements 4 -> code 6
    X[0, 64] = -5.0              # amax 5: X = 1, -5 ties between 4 and 6 -> even code: -4
    X[1, 3] = np.nan             # NaN block: code 255, signed zeros
    X[1, 4] = -1.0
    X[2, 40] = np.inf
    Q, S = oracle.quantize_mx(X, oracle.E2M1)
    q = oracle.unpack_fp4(Q)
    assert S[0].tolist() == [127, 125, 127]
    assert np.all(q[0, :32] == 7) and np.all(q[0, 32:64] == 6) and q[0, 64] == 8 | 6
    assert S[1, 0] == 255 and np.all(q[1, :32] == np.where(np.signbit(X[1, :32]), 8, 0))
    assert S[2, 1] == 255 and S[2, 0] == 0 and S[2, 2] == 0


def test_quantize_mx_fp4_power_of_two_equivariance():
    X = wl.normal((8, 128), 23)
    Q0, S0 = oracle.quantize_mx(X, oracle.E2M1)
    for t in (-5, 3, 40):
        Q1, S1 = oracle.quantize_mx((X * np.float32(2.0 ** t)).astype(np.float32), oracle.E2M1)
        assert np.array_equal(Q1, Q0)
        assert np.array_equal(S1.astype(int), S0.astype(int) + t)


@pytest.mark.parametrize("fa,fb", [(4, 4), (4, 0), (1, 4)])
def test_gemm_mx_fp4_matches_numpy(fa, fb):
    rng = np.random.default_rng(31)
    M, N, K = 24, 40, 192

    def make(rows, seed, fmt):
        X = wl.normal((rows, K), seed)
        return oracle.pack_fp4(oracle.encode_fp4(X)) if fmt == oracle.E2M1 else oracle.encode_fp8(X, fmt)
    A, B = make(M, 1, fa), make(N, 2, fb)
    SA = rng.integers(112, 142, size=(M, K // 32)).astype(np.uint8)
    SB = rng.integers(112, 142, size=(N, K // 32)).astype(np.uint8)
    C = wl.normal((M, N), 3)
    D, S = oracle.gemm_mx(A, B, fa, fb, SA, SB, C=C)
    a = oracle.decode_elems(A, fa) * expand(SA)
    b = oracle.decode_elems(B, fb) * expand(SB)
    ref = a @ b.T + C.astype(np.float64)
    assert np.all(np.abs(D - ref) <= 1e-12 * (S + np.abs(C)))


def test_gemm_mx_fp4_brute_force_rational():
    rng = np.random.default_rng(37)
    M, N, K = 8, 8, 64
    qa = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    qb = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    SA = rng.integers(120, 135, size=(M, 2)).astype(np.uint8)
    SB = rng.integers(120, 135, size=(N, 2)).astype(np.uint8)
    D, _ = oracle.gemm_mx(oracle.pack_fp4(qa), oracle.pack_fp4(qb), 4, 4, SA, SB)
    sgn = lambda c: -1 if c & 8 else 1
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                va = sgn(qa[i, k]) * Fraction(MAGS[qa[i, k] & 7])
                vb = sgn(qb[j, k]) * Fraction(MAGS[qb[j, k] & 7])
                acc += (va * Fraction(2) ** (int(SA[i, k // 32]) - 127) *
                        vb * Fraction(2) ** (int(SB[j, k // 32]) - 127))
            assert D[i, j] == float(acc)
