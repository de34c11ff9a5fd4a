"""Pins for the oracle's FP8 quantizer (amax -> scale -> saturating RNE).

The independent reference below recomputes each block with numpy FP32
arithmetic (IEEE single division and multiplication) and encodes with the
brute-force nearest-code search of test_oracle_codecs, so a slip in the
oracle's block walk, scale formula or encoder shows up as a mismatch.
"""
import numpy as np
import pytest

import oracle
from dense_matrix_unit_amd import workloads as wl
from test_oracle_codecs import brute_force_fp8


def numpy_quantize(X, fmt, br, bc):
    rows, cols = X.shape
    fmax = np.float32(oracle.FMAX[fmt])
    Q = np.empty(X.shape, np.uint8)
    scales = np.empty((rows // br, cols // bc), np.float32)
    for bi in range(rows // br):
        for bj in range(cols // bc):
            blk = X[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc]
            amax = np.float32(np.max(np.abs(blk)))
            if amax == 0:
                m = s = np.float32(1.0)
            else:
                m = np.float32(fmax / amax)
                s = np.float32(amax / fmax)
            y = (blk * m).astype(np.float32)
            Q[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc] = brute_force_fp8(y, fmt).reshape(blk.shape)
            scales[bi, bj] = s
    return Q, scales


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("block", [(None, None), (1, 128), (128, 128)])
def test_quantize_matches_independent_numpy(fmt, block):
    X, _ = wl.normal_with_outlier_rows((256, 384), 7, frac=0.02)
    br = X.shape[0] if block[0] is None else block[0]
    bc = X.shape[1] if block[1] is None else block[1]
    Q, s = oracle.quantize_fp8(X, fmt, *block)
    Qr, sr = numpy_quantize(X, fmt, br, bc)
    assert np.array_equal(s, sr)
    assert np.array_equal(Q, Qr)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_quantize_special_cases(fmt):
    maxcode = 0x7E if fmt == oracle.E4M3 else 0x7B
    fmax = oracle.FMAX[fmt]
    # the element equal to amax maps to +-max; scale is amax/FMAX
    X = wl.normal((4, 128), 3)
    Q, s = oracle.quantize_fp8(X, fmt, 1, 128)
    for r in range(4):
        j = int(np.argmax(np.abs(X[r])))
        assert Q[r, j] & 0x7F == maxcode
        assert s[r, 0] == np.float32(np.float32(np.abs(X[r]).max()) / np.float32(fmax))
    # all-equal block -> every code is +-max
    Q, s = oracle.quantize_fp8(np.full((2, 128), -3.25, np.float32), fmt)
    assert np.all(Q == (0x80 | maxcode))
    # all-zero block -> scale 1, codes +-0
    Z = np.zeros((1, 128), np.float32)
    Z[0, 5] = -0.0
    Q, s = oracle.quantize_fp8(Z, fmt, 1, 128)
    assert s[0, 0] == 1.0 and Q[0, 5] == 0x80 and np.all(np.delete(Q[0], 5) == 0)
    # power-of-two amax: m is exact, so codes are encode(x * 2^p)
    X = np.array([[2.0 ** -3, 0.05, -0.09, 0.11]], np.float32)
    Q, s = oracle.quantize_fp8(X, fmt)
    m = np.float32(fmax) / np.float32(2.0 ** -3)
    assert np.array_equal(Q[0], oracle.encode_fp8((X[0] * m).astype(np.float32), fmt))
    # NaN anywhere in a block -> NaN scale; Inf (no NaN) -> +Inf scale, finite -> 0 codes
    X = wl.normal((2, 128), 4)
    X[0, 7] = np.nan
    X[1, 9] = -np.inf
    Q, s = oracle.quantize_fp8(X, fmt, 1, 128)
    assert np.isnan(s[0, 0]) and s[1, 0] == np.inf
    assert np.all(Q[1, np.isfinite(X[1])] & 0x7F == 0) and Q[1, 9] & 0x7F == 0x7F


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_quantize_dequant_error_within_half_ulp(fmt):
    mbits = 3 if fmt == oracle.E4M3 else 2
    X = wl.normal((128, 256), 9)
    Q, s = oracle.quantize_fp8(X, fmt, 128, 128)
    deq = oracle.decode_fp8(Q, fmt) * np.repeat(np.repeat(s, 128, 0), 128, 1)
    fmax = oracle.FMAX[fmt]
    # normal range after scaling: relative error <= 2^-(mbits+1) (+ FP32 rounding of x*m)
    y = np.abs(X) * (fmax / np.repeat(np.repeat(np.abs(X).reshape(1, 128, 2, 128).max(axis=(1, 3)), 128, 0), 128, 1))
    normal = y >= 2.0 ** (-6 if fmt == oracle.E4M3 else -14)
    rel = np.abs(deq - X)[normal] / np.abs(X)[normal]
    assert rel.max() <= 2.0 ** -(mbits + 1) * (1 + 1e-6)


def test_rel_rms_and_bound_ratio_definitions():
    ref = np.array([3.0, -4.0])
    assert oracle.rel_rms(ref, ref) == 0.0
    assert abs(oracle.rel_rms(ref * 1.001, ref) - 0.001) < 1e-15
    assert oracle.rel_rms(ref + np.array([0.3, 0.4]), ref) == pytest.approx(0.1)
    assert oracle.bound_ratio(np.array([1.0 + 2e-6]), np.array([1.0]), np.array([0.5])) == pytest.approx(4e-6)
    ok = oracle.within_bound(np.array([1.0 + 2 ** -9]), np.array([1.0]), np.array([1.0]), True)
    assert ok.all()
