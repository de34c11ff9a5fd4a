"""Parity of gemm_fp8_scaled (HIP) against the FP64 oracle, per-tensor and
per-block (A: 1 x 128, B: 128 x 128) scales, E4M3 and E5M2."""
import numpy as np
import pytest
import torch

import oracle
import dense_matrix_unit_amd as dmu
from dense_matrix_unit_amd import workloads as wl
from gpu_helpers import assert_within_bound, dev, empty_padded, out_to_f64, padded, round_out

pytestmark = pytest.mark.gpu
FMT_PAIRS = [(0, 0), (0, 1), (1, 0), (1, 1)]
OUTS = [torch.float32, torch.bfloat16]


def run_fp8(A, B, fa, fb, sa, sb, mode, out_dtype, C=None):
    M, N = A.shape[0], B.shape[0]
    out = empty_padded(M, N, out_dtype)
    dmu.gemm_fp8_scaled(padded(A, 16), padded(B, 16), dev(np.ascontiguousarray(sa, np.float32)),
                        dev(np.ascontiguousarray(sb, np.float32)), out, fa, fb, mode,
                        C=None if C is None else padded(C, 4))
    torch.cuda.synchronize()
    return out_to_f64(out)


def check(A, B, fa, fb, sa, sb, mode, out_dtype, C=None, rows=None, what=""):
    D = run_fp8(A, B, fa, fb, sa, sb, mode, out_dtype, C)
    Dref, S = oracle.gemm_fp8(A, B, fa, fb, sa, sb, mode, C=C, rows=rows)
    if rows is not None:
        D = D[rows]
    if C is not None:
        S = S + np.abs(C if rows is None else C[rows])
    assert_within_bound(D, Dref, S, out_dtype == torch.bfloat16, what)
    return D, Dref


def quant(X, fmt, block=(None, None)):
    return oracle.quantize_fp8(X, fmt, *block)


@pytest.mark.parametrize("fa,fb", FMT_PAIRS)
@pytest.mark.parametrize("out_dtype", OUTS)
@pytest.mark.parametrize("shape", [(320, 264, 512), (1, 16, 16), (513, 600, 1040)])
def test_per_tensor(fa, fb, out_dtype, shape):
    M, N, K = shape
    A, sa = quant(wl.normal((M, K), 1), fa)
    B, sb = quant(wl.normal((N, K), 2), fb)
    C = wl.normal((M, N), 3) if shape[0] == 320 else None
    check(A, B, fa, fb, sa, sb, dmu.SCALE_TENSOR, out_dtype, C=C, what=str(shape))


@pytest.mark.parametrize("fa,fb", FMT_PAIRS)
@pytest.mark.parametrize("out_dtype", OUTS)
def test_integer_exact(fa, fb, out_dtype):
    M, N, K = 272, 288, 384
    A = oracle.encode_fp8(wl.small_ints((M, K), 1), fa)
    B = oracle.encode_fp8(wl.small_ints((N, K), 2), fb)
    C = wl.small_ints((M, N), 3, -1000, 1000)
    D = run_fp8(A, B, fa, fb, np.float32([2.0]), np.float32([0.5]), dmu.SCALE_TENSOR, out_dtype, C)
    Dref, _ = oracle.gemm_fp8(A, B, fa, fb, np.float32([2.0]), np.float32([0.5]), 0, C=C)
    assert np.array_equal(D, round_out(Dref, out_dtype == torch.bfloat16))
    # per-block power-of-two scales keep every partial exact too
    nkb = K // 128
    sa = (2.0 ** np.random.default_rng(4).integers(-3, 4, (M, nkb))).astype(np.float32)
    sb = (2.0 ** np.random.default_rng(5).integers(-3, 4, ((N + 127) // 128, nkb))).astype(np.float32)
    D = run_fp8(A, B, fa, fb, sa, sb, dmu.SCALE_BLOCK, out_dtype, C)
    Dref, _ = oracle.gemm_fp8(A, B, fa, fb, sa, sb, 1, C=C)
    assert np.array_equal(D, round_out(Dref, out_dtype == torch.bfloat16))


@pytest.mark.parametrize("fa,fb", FMT_PAIRS)
@pytest.mark.parametrize("shape", [(384, 384, 512), (300, 200, 256), (256, 520, 1024)])
def test_block_scaled(fa, fb, shape):
    M, N, K = shape
    Xa, _ = wl.normal_with_outlier_rows((M, K), 1, frac=0.02)
    A, sa = quant(Xa, fa, (1, 128))
    # B is stored N x K; pad N to a multiple of 128 for the 128 x 128 quantizer
    Np = (N + 127) // 128 * 128
    Bp, sb = quant(wl.normal((Np, K), 2), fb, (128, 128))
    B = np.ascontiguousarray(Bp[:N])
    check(A, B, fa, fb, sa, sb, dmu.SCALE_BLOCK, torch.bfloat16, what=str(shape))


def sample_rows(M, n=10, seed=0):
    rng = np.random.default_rng(seed)
    return np.array(sorted(set([0, M - 1]) | set(rng.integers(0, M, n).tolist())), np.int64)


@pytest.mark.parametrize("fmt", [dmu.E4M3, dmu.E5M2])
def test_4096_per_tensor_sampled(fmt):
    A, sa = quant(wl.normal((4096, 4096), wl.SEED_A), fmt)
    B, sb = quant(wl.normal((4096, 4096), wl.SEED_B), fmt)
    check(A, B, fmt, fmt, sa, sb, dmu.SCALE_TENSOR, torch.bfloat16, rows=sample_rows(4096),
          what="4096^3 fmt %d" % fmt)


def test_block_scaled_8192x7168x7168_sampled():
    Xa, out_rows = wl.normal_with_outlier_rows((8192, 7168), wl.SEED_A)
    A, sa = quant(Xa, dmu.E4M3, (1, 128))
    del Xa
    B, sb = quant(wl.normal((7168, 7168), wl.SEED_B), dmu.E4M3, (128, 128))
    rows = np.array(sorted(set(sample_rows(8192, 8).tolist()) | set(out_rows[:4].tolist())), np.int64)
    check(A, B, 0, 0, sa, sb, dmu.SCALE_BLOCK, torch.bfloat16, rows=rows, what="block 8192")
