"""Parity of gemm_bf16 (HIP, gfx950) against the FP64 oracle.

Bound (FP32 out): |D - D_ref| <= 1e-5 * sum_k |a_ik b_kj|; BF16 out adds
2^-8 * |D_ref|.  Integer-valued inputs must match exactly.  Sizes span several
256 x 256 tiles with ragged M, N and K tails; the full-size workloads are
checked on sampled rows the oracle computes one by one."""
import numpy as np
import pytest
import torch

import oracle
import dense_matrix_unit_amd as dmu
from dense_matrix_unit_amd import workloads as wl
from gpu_helpers import (assert_within_bound, bf16, dev, empty_padded, out_to_f64, round_out,
                         run_gemm_bf16)

pytestmark = pytest.mark.gpu
LAYOUTS = [dmu.B_ROW_MAJOR, dmu.B_COL_MAJOR]
OUTS = [torch.float32, torch.bfloat16]


def make_B(Bkn, layout):
    return Bkn if layout == dmu.B_ROW_MAJOR else np.ascontiguousarray(Bkn.T)


def check(A, B, layout, out_dtype, C=None, rows=None, what=""):
    out = run_gemm_bf16(A, B, layout, out_dtype, C)
    D = out_to_f64(out)
    Dref, S = oracle.gemm_bf16(A, B, layout, C=C, rows=rows)
    if rows is not None:
        D = D[rows]
    if C is not None:
        S = S + np.abs(C if rows is None else C[rows])
    assert_within_bound(D, Dref, S, out_dtype == torch.bfloat16, what)
    return D, Dref


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("out_dtype", OUTS)
def test_256_uniform(layout, out_dtype):
    # 256^3, A and B from U[-1, 1) rounded to BF16, FP32 (and BF16) output
    A = bf16(wl.uniform_pm1((256, 256), wl.SEED_A))
    B = make_B(bf16(wl.uniform_pm1((256, 256), wl.SEED_B)), layout)
    D, Dref = check(A, B, layout, out_dtype, what="256^3")
    if out_dtype == torch.float32:
        assert oracle.rel_rms(D, Dref) < 1e-6


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("out_dtype", OUTS)
@pytest.mark.parametrize("shape", [(300, 200, 264), (1, 8, 8), (17, 1000, 40),
                                   (513, 257, 1032), (64, 520, 4104)])
def test_ragged(layout, out_dtype, shape):
    M, N, K = shape
    A = bf16(wl.normal((M, K), 11))
    B = make_B(bf16(wl.normal((K, N), 12)), layout)
    check(A, B, layout, out_dtype, what=str(shape))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("out_dtype", OUTS)
def test_integer_inputs_exact(layout, out_dtype):
    M, N, K = 384, 320, 576
    A = bf16(wl.small_ints((M, K), 1))
    B = make_B(bf16(wl.small_ints((K, N), 2)), layout)
    C = wl.small_ints((M, N), 3, -1000, 1000)
    out = run_gemm_bf16(A, B, layout, out_dtype, C)
    Dref, _ = oracle.gemm_bf16(A, B, layout, C=C)
    assert np.array_equal(out_to_f64(out), round_out(Dref, out_dtype == torch.bfloat16))


def test_c_in_place():
    M, N, K = 260, 300, 128
    A = bf16(wl.normal((M, K), 5))
    B = bf16(wl.normal((N, K), 6))
    C = wl.normal((M, N), 7)
    Dg = dev(C.copy())
    dmu.gemm_bf16(dev(A), dev(B), Dg, dmu.B_COL_MAJOR, C=Dg)
    torch.cuda.synchronize()
    Dref, S = oracle.gemm_bf16(A, B, dmu.B_COL_MAJOR, C=C)
    assert_within_bound(out_to_f64(Dg), Dref, S + np.abs(C), False, "in-place C")


def test_strided_operands():
    M, N, K = 200, 136, 192
    Abig = bf16(wl.normal((M, K + 64), 8))
    Bbig = bf16(wl.normal((N, K + 32), 9))
    A_t, B_t = dev(Abig)[:, :K], dev(Bbig)[:, :K]
    out_big = torch.zeros((M, N + 8), dtype=torch.float32, device="cuda")
    out = out_big[:, :N]
    dmu.gemm_bf16(A_t, B_t, out, dmu.B_COL_MAJOR)
    torch.cuda.synchronize()
    Dref, S = oracle.gemm_bf16(np.ascontiguousarray(Abig[:, :K]),
                               np.ascontiguousarray(Bbig[:, :K]), dmu.B_COL_MAJOR)
    assert_within_bound(out.cpu().numpy().astype(np.float64), Dref, S, False, "strided")
    assert torch.all(out_big[:, N:] == 0)


@pytest.mark.parametrize("out_dtype", OUTS)
@pytest.mark.parametrize("shape", [(300, 200, 264), (513, 257, 1032), (64, 520, 4104),
                                   (40, 1000, 8)])
def test_row_major_b_reads_nothing_outside_the_view(out_dtype, shape):
    # B (K x N, row-major) is a view into a larger buffer whose other rows and
    # columns hold NaN: neither the rows past K (the K tail of the last
    # slice) nor the columns past N may reach D
    M, N, K = shape
    A = bf16(wl.normal((M, K), 41))
    B = bf16(wl.normal((K, N), 42))
    ldb = (N + 7) // 8 * 8 + 8
    big = torch.full((K + 64, ldb), float("nan"), dtype=torch.bfloat16, device="cuda")
    big[:K, :N] = dev(B)
    out = empty_padded(M, N, out_dtype)
    dmu.gemm_bf16(dev(A), big[:K, :N], out, dmu.B_ROW_MAJOR)
    torch.cuda.synchronize()
    Dref, S = oracle.gemm_bf16(A, B, dmu.B_ROW_MAJOR)
    assert_within_bound(out_to_f64(out), Dref, S, out_dtype == torch.bfloat16,
                        "row-major B view %s" % (shape,))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_4096_normal_bf16_out(layout):
    # 4096^3, N(0,1) inputs in BF16, BF16 output, B row- and column-major:
    # every one of the 16.8 M outputs against the oracle
    A = bf16(wl.normal((4096, 4096), wl.SEED_A))
    B = make_B(bf16(wl.normal((4096, 4096), wl.SEED_B)), layout)
    check(A, B, layout, torch.bfloat16, what="4096^3")


@pytest.mark.parametrize("M", [16, 128, 1024, 8192])
def test_llm_shapes(M):
    # N = 28672, K = 8192, every output (M = 8192: 235 M outputs)
    N, K = 28672, 8192
    A = bf16(wl.normal((M, K), wl.SEED_A))
    B = bf16(wl.normal((N, K), wl.SEED_B))
    check(A, B, dmu.B_COL_MAJOR, torch.bfloat16, what="M=%d" % M)


@pytest.mark.parametrize("K", [256, 1024, 4096, 16384, 65536])
def test_accuracy_vs_k(K):
    # M = N = 256, N(0,1) inputs in BF16, FP32 output; error against FP64 of
    # the rounded inputs ("from the sums") and of the FP32 sources ("total")
    Af = wl.normal((256, K), wl.SEED_A)
    Bf = wl.normal((256, K), wl.SEED_B)
    A, B = bf16(Af), bf16(Bf)
    D, Dref = check(A, B, dmu.B_COL_MAJOR, torch.float32, what="K=%d" % K)
    total_ref = Af.astype(np.float64) @ Bf.astype(np.float64).T
    print("K=%d rel-RMS sums %.3e total %.3e" % (K, oracle.rel_rms(D, Dref),
                                                 oracle.rel_rms(D, total_ref)))
    assert oracle.rel_rms(D, Dref) < 1e-5


@pytest.mark.parametrize("out_dtype", OUTS)
@pytest.mark.parametrize("shape", [(1, 113, 8), (5, 1000, 264), (33, 250, 520), (100, 3000, 1032),
                                   (128, 224, 4096), (16, 2000, 8192),
                                   (24, 700, 776), (64, 900, 1800)])
def test_skinny_m(out_dtype, shape):
    # M <= 128 with B stored N x K takes the bandwidth-bound skinny kernel
    M, N, K = shape
    A = bf16(wl.normal((M, K), 31))
    B = bf16(wl.normal((N, K), 32))
    C = wl.normal((M, N), 33)
    check(A, B, dmu.B_COL_MAJOR, out_dtype, C=C, what="skinny %s" % (shape,))


@pytest.mark.parametrize("layout", [dmu.LDS_SWIZZLED, dmu.LDS_PLAIN, dmu.LDS_PADDED])
@pytest.mark.parametrize("shape", [(256, 256, 512), (300, 520, 1024), (4096, 4096, 4096)])
def test_lds_layout_variants(layout, shape):
    # the bank-conflict ablation's kernels (swizzled, plain and padded LDS
    # rows) issue the same MFMAs on the same fragments, only the LDS addresses
    # differ: every output bit-identical to gemm_bf16's kernel (itself checked
    # against the oracle in full), and integer data exact
    M, N, K = shape
    A = bf16(wl.normal((M, K), 41))
    B = bf16(wl.normal((N, K), 42))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dmu.probe_gemm_bf16_layout(layout, dev(A), dev(B), out)
    ref = run_gemm_bf16(A, B, dmu.B_COL_MAJOR, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(out_to_f64(out), out_to_f64(ref))
    if M <= 512:
        Ai = bf16(wl.small_ints((M, K), 43))
        Bi = bf16(wl.small_ints((N, K), 44))
        dmu.probe_gemm_bf16_layout(layout, dev(Ai), dev(Bi), out)
        torch.cuda.synchronize()
        Dref, _ = oracle.gemm_bf16(Ai, Bi, dmu.B_COL_MAJOR)
        assert np.array_equal(out_to_f64(out), round_out(Dref, True))
