"""Seeded random shapes through every main entry point, each checked against the
oracle with the bound its own parity tests use: gemm_bf16 (both B layouts,
FP32 or BF16 out, with and without C; M <= 128 with B stored N x K takes the
skinny kernel), gemm_fp8_scaled per tensor and per block, quantize_fp8 (bit
for bit), gemm_mxfp8, gemm_bf16_fused (random activation, bias and output
type), gemm_grouped_bf16 (random expert row counts, some empty) and
attention_bf16.  The shapes are drawn once per case index from a
fixed generator, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import oracle
import dense_matrix_unit_amd as dmu
from dense_matrix_unit_amd import workloads as wl
from gpu_helpers import bf16

import test_gpu_attention as att
import test_gpu_gemm_bf16 as gb
import test_gpu_gemm_fp8 as gf
import test_gpu_quantize as gq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("i", range(16))
def test_gemm_bf16_random(i):
    r = np.random.default_rng([1, i])
    M, N, K = int(r.integers(1, 700)), int(r.integers(1, 700)), 8 * int(r.integers(1, 160))
    layout = [dmu.B_ROW_MAJOR, dmu.B_COL_MAJOR][int(r.integers(2))]
    out = [torch.float32, torch.bfloat16][int(r.integers(2))]
    A = bf16(wl.normal((M, K), 100 + i))
    B = gb.make_B(bf16(wl.normal((K, N), 200 + i)), layout)
    C = wl.normal((M, N), 300 + i) if r.integers(2) else None
    gb.check(A, B, layout, out, C=C, what="case %d: M=%d N=%d K=%d layout %d" % (i, M, N, K, layout))


@pytest.mark.parametrize("i", range(10))
def test_gemm_fp8_tensor_random(i):
    r = np.random.default_rng([2, i])
    M, N, K = int(r.integers(1, 600)), int(r.integers(1, 600)), 16 * int(r.integers(1, 75))
    fa, fb = int(r.integers(2)), int(r.integers(2))
    out = [torch.float32, torch.bfloat16][int(r.integers(2))]
    A, sa = gf.quant(wl.normal((M, K), 400 + i), fa)
    B, sb = gf.quant(wl.normal((N, K), 500 + i), fb)
    gf.check(A, B, fa, fb, sa, sb, oracle.SCALE_TENSOR, out,
             what="case %d: M=%d N=%d K=%d fmts %d %d" % (i, M, N, K, fa, fb))


@pytest.mark.parametrize("i", range(6))
def test_gemm_fp8_block_random(i):
    r = np.random.default_rng([3, i])
    M, N, K = int(r.integers(1, 600)), 128 * int(r.integers(1, 5)), 128 * int(r.integers(1, 9))
    fa, fb = int(r.integers(2)), int(r.integers(2))
    A, sa = gf.quant(wl.normal((M, K), 600 + i), fa, (1, 128))
    B, sb = gf.quant(wl.normal((N, K), 700 + i), fb, (128, 128))
    gf.check(A, B, fa, fb, sa, sb, oracle.SCALE_BLOCK, torch.bfloat16,
             what="case %d: M=%d N=%d K=%d fmts %d %d" % (i, M, N, K, fa, fb))


@pytest.mark.parametrize("i", range(12))
def test_quantize_random(i):
    r = np.random.default_rng([4, i])
    block = [None, (1, 128), (128, 128)][i % 3]
    fmt = int(r.integers(2))
    if block is None:
        rows, cols = int(r.integers(1, 500)), 4 * int(r.integers(1, 300))
    elif block == (1, 128):
        rows, cols = int(r.integers(1, 500)), 128 * int(r.integers(1, 9))
    else:
        rows, cols = 128 * int(r.integers(1, 5)), 128 * int(r.integers(1, 6))
    X = wl.normal((rows, cols), 800 + i) * np.float32(10.0 ** float(r.uniform(-3, 3)))
    Q, s = gq.run_quant(X, fmt, block, ldq_pad=(-cols) % 16 or 16 * (i % 2))  # Q rows 16-byte aligned
    gq.compare(X, fmt, block, Q, s)


@pytest.mark.parametrize("i", range(10))
def test_attention_random(i):
    r = np.random.default_rng([5, i])
    causal = bool(r.integers(2))
    d = [64, 128][int(r.integers(2))]
    H, Sq = int(r.integers(1, 4)), int(r.integers(1, 300))
    Sk = int(r.integers(Sq, 420)) if causal else int(r.integers(1, 420))
    Q = att.bf16((H, Sq, d), 900 + i)
    K = att.bf16((H, Sk, d), 1000 + i)
    V = att.bf16((H, Sk, d), 1100 + i)
    scale = float(r.uniform(0.02, 0.3))
    O, lse = att.run(Q, K, V, scale, causal)
    att.check(O, lse, Q, K, V, scale, causal,
              "case %d: H=%d Sq=%d Sk=%d d=%d causal %d" % (i, H, Sq, Sk, d, causal))


@pytest.mark.parametrize("i", range(6))
def test_gemm_mxfp8_random(i):
    import test_gpu_mx as gm
    r = np.random.default_rng([6, i])
    M, N, K = int(r.integers(1, 500)), int(r.integers(1, 500)), 128 * int(r.integers(1, 9))
    fa, fb = int(r.integers(2)), int(r.integers(2))
    out = [torch.float32, torch.bfloat16][int(r.integers(2))]
    A, SA = oracle.quantize_mx(wl.normal((M, K), 1200 + i), fa)
    B, SB = oracle.quantize_mx(wl.normal((N, K), 1300 + i), fb)
    gm.check(A, B, fa, fb, SA, SB, out, what="case %d: M=%d N=%d K=%d fmts %d %d" % (i, M, N, K, fa, fb))


@pytest.mark.parametrize("i", range(8))
def test_gemm_bf16_fused_random(i):
    import test_gpu_fused as fu
    r = np.random.default_rng([7, i])
    M, N, K = int(r.integers(1, 500)), int(r.integers(1, 500)), 8 * int(r.integers(1, 100))
    layout = [dmu.B_ROW_MAJOR, dmu.B_COL_MAJOR][int(r.integers(2))]
    act = int(r.integers(4))
    out_kind = ["f32", "bf16"][int(r.integers(2))]
    A = bf16(wl.normal((M, K), 1400 + i))
    B = gb.make_B(bf16(wl.normal((K, N), 1500 + i)), layout)
    bias = wl.normal((N,), 1600 + i) if r.integers(2) else None
    D = fu.run_bf16_fused(A, B, layout, out_kind, bias, act)
    Dref, S = oracle.gemm_bf16(A, B, layout)
    y = oracle.epilogue(Dref, 1.0, bias, act)
    fu.check_y(D, y, fu.tol_of(S, y, bias), out_kind == "bf16",
               "case %d: M=%d N=%d K=%d layout %d act %d" % (i, M, N, K, layout, act))


@pytest.mark.parametrize("i", range(6))
def test_gemm_grouped_random(i):
    import test_gpu_grouped as gg
    from gpu_helpers import assert_within_bound
    r = np.random.default_rng([8, i])
    G = int(r.integers(1, 12))
    counts = r.integers(0, 400, G)
    counts[r.random(G) < 0.2] = 0  # some experts get no rows
    off = gg.offsets_of(counts)
    N, K = 8 * int(r.integers(1, 50)), 8 * int(r.integers(1, 80))  # D rows 16-byte aligned
    out = [torch.float32, torch.bfloat16][int(r.integers(2))]
    A = bf16(wl.normal((max(int(off[-1]), 1), K), 1700 + i))
    B = bf16(wl.normal((G, N, K), 1800 + i))
    D = gg.run_grouped(A, B, off, out, max_m=int(off[-1]) if off[-1] > 0 else 1)
    Dref, S = oracle.gemm_grouped_bf16(A, B, off)
    rows = int(off[-1])
    assert_within_bound(D[:rows], Dref[:rows], S[:rows], out == torch.bfloat16,
                        what="case %d: counts %s N=%d K=%d" % (i, list(counts), N, K))
