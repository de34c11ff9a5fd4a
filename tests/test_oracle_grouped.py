"""Pins for the oracle's grouped (mixture-of-experts) product: rows
offsets[g] .. offsets[g+1]-1 of A use expert g's weight ("How Blackwell's
Tensor Memory Actually Works", section "What this does to serving economics",
third consequence: every expert's GEMM has its own M, set by routing).

References independent of the oracle's arithmetic: integer matmul per group,
numpy FP64 per group, and the block-diagonal reading (one GEMM against all
experts' weights stacked, keeping each row's own expert's columns)."""
import numpy as np
import pytest

import oracle
from dense_matrix_unit_amd import workloads as wl


def bf16(x):
    return oracle.encode_bf16(np.asarray(x, np.float32))


def offsets_of(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def test_grouped_integer_exact_per_group():
    counts = np.array([3, 0, 17, 1, 9, 0])
    off = offsets_of(counts)
    G, N, K = len(counts), 12, 40
    Ai = wl.small_ints((off[-1], K), 1, -8, 8)
    Bi = wl.small_ints((G, N, K), 2, -8, 8)
    D, _ = oracle.gemm_grouped_bf16(bf16(Ai), bf16(Bi), off)
    for g in range(G):
        ref = Ai[off[g]:off[g + 1]].astype(np.int64) @ Bi[g].astype(np.int64).T
        assert np.array_equal(D[off[g]:off[g + 1]], ref.astype(np.float64))


def test_grouped_matches_numpy_and_block_diagonal():
    counts = wl.expert_rows(7, 300, 5, spread=1.0)
    off = offsets_of(counts)
    G, N, K = 7, 24, 96
    A = bf16(wl.normal((off[-1], K), 3))
    B = bf16(wl.normal((G, N, K), 4))
    D, S = oracle.gemm_grouped_bf16(A, B, off)
    a = oracle.decode_bf16(A)
    b = oracle.decode_bf16(B)
    full = a @ b.reshape(G * N, K).T            # every row against every expert
    for g in range(G):
        rows = slice(off[g], off[g + 1])
        ref = a[rows] @ b[g].T
        assert np.all(np.abs(D[rows] - ref) <= 1e-12 * S[rows])
        assert np.all(np.abs(D[rows] - full[rows, g * N:(g + 1) * N]) <= 1e-12 * S[rows])
    assert np.allclose(S, np.concatenate([np.abs(a[off[g]:off[g + 1]]) @ np.abs(b[g]).T
                                          for g in range(G)]), rtol=1e-12)


def test_grouped_one_expert_is_the_plain_product():
    A = bf16(wl.normal((50, 64), 7))
    B = bf16(wl.normal((1, 20, 64), 8))
    D, S = oracle.gemm_grouped_bf16(A, B, [0, 50])
    D1, S1 = oracle.gemm_bf16(A, B[0], oracle.B_COL_MAJOR)
    assert np.array_equal(D, D1) and np.array_equal(S, S1)


def test_grouped_selected_rows_and_errors():
    off = np.array([2, 5, 5, 9], np.int64)      # rows 0, 1 and 9.. belong to no expert
    A = bf16(wl.normal((12, 32), 9))
    B = bf16(wl.normal((3, 8, 32), 10))
    D, _ = oracle.gemm_grouped_bf16(A, B, off)
    assert D.shape == (7, 8)
    Dr, _ = oracle.gemm_grouped_bf16(A, B, off, rows=[8, 2])
    assert np.array_equal(Dr, D[[6, 0]])
    with pytest.raises(ValueError):
        oracle.gemm_grouped_bf16(A, B, off, rows=[1])
    with pytest.raises(ValueError):
        oracle.gemm_grouped_bf16(A, B, [0, 4, 3, 9])  # decreasing offsets
