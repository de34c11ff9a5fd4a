"""Parity of gemm_grouped_bf16 (HIP) against the oracle's grouped product: one
launch over the experts of a mixture-of-experts layer, expert g multiplying
rows offsets[g] .. offsets[g+1]-1 ("How Blackwell's Tensor Memory Actually
Works", section "What this does to serving economics", third consequence).
The row offsets live on the GPU, as routing leaves them.  Tolerance: the BF16
GEMM bound (1e-5 * sum|ab|, plus 2^-8 |D| for BF16 output); integer inputs
exact."""
import numpy as np
import pytest
import torch

import oracle
import dense_matrix_unit_amd as dmu
from dense_matrix_unit_amd import workloads as wl
from gpu_helpers import assert_within_bound, bf16, dev, out_to_f64, round_out

pytestmark = pytest.mark.gpu


def offsets_of(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def run_grouped(A, B, off, out_dtype, max_m=None, sentinel=float("nan")):
    """A: [rows][K] BF16 codes (rows >= max_m), B: [G][N][K] codes."""
    max_m = A.shape[0] if max_m is None else max_m
    G, N, K = B.shape
    out = torch.full((max_m, N), sentinel, dtype=out_dtype, device="cuda")
    dmu.gemm_grouped_bf16(dev(A[:max_m]), dev(B), dev(np.asarray(off, np.int64)), out)
    torch.cuda.synchronize()
    return out_to_f64(out)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("counts,N,K", [
    ([0, 300, 1, 257, 0, 513], 264, 136),     # empty experts, ragged M, N and K
    ([1024], 256, 512),                       # one expert: the plain product
    ([7] * 40, 128, 64),                      # many tiny experts
])
def test_grouped_matches_oracle(counts, N, K, out_dtype):
    off = offsets_of(counts)
    G = len(counts)
    A = bf16(wl.normal((off[-1], K), 1))
    B = bf16(wl.normal((G, N, K), 2))
    D = run_grouped(A, B, off, out_dtype)
    Dref, S = oracle.gemm_grouped_bf16(A, B, off)
    assert_within_bound(D, Dref, S, out_dtype == torch.bfloat16, what=str(counts[:6]))


def test_grouped_integer_exact():
    counts = wl.expert_rows(9, 1500, 21, spread=1.0)
    off = offsets_of(counts)
    G, N, K = 9, 320, 384
    A = bf16(wl.small_ints((off[-1], K), 1))
    B = bf16(wl.small_ints((G, N, K), 2))
    D = run_grouped(A, B, off, torch.float32)
    Dref, _ = oracle.gemm_grouped_bf16(A, B, off)
    assert np.array_equal(D, round_out(Dref, False))


def test_grouped_leaves_unrouted_rows_alone():
    # max_m above the routed rows: rows past offsets[G] keep what they held
    off = np.array([0, 100, 100, 260], np.int64)
    G, N, K = 3, 192, 128
    A = bf16(wl.normal((600, K), 3))
    B = bf16(wl.normal((G, N, K), 4))
    D = run_grouped(A, B, off, torch.float32, sentinel=-7.0)
    Dref, S = oracle.gemm_grouped_bf16(A, B, off)
    assert_within_bound(D[:260], Dref, S, False)
    assert np.all(D[260:] == -7.0)


def test_grouped_clamps_offsets():
    # offsets that decrease or run past max_m are clamped into [0, max_m] and
    # made non-decreasing: [0, 300, 200, 500] with max_m 450 acts as
    # [0, 300, 300, 450]
    G, N, K = 3, 160, 64
    A = bf16(wl.normal((450, K), 5))
    B = bf16(wl.normal((G, N, K), 6))
    D = run_grouped(A, B, [0, 300, 200, 500], torch.float32)
    Dref, S = oracle.gemm_grouped_bf16(A, B, [0, 300, 300, 450])
    assert_within_bound(D, Dref, S, False)


def test_grouped_offsets_from_device_cumsum():
    # routing leaves counts on the GPU; offsets come from a device cumsum
    counts = wl.expert_rows(16, 3000, 31)
    G, N, K = 16, 256, 256
    A = bf16(wl.normal((3000, K), 7))
    B = bf16(wl.normal((G, N, K), 8))
    c = torch.from_numpy(counts).cuda()
    offs = torch.zeros(G + 1, dtype=torch.int64, device="cuda")
    offs[1:] = torch.cumsum(c, 0)
    out = torch.empty((3000, N), dtype=torch.bfloat16, device="cuda")
    dmu.gemm_grouped_bf16(dev(A), dev(B), offs, out)
    torch.cuda.synchronize()
    Dref, S = oracle.gemm_grouped_bf16(A, B, offsets_of(counts))
    assert_within_bound(out_to_f64(out), Dref, S, True)


def test_grouped_moe_workload():
    # the MoE workload in full: 32 experts, 16384 routed rows, N 4096, K 7168,
    # BF16 out, every routed row
    w = wl.WORKLOADS["moe_bf16_32x16384x4096x7168"]
    G, N, K = w["G"], w["N"], w["K"]
    counts = wl.expert_rows(G, w["total_rows"], wl.SEED_ROUTING)
    off = offsets_of(counts)
    A = bf16(wl.normal((off[-1], K), wl.SEED_A))
    B = bf16(wl.normal((G, N, K), wl.SEED_B))
    D = run_grouped(A, B, off, torch.bfloat16)
    Dref, S = oracle.gemm_grouped_bf16(A, B, off)
    assert_within_bound(D[:off[-1]], Dref, S, True, what="moe")
