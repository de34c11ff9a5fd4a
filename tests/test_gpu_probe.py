"""One-instruction probes of the gfx950 matrix unit and of the direct
global->LDS copy that the GEMM kernels rely on.  Inputs are small integers
(exact in BF16 and both FP8 formats), so every output must match the oracle
exactly -- the method of the page "Tensor Cores: Matrix Instructions,
Swizzling and FP8, Measured", Step 1 -- and the accumulator probe follows its
Step 5 (C = 2^e plus a product of 1)."""
import numpy as np
import pytest
import torch

import oracle
import dense_matrix_unit_amd as dmu
from dense_matrix_unit_amd import workloads as wl
from gpu_helpers import dev

pytestmark = pytest.mark.gpu

SHAPES = {  # kind: (m, n, k)
    dmu.PROBE_BF16_16X16X32: (16, 16, 32),
    dmu.PROBE_BF16_32X32X16: (32, 32, 16),
    dmu.PROBE_FP8_16X16X128: (16, 16, 128),
    dmu.PROBE_FP8_32X32X64: (32, 32, 64),
}


def run_probe(kind, A, B, C, fa=0, fb=0):
    m, n, _ = SHAPES[kind]
    D = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    dmu.probe_mfma(kind, dev(A), dev(B), dev(C), D, fa, fb)
    torch.cuda.synchronize()
    return D.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kind", [dmu.PROBE_BF16_16X16X32, dmu.PROBE_BF16_32X32X16])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_mfma_bf16_layout_exact(kind, seed):
    m, n, k = SHAPES[kind]
    A = oracle.encode_bf16(wl.small_ints((m, k), seed))
    B = oracle.encode_bf16(wl.small_ints((n, k), seed + 10))
    C = wl.small_ints((m, n), seed + 20, -50, 50)
    D = run_probe(kind, A, B, C)
    ref, _ = oracle.gemm_bf16(A, B, oracle.B_COL_MAJOR, C=C)
    assert np.array_equal(D, ref)


@pytest.mark.parametrize("kind", [dmu.PROBE_FP8_16X16X128, dmu.PROBE_FP8_32X32X64])
@pytest.mark.parametrize("fa,fb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_mfma_fp8_layout_exact(kind, fa, fb):
    m, n, k = SHAPES[kind]
    A = oracle.encode_fp8(wl.small_ints((m, k), 4) * 0.5, fa)
    B = oracle.encode_fp8(wl.small_ints((n, k), 5), fb)
    C = wl.small_ints((m, n), 6, -50, 50)
    D = run_probe(kind, A, B, C, fa, fb)
    one = np.float32([1.0])
    ref, _ = oracle.gemm_fp8(A, B, fa, fb, one, one, oracle.SCALE_TENSOR, C=C)
    assert np.array_equal(D, ref)


def accumulator_bits(kind, fmt=0):
    """Largest e such that C = 2^e plus one product 1*1 comes out exact."""
    m, n, k = SHAPES[kind]
    Af = np.zeros((m, k), np.float32)
    Bf = np.zeros((n, k), np.float32)
    Af[:, 0] = 1.0
    Bf[:, 0] = 1.0
    if kind in (dmu.PROBE_BF16_16X16X32, dmu.PROBE_BF16_32X32X16):
        A, B = oracle.encode_bf16(Af), oracle.encode_bf16(Bf)
    else:
        A, B = oracle.encode_fp8(Af, fmt), oracle.encode_fp8(Bf, fmt)
    best = -1
    for e in range(0, 31):
        C = np.full((m, n), 2.0 ** e, np.float32)
        D = run_probe(kind, A, B, C, fmt, fmt)
        if np.all(D == 2.0 ** e + 1):
            best = e
        else:
            break
    return best


@pytest.mark.parametrize("kind", list(SHAPES))
def test_accumulator_keeps_fp32_precision(kind):
    e = accumulator_bits(kind)
    print("accumulator probe kind %d: largest exact 2^e + 1 at e = %d" % (kind, e))
    # FP32 holds 24 significant bits: 2^23 + 1 is exact, 2^24 + 1 is not
    assert e == 23


def inner_sum_gap(kind, fmt=0):
    """Largest g such that two products 2^hi and 2^(hi-g) placed in ONE
    instruction (C = 0) come out exact."""
    m, n, k = SHAPES[kind]
    fp8 = kind in (dmu.PROBE_FP8_16X16X128, dmu.PROBE_FP8_32X32X64)
    best = -1
    for g in range(0, 30):
        hi = min(16, g)
        lo = g - hi
        if fp8 and lo > 9:
            break
        p = hi // 2
        Af = np.zeros((m, k), np.float32)
        Bf = np.zeros((n, k), np.float32)
        Af[:, 0], Bf[:, 0] = 2.0 ** p, 2.0 ** (hi - p)
        Af[:, 1], Bf[:, 1] = 2.0 ** -lo, 1.0
        if fp8:
            A, B = oracle.encode_fp8(Af, fmt), oracle.encode_fp8(Bf, fmt)
        else:
            A, B = oracle.encode_bf16(Af), oracle.encode_bf16(Bf)
        D = run_probe(kind, A, B, np.zeros((m, n), np.float32), fmt, fmt)
        if np.all(D == 2.0 ** hi + 2.0 ** -lo):
            best = g
        else:
            break
    return best


@pytest.mark.parametrize("kind", list(SHAPES))
def test_fp8_mfma_inner_sum_keeps_14_bits(kind):
    # The products inside one FP8 instruction are summed keeping ~14 bits
    # below the largest (the behaviour the vidyal.ai page reports for Ada's
    # FP8 instruction, Step 5); BF16 instructions keep FP32's 24 bits.  The
    # FP8 parity tolerance is derived from this.
    g = inner_sum_gap(kind)
    print("inner-sum probe kind %d: two products exact up to a gap of %d binades" % (kind, g))
    fp8 = kind in (dmu.PROBE_FP8_16X16X128, dmu.PROBE_FP8_32X32X64)
    assert g == (13 if fp8 else 23)


@pytest.mark.parametrize("mode,size", [(0, 16), (1, 4)])
@pytest.mark.parametrize("oob_from", [64, 40, 0])
def test_direct_to_lds_copy(mode, size, oob_from):
    rng = np.random.default_rng(9)
    src = rng.integers(1, 256, 64 * size, dtype=np.uint8)
    dst = torch.zeros(2048, dtype=torch.uint8, device="cuda")
    dmu.probe_lds_load(dev(src), dst, mode, oob_from)
    torch.cuda.synchronize()
    d = dst.cpu().numpy()
    v = oob_from * size
    assert np.array_equal(d[:v], src[:v])          # lane l's bytes at l*size
    assert np.all(d[v:64 * size] == 0)             # out-of-range lanes write zeros
    assert np.all(d[64 * size:] == 0xA5)           # nothing written past 64*size


@pytest.mark.parametrize("kind,k,one", [(dmu.PROBE_BF16_32X32X16, 16, 0x3F80),
                                        (dmu.PROBE_FP8_32X32X64, 64, 0x38)])
def test_mfma_rate_probe_counts_every_instruction(kind, k, one):
    # All-ones fragments: every accumulator element gains k per round, so lane
    # sums are 256 * k * iters exactly (well inside FP32's exact integers).
    iters, grid = 37, 3
    if kind == dmu.PROBE_BF16_32X32X16:
        src = torch.full((8 * 64 * 8,), one, dtype=torch.int16, device="cuda")
    else:
        src = torch.full((8 * 64 * 32,), one, dtype=torch.uint8, device="cuda")
    out = torch.full((grid * 256,), float("nan"), dtype=torch.float32, device="cuda")
    dmu.probe_mfma_rate(kind, src, iters, grid, out)
    torch.cuda.synchronize()
    assert torch.all(out == 256.0 * k * iters)
