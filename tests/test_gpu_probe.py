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


# ---- how one FP8 instruction forms its sum: the model behind the FP8 parity
# tolerance (oracle/tolerance.c).  The accumulator probe of the vidyal.ai page,
# Step 5, shows that Ada's FP8 instruction keeps about 14 bits; the tests below
# pin where gfx950's FP8 instructions drop bits: groups of 8 consecutive K
# positions, each product cut toward zero to the grid 2^(E - 13) of the
# group's largest exponent-field sum E, group sums added with FP32 rounding.

FP8_KINDS = [dmu.PROBE_FP8_16X16X128, dmu.PROBE_FP8_32X32X64]


def run_batch(kind, A, B, C, fa=0, fb=0):
    D = torch.full(C.shape, float("nan"), dtype=torch.float32, device="cuda")
    dmu.probe_mfma_batch(kind, dev(A), dev(B), dev(np.ascontiguousarray(C, np.float32)), D, fa, fb)
    torch.cuda.synchronize()
    return D.cpu().numpy().astype(np.float64)


def big_and_small(kind, n, fmt, small, seed):
    """n instructions; output (i, j) of instruction t holds exactly two
    products: 256 * 256 = 2^16 at position p[t][j] and small[i] * 1 at
    position q[t][i] (all positions distinct).  Returns A, B, p, q."""
    m, nn, k = SHAPES[kind]
    rng = np.random.default_rng(seed)
    Af = np.zeros((n, m, k), np.float32)
    Bf = np.zeros((n, nn, k), np.float32)
    P = np.zeros((n, nn), np.int64)
    Q = np.zeros((n, m), np.int64)
    for t in range(n):
        perm = rng.permutation(k)
        P[t], Q[t] = perm[:nn], perm[nn:nn + m]
        Af[t][:, P[t]] = 256.0
        Bf[t][np.arange(nn), P[t]] = 256.0
        Af[t][np.arange(m), Q[t]] = small
        Bf[t][:, Q[t]] = 1.0
    return oracle.encode_fp8(Af, fmt), oracle.encode_fp8(Bf, fmt), P, Q


@pytest.mark.parametrize("kind", FP8_KINDS)
@pytest.mark.parametrize("fmt", [0, 1])
def test_fp8_inner_sum_groups_of_eight(kind, fmt):
    # 1 next to 2^16 is 16 binades down: lost when both products fall in the
    # same aligned run of 8 K positions, kept otherwise
    m, nn, k = SHAPES[kind]
    A, B, P, Q = big_and_small(kind, 200, fmt, np.ones(m, np.float32), 81 + fmt)
    D = run_batch(kind, A, B, np.zeros((200, m, nn)), fmt, fmt)
    same = (Q[:, :, None] // 8) == (P[:, None, :] // 8)
    assert np.all(D[same] == 2.0 ** 16)
    assert np.all(D[~same] == 2.0 ** 16 + 1)
    # every group met a small product inside and outside it
    for g in range(k // 8):
        hit = (P[:, None, :] // 8 == g)
        assert (hit & same).any() and (hit & ~same).any()


@pytest.mark.parametrize("kind", FP8_KINDS)
def test_fp8_inner_sum_cuts_each_product_toward_zero(kind):
    # one group: 2^16 (grid 2^3 = 8) beside small products in E4M3.  Round to
    # nearest would give 8 for 6 (0.75 steps) and 16 for 12 (1.5 steps); a cut
    # of the exact sum toward -inf would give -8 for -6; a cut of the group's
    # exact sum (not of each product) would keep 8 of 4 + 4 and 16 of 6 + 6 + 6.
    m, nn, k = SHAPES[kind]
    cases = [([6], 0), ([-6], 0), ([12], 8), ([-12], -8), ([4, 4], 0), ([6, 6, 6], 0),
             ([40], 40), ([6, 12], 8), ([-3, -3, -3, -3], 0), ([24, 6], 24)]
    Af = np.zeros((len(cases), m, k), np.float32)
    Bf = np.zeros((len(cases), nn, k), np.float32)
    for t, (smalls, _) in enumerate(cases):
        Af[t, :, 0], Bf[t, :, 0] = 256.0, 256.0
        for s_i, v in enumerate(smalls):
            Af[t, :, 1 + s_i], Bf[t, :, 1 + s_i] = v, 1.0
    A, B = oracle.encode_fp8(Af, 0), oracle.encode_fp8(Bf, 0)
    D = run_batch(kind, A, B, np.zeros((len(cases), m, nn)))
    for t, (smalls, kept) in enumerate(cases):
        assert np.all(D[t] == 2.0 ** 16 + kept), (smalls, D[t, 0, 0] - 2.0 ** 16)


@pytest.mark.parametrize("kind", FP8_KINDS)
def test_fp8_inner_sum_grid_follows_the_exponent_fields(kind):
    # 448 * 224 = (1.75 * 2^8)(1.75 * 2^7): exponent fields sum to 15, so the
    # grid is 2^2 = 4 although the product is above 2^16.  6 keeps 4 (a grid
    # taken from the product's own binade, 8, would drop it); 2 is dropped.
    m, nn, k = SHAPES[kind]
    Af = np.zeros((2, m, k), np.float32)
    Bf = np.zeros((2, nn, k), np.float32)
    Af[:, :, 0], Bf[:, :, 0] = 448.0, 224.0
    Af[0, :, 3], Af[1, :, 5] = 6.0, 2.0
    Bf[:, :, 3], Bf[:, :, 5] = 1.0, 1.0
    D = run_batch(kind, oracle.encode_fp8(Af, 0), oracle.encode_fp8(Bf, 0), np.zeros((2, m, nn)))
    assert np.all(D[0] == 100352.0 + 4) and np.all(D[1] == 100352.0)


def instruction_model(A, B, fa, fb):
    """The pinned model of one FP8 instruction with C = 0: aligned groups of 8
    K positions, each product cut toward zero to 2^(E - 13), the exact sum of
    the groups rounded once to FP32.  A [n][m][k], B [n][nn][k] codes."""
    bias, mbits = {0: 7, 1: 15}, {0: 3, 1: 2}

    def efield(c, f):
        e = (c.astype(np.int64) >> mbits[f]) & ((1 << (7 - mbits[f])) - 1)
        return np.maximum(e, 1) - bias[f]

    va, vb = oracle.decode_fp8(A, fa), oracle.decode_fp8(B, fb)
    n, m, k = va.shape
    nn = vb.shape[1]
    P = (va[:, :, None, :] * vb[:, None, :, :]).reshape(n, m, nn, k // 8, 8)
    E = (efield(A, fa)[:, :, None, :] + efield(B, fb)[:, None, :, :]).reshape(n, m, nn, k // 8, 8)
    E = np.where(P != 0, E, -10000).max(axis=-1, keepdims=True)
    u = np.where(E > -10000, 2.0 ** (E - 13), 1.0)
    T = np.trunc(P / u) * u          # exact: FP8 products carry at most 8 bits
    return T.sum(axis=(-1, -2)).astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("kind", FP8_KINDS)
@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 1), (0, 1)])
def test_fp8_instruction_model_bit_exact_on_normal_data(kind, fa, fb):
    # N(0,1) values scaled to a quarter of each format's range, as a
    # per-tensor quantizer leaves them: the model reproduces every output bit
    m, nn, k = SHAPES[kind]
    rng = np.random.default_rng(90 + fa + 2 * fb)
    fmax = {0: 448.0, 1: 57344.0}
    A = oracle.encode_fp8((rng.standard_normal((300, m, k)) * fmax[fa] / 4).astype(np.float32), fa)
    B = oracle.encode_fp8((rng.standard_normal((300, nn, k)) * fmax[fb] / 4).astype(np.float32), fb)
    D = run_batch(kind, A, B, np.zeros((300, m, nn)), fa, fb)
    assert np.array_equal(D, instruction_model(A, B, fa, fb))


@pytest.mark.parametrize("kind", FP8_KINDS)
@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 1), (1, 0)])
def test_fp8_instruction_within_derived_bound(kind, fa, fb):
    # codes drawn over each format's whole finite range (subnormals and zeros
    # included), same-sign and mixed-sign, with and without C: every output
    # lies within the FP32 term 1e-5 (sum|ab| + |C|) plus the exact loss of
    # the per-product cuts (oracle.fp8_group_loss); half of the outputs need
    # the second term
    m, nn, k = SHAPES[kind]
    rng = np.random.default_rng(100 + fa + 2 * fb)

    def codes(shape, fmt):
        c = rng.integers(0, 256, shape).astype(np.uint8)
        return np.where(np.isfinite(oracle.decode_fp8(c, fmt)), c, 0).astype(np.uint8)

    n = 120
    A, B = codes((n, m, k), fa), codes((n, nn, k), fb)
    A[:n // 2] &= 0x7F  # the first half: every product positive
    B[:n // 2] &= 0x7F
    C = np.where(rng.random((n, 1, 1)) < 0.5, 0.0,
                 rng.standard_normal((n, m, nn)) * 2.0 ** rng.integers(-10, 20, (n, m, nn)))
    C = C.astype(np.float32)
    D = run_batch(kind, A, B, C, fa, fb)
    needs_loss = 0
    for t in range(n):
        ref, S = oracle.gemm_fp8(A[t], B[t], fa, fb, np.float32([1]), np.float32([1]),
                                 oracle.SCALE_TENSOR, C=C[t])
        fp32 = 1e-5 * (S + np.abs(C[t]))
        L = oracle.fp8_group_loss(A[t], B[t], fa, fb)
        err = np.abs(D[t] - ref)
        assert np.all(err <= fp32 + L), t
        needs_loss += int(np.sum(err > fp32))
    assert needs_loss > 0.05 * n * m * nn


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
                                        (dmu.PROBE_FP8_32X32X64, 64, 0x38),
                                        (dmu.PROBE_MXFP8_32X32X64, 64, 0x38),
                                        (dmu.PROBE_MXFP4_32X32X64, 64, 0x22)])
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


MX_SHAPES = {dmu.PROBE_MX_16X16X128: (16, 16, 128), dmu.PROBE_MX_32X32X64: (32, 32, 64)}


def run_mx(shape, A, B, SA, SB, C, fa=0, fb=0, opsel=0):
    m, n, _ = MX_SHAPES[shape]
    D = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    dmu.probe_mfma_mx(shape, dev(A), dev(B), dev(SA), dev(SB), dev(C), D, fa, fb, opsel)
    torch.cuda.synchronize()
    return D.cpu().numpy().astype(np.float64)


def cancelling_codes(m, n, groups, seed, lo=120, hi=134):
    """SA[i][g] = a_i + u_g and SB[j][g] = b_j - u_g: every product feeding
    D[i][j] carries the same power of two, so the instruction's sum of small
    integers stays exact, while a lane that took another row's scale, or a
    decoy byte, changes D.  A mix-up of K blocks shared by A and B cancels
    here; test_mfma_mx_k_positions pins those."""
    rng = np.random.default_rng(seed)
    u = rng.integers(-3, 4, size=groups)
    a = rng.integers(lo, hi, size=m)
    b = rng.integers(lo, hi, size=n)
    SA = (a[:, None] + u[None, :]).astype(np.uint8)
    SB = (b[:, None] - u[None, :]).astype(np.uint8)
    return SA, SB


@pytest.mark.parametrize("shape", [dmu.PROBE_MX_16X16X128, dmu.PROBE_MX_32X32X64])
@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("opsel", [0, 1, 2, 3])
def test_mfma_mx_layout_exact(shape, fa, fb, opsel):
    m, n, k = MX_SHAPES[shape]
    A = oracle.encode_fp8(wl.small_ints((m, k), 31) * 0.5, fa)
    B = oracle.encode_fp8(wl.small_ints((n, k), 32), fb)
    SA, SB = cancelling_codes(m, n, k // 32, 33 + opsel)
    C = wl.small_ints((m, n), 34, -50, 50)
    D = run_mx(shape, A, B, SA, SB, C, fa, fb, opsel)
    ref, _ = oracle.gemm_mx(A, B, fa, fb, SA, SB, C=C)
    assert np.array_equal(D, ref)


def mx_encode(X, fmt):
    """FP32 -> MX element array: FP8 codes, or packed E2M1 (format 4)."""
    if fmt == oracle.E2M1:
        return oracle.pack_fp4(oracle.encode_fp4(X))
    return oracle.encode_fp8(X, fmt)


@pytest.mark.parametrize("fmt", [0, 4])
@pytest.mark.parametrize("shape", [dmu.PROBE_MX_16X16X128, dmu.PROBE_MX_32X32X64])
def test_mfma_mx_k_positions(shape, fmt):
    # one product 1 x 1 at K position k, block scales 2^g on A and 2^(4g) on
    # B: D = 2^(5 * (k // 32)) exactly when the unit scales K position k with
    # the codes of its own 32-wide block, which pins where each of a lane's
    # bytes (FP8) or nibbles (FP4) sits along K (unscaled instructions cannot
    # show it)
    m, n, k = MX_SHAPES[shape]
    SA = np.tile((127 + np.arange(k // 32)).astype(np.uint8), (m, 1))
    SB = np.tile((127 + 4 * np.arange(k // 32)).astype(np.uint8), (n, 1))
    C = np.zeros((m, n), np.float32)
    for kk in range(k):
        Af = np.zeros((m, k), np.float32)
        Bf = np.zeros((n, k), np.float32)
        Af[:, kk] = 1.0
        Bf[:, kk] = 1.0
        A, B = mx_encode(Af, fmt), mx_encode(Bf, fmt)
        D = run_mx(shape, A, B, SA, SB, C, fmt, fmt)
        ref, _ = oracle.gemm_mx(A, B, fmt, fmt, SA, SB)
        assert np.all(ref == 2.0 ** (5 * (kk // 32)))
        assert np.array_equal(D, ref), "K position %d" % kk


@pytest.mark.parametrize("fa,fb", [(4, 4), (4, 0), (0, 4)])
@pytest.mark.parametrize("shape", [dmu.PROBE_MX_16X16X128, dmu.PROBE_MX_32X32X64])
def test_mfma_mx_fp4_exact(shape, fa, fb):
    # E2M1 (and E2M1 x E4M3) operands with values in {0, +-0.5, ..., +-2} and
    # cancelling block codes: every sum is exact
    m, n, k = MX_SHAPES[shape]
    A = mx_encode(wl.small_ints((m, k), 61) * 0.5, fa)
    B = mx_encode(wl.small_ints((n, k), 62) * 0.5, fb)
    SA, SB = cancelling_codes(m, n, k // 32, 63)
    C = wl.small_ints((m, n), 64, -50, 50)
    D = run_mx(shape, A, B, SA, SB, C, fa, fb, 1)
    ref, _ = oracle.gemm_mx(A, B, fa, fb, SA, SB, C=C)
    assert np.array_equal(D, ref)


@pytest.mark.parametrize("shape", [dmu.PROBE_MX_16X16X128, dmu.PROBE_MX_32X32X64])
def test_mfma_mx_fp4_random_within_instruction_precision(shape):
    m, n, k = MX_SHAPES[shape]
    rng = np.random.default_rng(71)
    A = mx_encode(wl.normal((m, k), 72) * 3, 4)
    B = mx_encode(wl.normal((n, k), 73) * 3, 4)
    SA = rng.integers(118, 137, size=(m, k // 32)).astype(np.uint8)
    SB = rng.integers(118, 137, size=(n, k // 32)).astype(np.uint8)
    C = wl.normal((m, n), 74)
    D = run_mx(shape, A, B, SA, SB, C, 4, 4)
    ref, S = oracle.gemm_mx(A, B, 4, 4, SA, SB, C=C)
    # E2M1 x E2M1 products are multiples of 2^-2 below 2^6: every one lies on
    # its group's grid, so only the FP32 term remains
    bound = 1e-5 * (S + np.abs(C))
    assert np.all(np.abs(D - ref) <= bound)


@pytest.mark.parametrize("shape", [dmu.PROBE_MX_16X16X128, dmu.PROBE_MX_32X32X64])
def test_mfma_mx_extreme_codes_cancel(shape):
    # 2^-127 on one side and 2^127 on the other (rows and columns of the same
    # parity): exact if the instruction combines the two exponents before it
    # scales the product.  Outputs whose products carry 2^-254 come out zero;
    # those carrying 2^254 overflow in each 32-wide K group on its own, so the
    # result is non-finite but its sign need not be the exact sum's.
    m, n, k = MX_SHAPES[shape]
    A = oracle.encode_fp8(wl.small_ints((m, k), 41), 0)
    B = oracle.encode_fp8(wl.small_ints((n, k), 42), 0)
    SA = np.zeros((m, k // 32), np.uint8)
    SB = np.full((n, k // 32), 254, np.uint8)
    SA[1::2] = 254
    SB[1::2] = 0
    C = np.zeros((m, n), np.float32)
    D = run_mx(shape, A, B, SA, SB, C)
    ref, _ = oracle.gemm_mx(A, B, 0, 0, SA, SB)
    ri, cj = np.arange(m)[:, None] % 2, np.arange(n)[None, :] % 2
    same = ri == cj
    assert np.array_equal(D[same], ref[same])
    assert np.all(D[(ri == 0) & (cj == 1)] == 0.0)
    huge = (ri == 1) & (cj == 0) & (ref != 0)
    assert not np.isfinite(D[huge]).any()


@pytest.mark.parametrize("shape", [dmu.PROBE_MX_16X16X128, dmu.PROBE_MX_32X32X64])
@pytest.mark.parametrize("seed", [1, 2])
def test_mfma_mx_random_within_instruction_precision(shape, seed):
    # unrelated scale codes: products of different magnitudes meet inside one
    # instruction, which cuts each product to the grid of its group of 8
    # (probes above); the bound is the FP8 GEMM bound of one instruction
    m, n, k = MX_SHAPES[shape]
    rng = np.random.default_rng(seed)
    A = oracle.encode_fp8(wl.normal((m, k), seed), 0)
    B = oracle.encode_fp8(wl.normal((n, k), seed + 5), 1)
    SA = rng.integers(118, 137, size=(m, k // 32)).astype(np.uint8)
    SB = rng.integers(118, 137, size=(n, k // 32)).astype(np.uint8)
    C = wl.normal((m, n), seed + 9)
    D = run_mx(shape, A, B, SA, SB, C, 0, 1)
    ref, S = oracle.gemm_mx(A, B, 0, 1, SA, SB, C=C)
    L = oracle.fp8_group_loss(A, B, 0, 1, oracle.decode_e8m0(SA), oracle.decode_e8m0(SB),
                              k_per_scale=32, b_rows_per_scale=1)
    bound = 1e-5 * (S + np.abs(C)) + L
    assert np.all(np.abs(D - ref) <= bound)


def test_mfma_mx_nan_scale_code():
    # E8M0 code 255 is NaN: every output that uses that scale is NaN
    m, n, k = MX_SHAPES[dmu.PROBE_MX_32X32X64]
    A = oracle.encode_fp8(wl.small_ints((m, k), 51), 0)
    B = oracle.encode_fp8(wl.small_ints((n, k), 52), 0)
    SA = np.full((m, 2), 127, np.uint8)
    SB = np.full((n, 2), 127, np.uint8)
    SA[3, 1] = 255
    C = np.zeros((m, n), np.float32)
    D = run_mx(dmu.PROBE_MX_32X32X64, A, B, SA, SB, C)
    ref, _ = oracle.gemm_mx(A, B, 0, 0, SA, SB)
    assert np.all(np.isnan(ref[3])) and np.all(np.isnan(D[3]))
    assert np.array_equal(np.delete(D, 3, axis=0), np.delete(ref, 3, axis=0))


def cvt_points(fmt):
    """FP32 values that decide an FP8 encoder: every finite code value, every
    midpoint between neighbours and one FP32 step either side of it, signed
    zeros, FP32 subnormals, values past the largest finite, infinities, NaN,
    and random values over the whole range."""
    rng = np.random.default_rng(fmt)
    vals = oracle.decode_fp8(np.arange(256, dtype=np.uint8), fmt)
    fin = np.sort(np.unique(np.abs(vals[np.isfinite(vals)])))
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    special = np.float32([0.0, -0.0, 1e-45, -1e-45, 1e-38, np.inf, -np.inf, np.nan, 1e30, -1e30,
                          fin[-1] * 1.01, -fin[-1] * 1.2, fin[-1] * 2])
    x = np.concatenate([special, fin, -fin, mids, -mids, up, -up, dn, -dn,
                        (rng.standard_normal(100000) * fin[-1] / 4),
                        np.exp(rng.uniform(-40, 12, 100000)) * rng.choice([-1, 1], 100000)])
    x = x.astype(np.float32)
    return x if x.size % 2 == 0 else np.append(x, np.float32(0))


@pytest.mark.parametrize("fmt", [0, 1])
def test_hardware_fp8_conversion(fmt):
    # gfx950's v_cvt_pk_{fp8,bf8}_f32 rounds to nearest even but does not
    # saturate: past the largest finite value E4M3 gives NaN and E5M2 gives
    # Inf.  Clamped to +-max first (NaN passed through) it is exactly the
    # saturating encoder of the oracle -- what the fused epilogue and the
    # quantizers (for blocks with finite amax and multiplier) rely on.
    x = cvt_points(fmt)
    want = oracle.encode_fp8(x, fmt)
    xt = dev(x)
    out = {}
    for clamp in (0, 1):
        q = torch.empty(x.size, dtype=torch.uint8, device="cuda")
        dmu.probe_cvt_fp8(xt, q, fmt, clamp)
        torch.cuda.synchronize()
        out[clamp] = q.cpu().numpy()
    nan = np.isnan(x)
    assert np.array_equal(out[1][~nan], want[~nan])
    assert np.all(np.isnan(oracle.decode_fp8(out[1][nan], fmt)))
    fmax = 448.0 if fmt == 0 else 57344.0
    big = np.abs(x.astype(np.float64)) > fmax * (1 + 2.0 ** -(4 if fmt == 0 else 3))
    raw = oracle.decode_fp8(out[0][big], fmt)
    assert np.all(np.isnan(raw)) if fmt == 0 else np.all(np.isinf(raw))
    inrange = ~nan & (np.abs(x) <= fmax)
    assert np.array_equal(out[0][inrange], want[inrange])


def test_hardware_fp4_conversion():
    # gfx950's v_cvt_scalef32_pk_fp4_f32 (scale 1) after a clamp to +-6 is the
    # oracle's saturating round-to-nearest-even E2M1 encoder on every finite
    # input: every code value, every midpoint and one FP32 step either side,
    # signed zeros, FP32 subnormals, values past 6 and random values.  The MX
    # quantizer relies on it for blocks with a finite amax.  The pair
    # x[2i], x[2i+1] lands in one byte, the first value in the low nibble.
    rng = np.random.default_rng(4)
    vals = oracle.decode_fp4(np.arange(16, dtype=np.uint8))
    fin = np.sort(np.unique(np.abs(vals)))
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    up, dn = np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))
    special = np.float32([0.0, -0.0, 1e-45, -1e-45, 1e-38, -1e-38, 6.5, -7.0, 7.99, 1e30, -1e30,
                          np.inf, -np.inf, 0.25, -0.25, 0.2500001, 5.0, -5.0])
    x = np.concatenate([special, fin, -fin, mids, -mids, up, -up, dn, -dn,
                        rng.uniform(-8, 8, 100000),
                        np.exp(rng.uniform(-30, 2.1, 100000)) * rng.choice([-1, 1], 100000)])
    x = x.astype(np.float32)
    if x.size % 2:
        x = np.append(x, np.float32(0))
    want = oracle.encode_fp4(x).astype(np.uint8)
    q = torch.empty(x.size // 2, dtype=torch.uint8, device="cuda")
    dmu.probe_cvt_fp8(dev(x), q, dmu.E2M1, 1)
    torch.cuda.synchronize()
    got = q.cpu().numpy()
    lo, hi = got & 0xF, got >> 4
    assert np.array_equal(lo, want[0::2]), np.flatnonzero(lo != want[0::2])[:8]
    assert np.array_equal(hi, want[1::2]), np.flatnonzero(hi != want[1::2])[:8]


def run_tr16(offsets):
    src = torch.arange(1024, dtype=torch.int16, device="cuda")
    out = torch.full((256,), -1, dtype=torch.int16, device="cuda")
    dmu.probe_lds_tr16(src, offsets, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.int64).reshape(64, 4)


@pytest.mark.parametrize("row_elems", [32, 64, 128])
def test_lds_transpose_read_layout(row_elems):
    # The use the attention kernel makes of ds_read_b64_tr_b16: within each
    # group of 16 lanes, lane i points at row i // 4, elements 4 (i % 4) ..
    # 4 (i % 4) + 3 of a row-major block; lane j of the group then receives
    # element j of rows 0 .. 3, in row order (a 4 x 16 block transposed).
    # Groups start at different rows and columns to show they are independent.
    offs, want = [], np.zeros((64, 4), np.int64)
    for l in range(64):
        g, i = l // 16, l % 16
        # (rows start inside the probe's 2 KiB of LDS)
        row0, col0 = (3 - g) * (4 if row_elems < 128 else 1), 16 * (g % 2)
        offs.append(((row0 + i // 4) * row_elems + col0 + 4 * (i % 4)) * 2)
        for e in range(4):
            want[l, e] = (row0 + e) * row_elems + col0 + i
    got = run_tr16(offs)
    assert np.array_equal(got, want), "lane -> element indices:\n%s" % got
