"""Parity of the fused epilogue (gemm_bf16_fused, gemm_fp8_fused) against the
oracle: y = act(alpha * (A B) + bias), cast to FP32, BF16 or FP8 ("How
Blackwell's Tensor Memory Actually Works", section "The cost of getting the
answer back": scale, bias, activation and cast applied to the accumulator).

Tolerance: the product's bound (1e-5 sum|ab|, plus the FP8 in-instruction
term for FP8 inputs) carried through the activation (slope at most 1.13 for
GELU and 1.1 for SiLU, so x 1.2), plus 2^-20 |y| for the FP32 activation
itself (device erf / exp), plus 2^-8 |y| for BF16 output.  FP8 output: the
code must lie between the oracle's codes of y - tol and y + tol (the encode
is monotone), i.e. within half an FP8 step of y up to the product's error."""
import numpy as np
import pytest
import torch

import oracle
import dense_matrix_unit_amd as dmu
from dense_matrix_unit_amd import workloads as wl
from gpu_helpers import bf16, dev, empty_padded, out_to_f64, padded, round_out

pytestmark = pytest.mark.gpu
ACTS = [dmu.ACT_NONE, dmu.ACT_RELU, dmu.ACT_GELU, dmu.ACT_SILU]


def tol_of(S, y, bias, extra=0.0):
    t = 1.2 * (1e-5 * (S + (0 if bias is None else np.abs(bias)[None, :])) + extra)
    return t + 2.0 ** -20 * np.abs(y) + 1e-30


def check_y(D, y, tol, bf16_out, what):
    if bf16_out:
        tol = tol + 2.0 ** -8 * np.abs(y)
    bad = ~(np.abs(D - y) <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d of %d outside; first %s got %r want %r tol %r"
                             % (what, bad.sum(), bad.size, i, D[i], y[i], tol[i]))


def check_fp8_codes(Q, y, tol, fmt, s, what):
    lo = oracle.encode_fp8(((y - tol) / s).astype(np.float32), fmt)
    hi = oracle.encode_fp8(((y + tol) / s).astype(np.float32), fmt)
    v = oracle.decode_fp8(Q, fmt)
    ok = (v >= oracle.decode_fp8(lo, fmt)) & (v <= oracle.decode_fp8(hi, fmt))
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError("%s: %d of %d codes outside; first %s got %r (%r) want %r"
                             % (what, (~ok).sum(), ok.size, i, Q[i], v[i] * s, y[i]))


def run_bf16_fused(A, B, layout, out_kind, bias, act, s=None):
    M = A.shape[0]
    N = B.shape[1] if layout == dmu.B_ROW_MAJOR else B.shape[0]
    if out_kind in ("e4m3", "e5m2"):
        out = empty_padded(M, N, torch.uint8, 16)
        fmt = dmu.E4M3 if out_kind == "e4m3" else dmu.E5M2
        dmu.gemm_bf16_fused(padded(A, 8), padded(B, 8), out, layout,
                            None if bias is None else dev(bias), act, fmt,
                            dev(np.float32([s])))
        torch.cuda.synchronize()
        return out.cpu().numpy()
    out = empty_padded(M, N, torch.float32 if out_kind == "f32" else torch.bfloat16)
    dmu.gemm_bf16_fused(padded(A, 8), padded(B, 8), out, layout,
                        None if bias is None else dev(bias), act)
    torch.cuda.synchronize()
    return out_to_f64(out)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("shape,layout", [((320, 264, 512), dmu.B_COL_MAJOR),
                                          ((1, 16, 64), dmu.B_COL_MAJOR),
                                          ((200, 262, 136), dmu.B_COL_MAJOR),
                                          ((300, 520, 264), dmu.B_ROW_MAJOR)])
def test_bf16_fused(shape, layout, out_kind, act):
    M, N, K = shape
    A = bf16(wl.normal((M, K), 1))
    B = bf16(wl.normal((K, N) if layout == dmu.B_ROW_MAJOR else (N, K), 2))
    bias = wl.normal((N,), 3) * np.float32(4.0)
    D = run_bf16_fused(A, B, layout, out_kind, bias, act)
    Dref, S = oracle.gemm_bf16(A, B, layout)
    y = oracle.epilogue(Dref, 1.0, bias, act)
    check_y(D, y, tol_of(S, y, bias), out_kind == "bf16", "%s act %d" % (shape, act))


@pytest.mark.parametrize("out_kind", ["e4m3", "e5m2"])
@pytest.mark.parametrize("act", [dmu.ACT_NONE, dmu.ACT_GELU])
def test_bf16_fused_fp8_out(out_kind, act):
    M, N, K = 384, 272, 640
    A = bf16(wl.normal((M, K), 4))
    B = bf16(wl.normal((N, K), 5))
    bias = wl.normal((N,), 6)
    Dref, S = oracle.gemm_bf16(A, B, dmu.B_COL_MAJOR)
    y = oracle.epilogue(Dref, 1.0, bias, act)
    fmt = dmu.E4M3 if out_kind == "e4m3" else dmu.E5M2
    fmax = 448.0 if fmt == dmu.E4M3 else 57344.0
    s = float(np.float32(np.abs(y).max() / fmax * 0.5))  # half the range: no saturation
    Q = run_bf16_fused(A, B, dmu.B_COL_MAJOR, out_kind, bias, act, s)
    check_fp8_codes(Q, y, tol_of(S, y, bias), fmt, s, "%s act %d" % (out_kind, act))


def test_bf16_fused_fp8_out_saturates():
    M, N, K = 256, 256, 256
    A = bf16(wl.normal((M, K), 7))
    B = bf16(wl.normal((N, K), 8))
    Dref, S = oracle.gemm_bf16(A, B, dmu.B_COL_MAJOR)
    s = float(np.float32(np.abs(Dref).max() / 448.0 / 8))  # many values beyond +-448
    Q = run_bf16_fused(A, B, dmu.B_COL_MAJOR, "e4m3", None, dmu.ACT_NONE, s)
    check_fp8_codes(Q, Dref, tol_of(S, Dref, None), dmu.E4M3, s, "saturating")
    assert np.any(Q == 0x7E) and np.any(Q == 0xFE)


@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
def test_bf16_fused_integer_exact(out_kind):
    M, N, K = 272, 288, 384
    A = bf16(wl.small_ints((M, K), 1))
    B = bf16(wl.small_ints((N, K), 2))
    bias = wl.small_ints((N,), 3, -100, 100)
    D = run_bf16_fused(A, B, dmu.B_COL_MAJOR, out_kind, bias, dmu.ACT_RELU)
    Dref, _ = oracle.gemm_bf16(A, B, dmu.B_COL_MAJOR)
    y = oracle.epilogue(Dref, 1.0, bias, dmu.ACT_RELU)
    assert np.array_equal(D, round_out(y, out_kind == "bf16"))


@pytest.mark.parametrize("act", [dmu.ACT_RELU, dmu.ACT_SILU])
def test_fp8_in_fp8_out_chain(act):
    # an FP8 linear layer: E4M3 activations and weights with per-tensor
    # scales in, act(. + bias) out as E4M3 with a static scale, ready for the
    # next gemm_fp8_scaled
    M, N, K = 512, 384, 1024
    A, sa = oracle.quantize_fp8(wl.normal((M, K), 11), dmu.E4M3)
    B, sb = oracle.quantize_fp8(wl.normal((N, K), 12), dmu.E4M3)
    bias = wl.normal((N,), 13)
    Dref, S = oracle.gemm_fp8(A, B, 0, 0, sa, sb, oracle.SCALE_TENSOR)
    y = oracle.epilogue(Dref, 1.0, bias, act)
    s = float(np.float32(np.abs(y).max() / 448.0))
    out = empty_padded(M, N, torch.uint8, 16)
    dmu.gemm_fp8_fused(padded(A, 16), padded(B, 16), dev(sa), dev(sb), out, dmu.E4M3, dmu.E4M3,
                       dev(bias), act, dmu.E4M3, dev(np.float32([s])))
    torch.cuda.synchronize()
    Q = out.cpu().numpy()
    check_fp8_codes(Q, y, tol_of(S, y, bias, fp8_in_term(A, B, sa, sb)), dmu.E4M3, s,
                    "fp8 chain")


def fp8_in_term(A, B, sa, sb, fa=0, fb=0):
    # the in-instruction term of the FP8 bound: what the FP8 instructions
    # discard (exact per-product cuts, oracle.fp8_group_loss), times sa sb
    return oracle.fp8_group_loss(A, B, fa, fb, sa, sb)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("out_kind", ["f32", "bf16", "e5m2"])
@pytest.mark.parametrize("shape", [(300, 330, 448), (64, 130, 128)])
def test_fp8_fused(shape, out_kind, act):
    # ragged M and N (N % 4 != 0 in the second shape), a K tail in the first
    M, N, K = shape
    A, sa = oracle.quantize_fp8(wl.normal((M, K), 31), dmu.E4M3)
    B, sb = oracle.quantize_fp8(wl.normal((N, K), 32), dmu.E5M2)
    bias = wl.normal((N,), 33) * np.float32(2.0)
    Dref, S = oracle.gemm_fp8(A, B, 0, 1, sa, sb, oracle.SCALE_TENSOR)
    y = oracle.epilogue(Dref, 1.0, bias, act)
    tol = tol_of(S, y, bias, fp8_in_term(A, B, sa, sb, 0, 1))
    args = (padded(A, 16), padded(B, 16), dev(sa), dev(sb))
    if out_kind == "e5m2":
        s = float(np.float32(np.abs(y).max() / 57344.0 * 4))
        out = empty_padded(M, N, torch.uint8, 16)
        dmu.gemm_fp8_fused(*args, out, dmu.E4M3, dmu.E5M2, dev(bias), act, dmu.E5M2,
                           dev(np.float32([s])))
        torch.cuda.synchronize()
        check_fp8_codes(out.cpu().numpy(), y, tol, dmu.E5M2, s, "%s act %d" % (shape, act))
        return
    out = empty_padded(M, N, torch.float32 if out_kind == "f32" else torch.bfloat16)
    dmu.gemm_fp8_fused(*args, out, dmu.E4M3, dmu.E5M2, dev(bias), act)
    torch.cuda.synchronize()
    check_y(out_to_f64(out), y, tol, out_kind == "bf16", "%s act %d" % (shape, act))


def test_plain_entry_unchanged_by_fused_build():
    # the plain BF16 entry keeps its BF16-staged epilogue and results
    A = bf16(wl.normal((256, 256), 21))
    B = bf16(wl.normal((256, 256), 22))
    out = torch.empty((256, 256), dtype=torch.bfloat16, device="cuda")
    dmu.gemm_bf16(dev(A), dev(B), out, dmu.B_COL_MAJOR)
    fused = torch.empty_like(out)
    dmu.gemm_bf16_fused(dev(A), dev(B), fused, dmu.B_COL_MAJOR)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), fused.view(torch.int16))


def test_fused_4096_bf16_gelu():
    # the bench leg bf16_4096_bias_gelu in full: N(0,1) BF16 operands (seeds
    # 1, 2), B stored N x K, N(0,1) bias (seed 3), GELU, BF16 out
    M = N = K = 4096
    A = bf16(wl.normal((M, K), wl.SEED_A))
    B = bf16(wl.normal((N, K), wl.SEED_B))
    bias = wl.normal((N,), 3)
    D = run_bf16_fused(A, B, dmu.B_COL_MAJOR, "bf16", bias, dmu.ACT_GELU)
    Dref, S = oracle.gemm_bf16(A, B, dmu.B_COL_MAJOR)
    y = oracle.epilogue(Dref, 1.0, bias, dmu.ACT_GELU)
    check_y(D, y, tol_of(S, y, bias), True, "4096^3 bias + GELU")


def test_fused_4096_fp8_relu_fp8out():
    # the bench leg fp8_e4m3_4096_bias_relu_fp8out in full: per-tensor E4M3
    # operands, N(0,1) bias, ReLU, E4M3 out with d_scale 0.25 (many saturate)
    M = N = K = 4096
    A, sa = oracle.quantize_fp8(wl.normal((M, K), wl.SEED_A), dmu.E4M3)
    B, sb = oracle.quantize_fp8(wl.normal((N, K), wl.SEED_B), dmu.E4M3)
    bias = wl.normal((N,), 3)
    out = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    dmu.gemm_fp8_fused(dev(A), dev(B), dev(sa), dev(sb), out, dmu.E4M3, dmu.E4M3, dev(bias),
                       dmu.ACT_RELU, dmu.E4M3, dev(np.float32([0.25])))
    torch.cuda.synchronize()
    Q = out.cpu().numpy()
    Dref, S = oracle.gemm_fp8(A, B, 0, 0, sa, sb, oracle.SCALE_TENSOR)
    y = oracle.epilogue(Dref, 1.0, bias, dmu.ACT_RELU)
    tol = tol_of(S, y, bias, fp8_in_term(A, B, sa, sb))
    check_fp8_codes(Q, y, tol, dmu.E4M3, 0.25, "4096^3 bias + ReLU -> E4M3")
    assert np.any(Q == 0x7E)  # saturated codes occur at this scale
